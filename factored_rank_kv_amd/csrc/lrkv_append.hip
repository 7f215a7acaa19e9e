// LRKV append (Algorithm 1 of the LRKV notes, §3): project new rows into the shared and
// per-head private coordinates and scatter them into their pages.
//
// The projection is one product X [n x d] . [W_SK | W_SV | U_K | U_V] [d x N] with
// N = 2 d_h + 2 H r columns; column c of the product is written, rounded to nearest even,
// at the row's (page, slot) in the section that column belongs to.  Accumulation is
// float32 in a fixed order (no atomics), so results are deterministic.
#include "lrkv_device.h"
#include "lrkv_launch.h"

namespace lrkv {

// Element index, inside a page, of output column `col` for token slot `t`.
template <class S>
__device__ __forceinline__ int append_dest(int col, int t) {
  int base, k;
  if (col < S::DH) {
    base = 0;
    k = col;
  } else if (col < 2 * S::DH) {
    base = S::P * S::DH;
    k = col - S::DH;
  } else if (col < 2 * S::DH + S::H * S::R) {
    const int c = col - 2 * S::DH;
    const int h = c / S::R;
    base = 2 * S::P * S::DH + h * S::P * S::R;
    k = c - h * S::R;
  } else {
    const int c = col - 2 * S::DH - S::H * S::R;
    const int h = c / S::R;
    base = 2 * S::P * S::DH + S::H * S::P * S::R + h * S::P * S::R;
    k = c - h * S::R;
  }
  return base + ((k / S::CE) * S::P + t) * S::CE + (k % S::CE);
}

// Weight matrix, its row length and the column inside it for product column `col`.
template <class S>
__device__ __forceinline__ const uint8_t* weight_column(const AppendArgs& a, int col, int& ldw,
                                                        int& wc) {
  if (col < S::DH) {
    ldw = S::DH; wc = col;
    return static_cast<const uint8_t*>(a.W_SK);
  }
  if (col < 2 * S::DH) {
    ldw = S::DH; wc = col - S::DH;
    return static_cast<const uint8_t*>(a.W_SV);
  }
  if (col < 2 * S::DH + S::H * S::R) {
    ldw = S::H * S::R; wc = col - 2 * S::DH;
    return static_cast<const uint8_t*>(a.U_K);
  }
  ldw = S::H * S::R; wc = col - 2 * S::DH - S::H * S::R;
  return static_cast<const uint8_t*>(a.U_V);
}

template <class S>
__device__ __forceinline__ void store_elem(void* pool, size_t e, float v) {
  if constexpr (S::BF) static_cast<uint16_t*>(pool)[e] = (uint16_t)f32_to_bf16_rne(v);
  else static_cast<float*>(pool)[e] = v;
}

// ---------------------------------------------------------------------------------------
// Few rows (a decode step appends one row per request).  Workgroup = one 16-byte chunk of
// product columns (8 bf16 / 4 f32) x up to 8 rows, 256 threads.  Reading the weights once
// dominates and each workgroup reads only its d x 16-byte column strip, so thread t takes
// the 8 consecutive k of slice t (slices 256 apart for d > 2048) and issues all its weight
// and X loads at once: one memory round trip per pass.  Each thread then holds 8 x CE
// partial sums (row, column), which a halving exchange across the wavefront reduces
// (each round a lane keeps half of the sums and adds its partner's copy of that half), so
// lane i ends with sum i over the wavefront; four wavefronts add in a fixed order.
// Chunks that share a 128-byte line of a weight row go to blocks on the same XCD (blocks
// go to the XCDs round robin).  bf16: v_perm_b32 packs (W[k][c], W[k+1][c]) from two weight
// rows and v_dot2_f32_bf16 multiplies them with (X[n][k], X[n][k+1]) (products exact,
// float32 sums).
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(256)
append_few_rows_kernel(AppendArgs a, int n_chunks) {
  constexpr int CE = S::CE;
  constexpr int KT = 8;                 // k per thread per pass
  constexpr int NV = 8 * CE;            // sums per thread: 8 rows x CE columns
  constexpr int XW = KT * S::EB / 16;   // 16-byte X loads per row and pass
  constexpr int LOG_NV = NV == 64 ? 6 : 5;
  static_assert(NV == 64 || NV == 32, "8 rows x one 16-byte chunk of columns");
  __shared__ float red[4][NV];
  const int bx = blockIdx.x;
  const int chunk = (n_chunks % 8 == 0) ? (bx % 8) * (n_chunks / 8) + bx / 8 : bx;
  const int col0 = chunk * CE;
  int ldw, wc;
  const uint8_t* W = weight_column<S>(a, col0, ldw, wc);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int row0 = blockIdx.y * 8;
  const int nr = min(8, a.n_rows - row0);
  const size_t wrow = (size_t)ldw * S::EB;  // bytes per weight row
  const uint8_t* wcol = W + (size_t)wc * S::EB;
  const uint8_t* X = static_cast<const uint8_t*>(a.X);

  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = 0.f;
  for (int k0 = KT * t; k0 < a.d; k0 += KT * 256) {
    uint4 w[KT];
#pragma unroll
    for (int i = 0; i < KT; ++i) w[i] = *reinterpret_cast<const uint4*>(wcol + (size_t)(k0 + i) * wrow);
    uint4 x[8][XW];
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int q = 0; q < XW; ++q)
        x[n][q] = n < nr ? *reinterpret_cast<const uint4*>(
                               X + ((size_t)(row0 + n) * a.d + k0) * S::EB + 16 * q)
                         : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (S::BF) {
      // pk[kp][c] = (W[k0 + 2kp][c], W[k0 + 2kp + 1][c])
      uint32_t pk[KT / 2][CE];
#pragma unroll
      for (int kp = 0; kp < KT / 2; ++kp) {
        const uint32_t a0[4] = {w[2 * kp].x, w[2 * kp].y, w[2 * kp].z, w[2 * kp].w};
        const uint32_t a1[4] = {w[2 * kp + 1].x, w[2 * kp + 1].y, w[2 * kp + 1].z,
                                w[2 * kp + 1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[kp][2 * e] = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);
          pk[kp][2 * e + 1] = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);
        }
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint32_t xs[4] = {x[n][0].x, x[n][0].y, x[n][0].z, x[n][0].w};
#pragma unroll
        for (int kp = 0; kp < KT / 2; ++kp)
#pragma unroll
          for (int c = 0; c < CE; ++c) v[n * CE + c] = dot2_bf16(xs[kp], pk[kp][c], v[n * CE + c]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float xs[8] = {__uint_as_float(x[n][0].x), __uint_as_float(x[n][0].y),
                             __uint_as_float(x[n][0].z), __uint_as_float(x[n][0].w),
                             __uint_as_float(x[n][XW - 1].x), __uint_as_float(x[n][XW - 1].y),
                             __uint_as_float(x[n][XW - 1].z), __uint_as_float(x[n][XW - 1].w)};
#pragma unroll
        for (int i = 0; i < KT; ++i) {
          const float wk[4] = {__uint_as_float(w[i].x), __uint_as_float(w[i].y),
                               __uint_as_float(w[i].z), __uint_as_float(w[i].w)};
#pragma unroll
          for (int c = 0; c < CE; ++c) v[n * CE + c] = fmaf(xs[i], wk[c], v[n * CE + c]);
        }
      }
    }
  }
  // halving exchange: after the round with mask m the sum index's bit log2(m) equals the
  // lane's; once one sum is left, the remaining rounds add the partner's copy
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int m = 32 >> s;
    const int half = NV >> (s + 1);
    if (half >= 1) {
      const bool up = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float mine = up ? v[i + half] : v[i];
        const float give = up ? v[i] : v[i + half];
        v[i] = mine + __shfl_xor(give, m);
      }
    } else {
      v[0] += __shfl_xor(v[0], m);
    }
  }
  if ((lane & ((64 >> LOG_NV) - 1)) == 0) red[wave][lane >> (6 - LOG_NV)] = v[0];
  __syncthreads();
  if (t < NV) {
    const int n = t / CE, c = t % CE;
    if (n < nr) {
      const float sum = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
      const int r = row0 + n;
      const int req = a.row_req[r];
      const int pos = a.row_pos[r];
      const int page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      store_elem<S>(a.pool, (size_t)page * (S::PAGE / S::EB) + append_dest<S>(col0 + c, pos % S::P),
                    sum);
    }
  }
}


// ---------------------------------------------------------------------------------------
// Many rows (prefill, cache build), bf16: the product on MFMA.  Workgroup = 128 rows x 128
// product columns (one 128-column slice of one weight matrix), 256 threads = 2 x 2 waves of
// 64 x 64, K in steps of 32 through double-buffered LDS; v_mfma_f32_16x16x32_bf16 with
// float32 accumulation.  X tiles are stored as they are ([row][k], the A layout); weight
// tiles keep their natural [k][column] order and are read with ds_read_b64_tr_b16, whose
// 16-lane transpose hands each lane the 8 consecutive k of one column that the B operand
// needs.  The 128 x 128 result is rounded to bf16 into LDS, then written to the pages as
// 16-byte chunks (16 consecutive rows of one page fill 256 contiguous bytes of a section).
// Blocks are numbered so that the 128-column slices of one row block run on one XCD
// (blocks go to the 8 XCDs round robin), where they share that row block's X in L2.
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef short short4_v __attribute__((ext_vector_type(4)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_v lds_short4;

template <class S>
struct GemmCfg {
  static constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
  static constexpr int XS = BK * 2;              // bytes per X row in LDS
  static constexpr int WS = BN * 2 + 32;         // bytes per weight row in LDS (padded)
  static constexpr int X_BYTES = BM * XS;        // 8 KiB
  static constexpr int W_BYTES = BK * WS;        // 9 KiB
  static constexpr int STAGE = X_BYTES + W_BYTES;
  static constexpr int OS = BN * 2 + 16;         // bytes per output row in LDS (padded)
  static constexpr int NS_TILES = S::DH / BN;    // slices of W_SK (and of W_SV)
  static constexpr int NU_TILES = S::H * S::R / BN;  // slices of U_K (and of U_V)
  static constexpr int COL_TILES = 2 * NS_TILES + 2 * NU_TILES;
  static_assert(S::BF && S::DH % BN == 0 && (S::H * S::R) % BN == 0, "128-column slices");
  static_assert(2 * STAGE >= BM * OS, "output tile reuses the stage buffers");
};

template <class S>
__global__ void __launch_bounds__(256)
append_gemm_kernel(AppendArgs a, int row_tiles) {
  using G = GemmCfg<S>;
  __shared__ __align__(16) uint8_t smem[2 * G::STAGE];
  __shared__ int row_page[G::BM];
  __shared__ int row_slot[G::BM];

  // block -> (row tile, column tile): the j-th block on XCD x takes column tile j % CT of
  // row tile x + 8 * (j / CT)
  const int L = blockIdx.x;
  const int jx = L >> 3;
  const int ct = jx % G::COL_TILES;
  const int rt = (L & 7) + 8 * (jx / G::COL_TILES);
  if (rt >= row_tiles) return;
  const int row0 = rt * G::BM;

  // this column tile's weight matrix, its row length and first column
  const uint8_t* W;
  int ldw, wc0, col0;  // col0: first product column
  if (ct < G::NS_TILES) {
    W = static_cast<const uint8_t*>(a.W_SK); ldw = S::DH; wc0 = ct * G::BN;
  } else if (ct < 2 * G::NS_TILES) {
    W = static_cast<const uint8_t*>(a.W_SV); ldw = S::DH; wc0 = (ct - G::NS_TILES) * G::BN;
  } else if (ct < 2 * G::NS_TILES + G::NU_TILES) {
    W = static_cast<const uint8_t*>(a.U_K); ldw = S::H * S::R;
    wc0 = (ct - 2 * G::NS_TILES) * G::BN;
  } else {
    W = static_cast<const uint8_t*>(a.U_V); ldw = S::H * S::R;
    wc0 = (ct - 2 * G::NS_TILES - G::NU_TILES) * G::BN;
  }
  col0 = ct * G::BN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  if (t < G::BM) {
    const int r = row0 + t;
    int page = 0, slot = 0;
    if (r < a.n_rows) {
      const int req = a.row_req[r], pos = a.row_pos[r];
      page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      slot = pos % S::P;
    }
    row_page[t] = page;
    row_slot[t] = slot;
  }

  // global -> register staging: X: 2 chunks of 16 B per thread (row t/4 (+64), k-chunk t%4);
  // W: 2 chunks per thread (k row t/16 (+16), column chunk t%16)
  const uint8_t* X = static_cast<const uint8_t*>(a.X);
  const size_t xrow = (size_t)a.d * 2;
  const int xr0 = min(row0 + t / 4, a.n_rows - 1);  // rows past the end read a valid
  const int xr1 = min(row0 + t / 4 + 64, a.n_rows - 1);  // row whose result is dropped
  const uint8_t* xp0 = X + xr0 * xrow + 16 * (t & 3);
  const uint8_t* xp1 = X + xr1 * xrow + 16 * (t & 3);
  const size_t wrow = (size_t)ldw * 2;
  const uint8_t* wp0 = W + (size_t)(t / 16) * wrow + (size_t)(wc0 + 8 * (t & 15)) * 2;
  const uint8_t* wp1 = wp0 + 16 * wrow;
  const int xo0 = (t / 4) * G::XS + 16 * (t & 3), xo1 = xo0 + 64 * G::XS;
  const int wo0 = G::X_BYTES + (t / 16) * G::WS + 16 * (t & 15), wo1 = wo0 + 16 * G::WS;
  uint4 x0, x1, w0, w1;
#define LRKV_LOAD_STAGE(k0)                                                   \
  x0 = *reinterpret_cast<const uint4*>(xp0 + (size_t)(k0) * 2);               \
  x1 = *reinterpret_cast<const uint4*>(xp1 + (size_t)(k0) * 2);               \
  w0 = *reinterpret_cast<const uint4*>(wp0 + (size_t)(k0) * wrow);            \
  w1 = *reinterpret_cast<const uint4*>(wp1 + (size_t)(k0) * wrow);
#define LRKV_STORE_STAGE(buf)                                                 \
  *reinterpret_cast<uint4*>(smem + (buf) * G::STAGE + xo0) = x0;              \
  *reinterpret_cast<uint4*>(smem + (buf) * G::STAGE + xo1) = x1;              \
  *reinterpret_cast<uint4*>(smem + (buf) * G::STAGE + wo0) = w0;              \
  *reinterpret_cast<uint4*>(smem + (buf) * G::STAGE + wo1) = w1;

  f32x4_v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const int nk = a.d / G::BK;
  LRKV_LOAD_STAGE(0)
  LRKV_STORE_STAGE(0)
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) { LRKV_LOAD_STAGE((ks + 1) * G::BK) }
    const uint8_t* st = smem + buf * G::STAGE;
    bf16x8_v av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      av[i] = *reinterpret_cast<const bf16x8_v*>(st + (64 * wm + 16 * i + li) * G::XS + 16 * lg);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // lane (lg, li): k rows 8*lg + li/4 (+4), columns 64*wn + 16*j + 4*(li%4)
      const uint8_t* wb = st + G::X_BYTES + (8 * lg + li / 4) * G::WS +
                          (64 * wn + 16 * j + 4 * (li & 3)) * 2;
      const short4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(wb));
      const short4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(wb + 4 * G::WS));
      typedef short short8_v __attribute__((ext_vector_type(8)));
      const short8_v both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      bv[j] = __builtin_bit_cast(bf16x8_v, both);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    if (ks + 1 < nk) { LRKV_STORE_STAGE(buf ^ 1) }
    __syncthreads();
  }

#undef LRKV_LOAD_STAGE
#undef LRKV_STORE_STAGE

  // result tile -> bf16 [row][column] in LDS (D[i][j] at lane 16*(i/4) + j, element i%4)
  uint8_t* ot = smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 64 * wm + 16 * i + 4 * lg + e;
        const int c = 64 * wn + 16 * j + li;
        *reinterpret_cast<uint16_t*>(ot + r * G::OS + 2 * c) = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
      }
  __syncthreads();
  // 16-byte chunks to the pages: thread -> (row t%128 ... ), column chunks
  uint16_t* pool = static_cast<uint16_t*>(a.pool);
#pragma unroll
  for (int k = 0; k < (G::BM * G::BN / 8) / G::NT; ++k) {
    const int idx = t + k * G::NT;
    const int r = idx % G::BM;
    const int cc = idx / G::BM;  // column chunk 0..15
    if (row0 + r < a.n_rows) {
      const uint4 v = *reinterpret_cast<const uint4*>(ot + r * G::OS + 16 * cc);
      const size_t e = (size_t)row_page[r] * (S::PAGE / 2) +
                       append_dest<S>(col0 + 8 * cc, row_slot[r]);
      *reinterpret_cast<uint4*>(pool + e) = v;
    }
  }
}

// Rows at or above this count (bf16, d a multiple of 32) take the MFMA product.
constexpr int kGemmMinRows = 64;

template <class S>
hipError_t launch_append(const AppendArgs& a) {
  if constexpr (S::BF) {
    if (a.n_rows >= kGemmMinRows && a.d % GemmCfg<S>::BK == 0) {
      const int row_tiles = (a.n_rows + GemmCfg<S>::BM - 1) / GemmCfg<S>::BM;
      const int blocks = ((row_tiles + 7) / 8) * 8 * GemmCfg<S>::COL_TILES;
      hipLaunchKernelGGL(append_gemm_kernel<S>, dim3(blocks), dim3(GemmCfg<S>::NT), 0, a.stream,
                         a, row_tiles);
      return hipGetLastError();
    }
  }
  constexpr int N = 2 * S::DH + 2 * S::H * S::R;
  constexpr int n_chunks = N / S::CE;
  dim3 grid(n_chunks, (a.n_rows + 7) / 8);
  hipLaunchKernelGGL(append_few_rows_kernel<S>, grid, dim3(256), 0, a.stream, a, n_chunks);
  return hipGetLastError();
}

template hipError_t launch_append<ShapeC0>(const AppendArgs&);
template hipError_t launch_append<ShapeC1>(const AppendArgs&);
template hipError_t launch_append<ShapeC3>(const AppendArgs&);

}  // namespace lrkv
