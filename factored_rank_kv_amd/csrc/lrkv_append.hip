// LRKV append (Algorithm 1 of the LRKV notes, §3): project new rows into the shared and
// per-head private coordinates and scatter them into their pages.
//
// The projection is one product X [n x d] . [W_SK | W_SV | U_K | U_V] [d x N] with
// N = 2 d_h + 2 H r columns; column c of the product is written, rounded to nearest even,
// at the row's (page, slot) in the section that column belongs to.  The weights are held
// output-major (the weights of one product column are d contiguous values), so both
// operands of the product are read along k.  Accumulation is float32 in a fixed order (no
// atomics), so results are deterministic.
#include "lrkv_device.h"
#include "lrkv_launch.h"
#include "lrkv_private.h"

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

// The d weights of product column `col` (one row of the output-major weight matrices).
template <class S>
__device__ __forceinline__ const uint8_t* weight_row(const AppendArgs& a, int col) {
  const size_t rb = (size_t)a.d * S::EB;
  if (col < S::DH) return static_cast<const uint8_t*>(a.W_SK) + col * rb;
  if (col < 2 * S::DH) return static_cast<const uint8_t*>(a.W_SV) + (col - S::DH) * rb;
  if (col < 2 * S::DH + S::H * S::R)
    return static_cast<const uint8_t*>(a.U_K) + (col - 2 * S::DH) * rb;
  return static_cast<const uint8_t*>(a.U_V) + (col - 2 * S::DH - S::H * S::R) * rb;
}

template <class S>
__device__ __forceinline__ void store_elem(void* pool, size_t e, float v) {
  if constexpr (S::BF) static_cast<uint16_t*>(pool)[e] = (uint16_t)f32_to_bf16_rne(v);
  else static_cast<float*>(pool)[e] = v;
}

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Few rows (a decode step appends one row per request), bf16: the product on MFMA.
// Workgroup = 8 product columns x 16 rows, 256 threads = 4 wavefronts that split k into
// 32-wide blocks (wavefront w takes blocks w, w + 4, ...).  v_mfma_f32_16x16x32_bf16 with
// A = X (lane 16*(k/8) + i: 8 consecutive k of row i) and B = the weight rows (lane
// 16*(k/8) + j: 8 consecutive k of column j, j < 8; lanes j >= 8 hold zeros and their
// results are dropped): both operands are 16-byte loads straight from memory, and a
// wavefront issues all of them for 16 blocks before the first product, so a pass costs
// one memory round trip.  Rows past the last are zeros and their results dropped (an
// output row of the product depends on its own A row only).  The
// destination (request, position, then page) of each stored element is requested before
// and during the operand loads.  The four partial tiles add in a fixed order through LDS.
// Each column's weights are one contiguous run of d values, so the workgroups need no
// placement on XCDs to share cache lines.
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(256)
append_few_rows_mfma_kernel(AppendArgs a) {
  static_assert(S::BF, "bf16 cache");
  constexpr int NB = 16;  // 32-k blocks per wavefront and pass
  __shared__ float red[4][16][8];
  const int col0 = blockIdx.x * 8;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int row0 = blockIdx.y * 16;
  const int nr = min(16, a.n_rows - row0);
  const size_t rb = (size_t)a.d * 2;  // bytes per X row and per weight row

  // storing thread t < 128: row t/8, column t%8
  const bool storer = t < 128 && (t >> 3) < nr;
  const int srow = row0 + min(t >> 3, nr - 1);
  int req = 0, pos = 0, page = 0;
  if (t < 128) {
    req = a.row_req[srow];
    pos = a.row_pos[srow];
  }
  const uint8_t* wr = weight_row<S>(a, col0 + (li & 7));
  const uint8_t* xr = static_cast<const uint8_t*>(a.X) + (size_t)(row0 + min(li, nr - 1)) * rb;
  const int nkb = (a.d + 31) / 32;
  f32x4_v acc = f32x4_v{0.f, 0.f, 0.f, 0.f};
  bool have_page = false;
  for (int kb0 = wave; kb0 < nkb; kb0 += 4 * NB) {
    bf16x8_v av[NB], bv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      // k past the end: a valid address, zero weights
      // lanes j >= 8 (B) and rows past the last (A) load nothing: their products are
      // dropped, and zeros keep them finite; k past the end: zero weights
      const int k = (kb0 + 4 * u) * 32 + 8 * lg;
      const int kc = min(k, a.d - 8) * 2;
      bv[u] = (li < 8 && k < a.d) ? *reinterpret_cast<const bf16x8_v*>(wr + kc) : bf16x8_v{};
      av[u] = li < nr ? *reinterpret_cast<const bf16x8_v*>(xr + kc) : bf16x8_v{};
    }
    if (!have_page && t < 128) {
      asm volatile("" ::: "memory");  // after the operand loads, not ahead of them
      page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      have_page = true;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u], acc, 0, 0, 0);
  }
  if (!have_page && t < 128) page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
  // D[i][j] at lane 16*(i/4) + j, element i%4
  if (li < 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * lg + e][li] = acc[e];
  }
  __syncthreads();
  if (storer) {
    const int r = t >> 3, c = t & 7;
    const float sum = (red[0][r][c] + red[1][r][c]) + (red[2][r][c] + red[3][r][c]);
    store_elem<S>(a.pool, (size_t)page * a.page_elems + a.elem_off + append_dest<S>(col0 + c, pos % S::P),
                  sum);
  }
}

// ---------------------------------------------------------------------------------------
// At most 8 rows, bf16 (the usual decode step): the same product with two k-blocks per
// MFMA.  Rows 8..15 of the A operand repeat X rows 0..7 at a second k-block and columns
// 8..15 of the B operand hold the 8 weight columns at that block, so the product's two
// diagonal 8 x 8 blocks are partial sums over two different k-blocks (the off-diagonal
// blocks pair different blocks and are dropped): out[r][c] = D[r][c] + D[r+8][c+8].  Every
// lane of every 16-byte load carries product data, half the load instructions and products
// of the 16-row kernel.  Loads are unconditional (rows past the last re-read a valid row,
// whose outputs are dropped; k past d reads a valid chunk and the weights are masked to
// zero), so that the compiler waits for each operand in turn rather than for all of them.
// ---------------------------------------------------------------------------------------
template <class S>
__device__ __forceinline__ void append_eight_rows(const AppendArgs& a, int blk) {
  static_assert(S::BF, "bf16 cache");
  // every argument requested at entry, under one wait: first used inside different
  // branches, they were otherwise fetched in four dependent rounds of scalar loads
  asm volatile("" ::"s"(a.X), "s"(a.n_rows), "s"(a.d), "s"(a.W_SK), "s"(a.W_SV), "s"(a.U_K),
               "s"(a.U_V), "s"(a.row_req), "s"(a.row_pos), "s"(a.page_table), "s"(a.max_pages),
               "s"(a.pool), "s"(a.page_elems), "s"(a.elem_off));
  constexpr int NB = 8;  // products (pairs of 32-k blocks) per wavefront and pass
  __shared__ float red[4][2][8][8];
  const int col0 = blk * 8;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int half = li >> 3;                 // which k-block of the pair this lane carries
  const int nr = min(8, a.n_rows);
  const size_t rb = (size_t)a.d * 2;  // bytes per X row and per weight row

  // storing thread t < 64: row t/8, column t%8
  const bool storer = t < 64 && (t >> 3) < nr;
  const int srow = min(t >> 3, nr - 1);
  int req = 0, pos = 0, page = 0;
  if (t < 64) {
    req = a.row_req[srow];
    pos = a.row_pos[srow];
  }
  const uint8_t* wr = weight_row<S>(a, col0 + (li & 7));
  const uint8_t* xr = static_cast<const uint8_t*>(a.X) + (size_t)min(li & 7, nr - 1) * rb;
  const int nkb = (a.d + 31) / 32;
  f32x4_v acc = f32x4_v{0.f, 0.f, 0.f, 0.f};
  bool have_page = false;
  for (int kb0 = wave; kb0 < nkb; kb0 += 8 * NB) {
    bf16x8_v av[NB], bv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int k = (kb0 + 4 * (2 * u + half)) * 32 + 8 * lg;  // block kb0 + 4(2u + half)
      const int kc = min(k, a.d - 8) * 2;
      const uint4 w = *reinterpret_cast<const uint4*>(wr + kc);
      const uint32_t m = k < a.d ? ~0u : 0u;  // weights past d: zero
      bv[u] = __builtin_bit_cast(bf16x8_v, make_uint4(w.x & m, w.y & m, w.z & m, w.w & m));
      av[u] = *reinterpret_cast<const bf16x8_v*>(xr + kc);
    }
    if (!have_page && t < 64) {
      // after the operand loads: req and pos made opaque here, or the page-table address is
      // computed before the loop and the row lookups waited for before the first load
      asm volatile("" : "+v"(req), "+v"(pos)::"memory");
      page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      have_page = true;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u], acc, 0, 0, 0);
  }
  if (!have_page && t < 64) page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
  // D[i][j] at lane 16*(i/4) + j, element i%4: the diagonal blocks are lanes g < 2, j < 8
  // (D[r][c]) and g >= 2, j >= 8 (D[r+8][c+8])
  if ((lg >> 1) == half) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][half][4 * (lg & 1) + e][li & 7] = acc[e];
  }
  __syncthreads();
  if (storer) {
    const int r = t >> 3, c = t & 7;
    const float sum = ((red[0][0][r][c] + red[0][1][r][c]) + (red[1][0][r][c] + red[1][1][r][c])) +
                      ((red[2][0][r][c] + red[2][1][r][c]) + (red[3][0][r][c] + red[3][1][r][c]));
    store_elem<S>(a.pool, (size_t)page * a.page_elems + a.elem_off + append_dest<S>(col0 + c, pos % S::P),
                  sum);
  }
}

template <class S>
__global__ void __launch_bounds__(256)
append_eight_rows_mfma_kernel(AppendArgs a) {
  append_eight_rows<S>(a, (int)blockIdx.x);
}

// The decode step's two independent products in one launch: the last append_blocks
// workgroups append the new rows as above, the ones before them form the private queries
// p = q B_K of the step's query rows (a workgroup per head and block of rows,
// lrkv_private.h).  The formation goes first: dispatched after the append workgroups, its
// loads queued behind their weight stream and the launch took 5.6 us against 4.9 (B=8,
// C1 sizes, the append alone 3.6 us).
struct PrivArgs {
  const void* q;
  const void* BK;
  int rows;
  uint4* p;
};

template <class S>
__global__ void __launch_bounds__(256)
append_eight_rows_pq_kernel(AppendArgs a, PrivArgs pa, int append_blocks) {
  const int pq_blocks = (int)gridDim.x - append_blocks;
  const int blk = (int)blockIdx.x;
  if (blk >= pq_blocks) {
    append_eight_rows<S>(a, blk - pq_blocks);
    return;
  }
  private_query_block<S>(pa.q, pa.BK, pa.rows, pa.p, blk);
}

// ---------------------------------------------------------------------------------------
// Few rows, float32 cache.  Workgroup = 4 product columns x 8 rows, 256 threads = (row,
// column, k-lane) with 8 k-lanes taking 4 consecutive k at a time (float4 loads of X and of
// the weight row); the k-lanes add in a fixed order through LDS.
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(256)
append_few_rows_f32_kernel(AppendArgs a) {
  static_assert(!S::BF, "float32 cache");
  __shared__ float red[8][8][4];
  const int col0 = blockIdx.x * 4;
  const int t = threadIdx.x;
  const int n = t & 7, c = (t >> 3) & 3, kl = t >> 5;
  const int row0 = blockIdx.y * 8;
  const int nr = min(8, a.n_rows - row0);
  const int row = row0 + min(n, nr - 1);
  const float* xr = static_cast<const float*>(a.X) + (size_t)row * a.d;
  const float* wr = reinterpret_cast<const float*>(weight_row<S>(a, col0 + c));
  float acc = 0.f;
  for (int k = 4 * kl; k < a.d; k += 32) {
    const float4 x = *reinterpret_cast<const float4*>(xr + k);
    const float4 w = *reinterpret_cast<const float4*>(wr + k);
    acc = fmaf(x.x, w.x, acc);
    acc = fmaf(x.y, w.y, acc);
    acc = fmaf(x.z, w.z, acc);
    acc = fmaf(x.w, w.w, acc);
  }
  red[kl][n][c] = acc;
  __syncthreads();
  if (t < 32) {
    const int rn = t >> 2, cc = t & 3;
    if (rn < nr) {
      float sum = red[0][rn][cc];
#pragma unroll
      for (int q = 1; q < 8; ++q) sum += red[q][rn][cc];
      const int r = row0 + rn;
      const int req = a.row_req[r];
      const int pos = a.row_pos[r];
      const int page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      store_elem<S>(a.pool, (size_t)page * a.page_elems + a.elem_off +
                                append_dest<S>(col0 + cc, pos % S::P),
                    sum);
    }
  }
}


// ---------------------------------------------------------------------------------------
// Many rows (prefill, cache build), bf16: the product on MFMA.  Workgroup = 256 rows x 256
// product columns, 512 threads = 2 x 4 wavefronts of 128 x 64, K in stages of 64 through
// two LDS buffers that direct global->LDS loads fill one stage ahead of the products (no
// register staging); v_mfma_f32_16x16x32_bf16 with float32 accumulation.  A
// 256 x 256 tile reads (256 + 256) x d operands for 256^2 outputs, a third less L2 -> LDS
// traffic per product than 256 x 128.  The 256 columns may span weight matrices (W_SK and
// W_SV, U_K and U_V): each 16-column group of the staging loads is one matrix's rows, with a
// base of its own.  X tiles ([row][k]) and weight tiles ([column][k], the weights being
// output-major) are stored alike, and each lane reads the 8 consecutive k of one row (A
// operand) or of one column (B operand) as one 16-byte LDS read; a wavefront's A and B
// reads serve 8 x 4 products.  The operand reads run 32 k ahead in registers: a stage's
// second 32 k are read during its first 32 k's products, then the next stage is waited for
// (one barrier per 64 k, half as many as with stages of 32: 245.5 -> 228.7 us for 32768
// rows, the plain hipBLASLt product 228.7 us in the same process) and its first operands
// are read during the second 32 k's products.  The result is rounded to
// bf16 into LDS, 128 rows at a time, then written to the pages as 16-byte chunks (16
// consecutive rows of one page fill 256 contiguous bytes of a section).  Blocks are
// numbered so that the column tiles of one row block run on one XCD (blocks go to the 8
// XCDs round robin), where they share that row block's X in L2.
// ---------------------------------------------------------------------------------------
template <class S>
struct GemmCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
  static constexpr int NWN = 4;                  // wavefronts across the columns
  static constexpr int WM = BM / 2, WN = BN / NWN;  // rows and columns per wavefront
  static constexpr int IT = WM / 16, JT = WN / 16;  // 16 x 16 product tiles per wavefront
  // bytes per X row / weight column in LDS: the 128 bytes of a stage's k, the eight 16-byte
  // chunks of row r at positions c ^ (r & 7), so that the 16 rows an operand read touches
  // (one chunk each) spread over all chunk positions, 8 rows apart; the staging writes are
  // whole 1 KiB blocks.
  static constexpr int XS = BK * 2;
  static constexpr int X_BYTES = BM * XS;
  static constexpr int W_BYTES = BN * XS;
  static constexpr int STAGE = X_BYTES + W_BYTES;
  static constexpr int NSTAGE = 2;
  static constexpr int OUT_ROWS = 128;           // result rows staged in LDS at a time
  static constexpr int OS = BN * 2 + 16;         // bytes per output row in LDS (padded)
  static constexpr int N = 2 * S::DH + 2 * S::H * S::R;  // product columns
  static constexpr int COL_TILES = N / BN;
  static_assert(S::BF && N % BN == 0, "256-column tiles");
  static_assert(S::DH % 16 == 0 && (S::H * S::R) % 16 == 0,
                "16-column staging groups never straddle two weight matrices");
  // staging: 1 KiB (8 rows of 128 bytes) per wavefront load; 4 of X and 4 of weights
  // per wavefront and stage
  static_assert(BK == 64 && NT == 512 && X_BYTES == 4 * 8 * 1024 && W_BYTES == 4 * 8 * 1024,
                "staging geometry");
  static constexpr int SMEM = NSTAGE * STAGE;    // the output tile reuses the stage buffers
  static_assert(OUT_ROWS * OS <= SMEM && BM % OUT_ROWS == 0 && OUT_ROWS == WM, "output staging");
};

// One GEMM stage of direct global->LDS loads (global_load_lds_dwordx4, 16 bytes per lane:
// lane i of the wavefront writes LDS bytes [m0 + 16 i, m0 + 16 i + 16), M0 wave-uniform):
// four 1 KiB loads of X rows (global xb + xoff[2 m + h]) to x_lds + 16 KiB m + 1 KiB h,
// then four of weight rows (global wb0 + woff[h], wb1 + woff[h]: two 16-column groups, each
// of one weight matrix) to w_lds + 1 KiB h and w_lds + 16 KiB + 1 KiB h.  The global bases
// are wave-uniform (scalar registers), the per-lane parts 32-bit offsets; M0 is set,
// stepped, and restored at the end.  Written as inline assembly, so the compiler's wait
// counters do not see these loads (it would otherwise wait for all of them before any LDS
// read); the caller waits with s_waitcnt vmcnt and a barrier before reading the bytes.
__device__ __forceinline__ void lds_dma_stage(const void* xb, const void* wb0, const void* wb1,
                                              const uint32_t (&xoff)[4], const uint32_t (&woff)[2],
                                              uint32_t x_lds, uint32_t w_lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "global_load_lds_dwordx4 %1, %7\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "global_load_lds_dwordx4 %2, %7\n\t"
      "s_add_u32 m0, m0, 0x3c00\n\t"
      "global_load_lds_dwordx4 %3, %7\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "global_load_lds_dwordx4 %4, %7\n\t"
      "s_mov_b32 m0, %6\n\t"
      "global_load_lds_dwordx4 %8, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "global_load_lds_dwordx4 %10, %9\n\t"
      "s_add_u32 m0, m0, 0x3c00\n\t"
      "global_load_lds_dwordx4 %8, %11\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "global_load_lds_dwordx4 %10, %11\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(xoff[0]), "v"(xoff[1]), "v"(xoff[2]), "v"(xoff[3]), "s"(x_lds), "s"(w_lds), "s"(xb),
        "v"(woff[0]), "s"(wb0), "v"(woff[1]), "s"(wb1)
      : "memory", "scc");
}

template <class S>
__global__ void __launch_bounds__(512, 2)
append_gemm_kernel(AppendArgs a, int row_tiles) {
  using G = GemmCfg<S>;
  __shared__ __align__(16) uint8_t smem[G::SMEM];
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
  const int col0 = ct * G::BN;  // first product column of this column tile

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: scalar addresses
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int li = lane & 15, lg = lane >> 4;

  // global -> LDS staging by direct loads (global_load_lds_dwordx4): one wavefront
  // instruction fills 1 KiB = 8 rows x 128 bytes; lane i writes bytes [16 i, 16 i + 16) of
  // it, i.e. row i/8, chunk position i%8, so it loads k-chunk (i%8) ^ (i/8) of that row.
  // Wavefront w stages X rows and weight columns 16 (w + 8 m) + 8 h + i/8, m, h = 0, 1.
  const uint8_t* X = static_cast<const uint8_t*>(a.X);
  const size_t xrow = (size_t)a.d * 2;  // bytes per X row and per weight row
  const int r8 = lane >> 3;          // row within a 1 KiB block of 8 rows of 128 bytes
  const int kc = (lane & 7) ^ r8;     // position lane & 7 of the row holds k-chunk kc
  // per-lane 32-bit offsets from the X and weight bases (loop invariant); rows past the
  // end read row n-1
  uint32_t xoff[4], woff[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = min(row0 + 16 * (wave + 8 * m) + 8 * h + r8, a.n_rows - 1);
      xoff[2 * m + h] = (uint32_t)((size_t)r * xrow + 16 * kc);
    }
#pragma unroll
  for (int h = 0; h < 2; ++h) woff[h] = (uint32_t)((size_t)(8 * h + r8) * xrow + 16 * kc);
  const uint8_t* W0 = weight_row<S>(a, col0 + 16 * wave);
  const uint8_t* W1 = weight_row<S>(a, col0 + 16 * (wave + 8));
  const int lsw0 = 16 * (lg ^ (li & 7));  // operand reads of rows 16 x + li, k-chunks 0..3
  const int lsw1 = lsw0 ^ 64;              // k-chunks 4..7
  typedef __attribute__((address_space(3))) uint8_t* lds_p;
  const uint32_t smem_base = (uint32_t)(size_t)(lds_p)smem;
  auto issue = [&](int ks, int buf) {
    const uint32_t st = smem_base + buf * G::STAGE + 2048 * wave;
    const size_t ko = (size_t)ks * G::BK * 2;
    lds_dma_stage(X + ko, W0 + ko, W1 + ko, xoff, woff, st, st + G::X_BYTES);
  };
  f32x4_v acc[G::IT][G::JT];
#pragma unroll
  for (int i = 0; i < G::IT; ++i)
#pragma unroll
    for (int j = 0; j < G::JT; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const int nk = a.d / G::BK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  // destinations of the tile's rows, looked up while the first two stages travel
  for (int i = t; i < G::BM; i += G::NT) {
    const int r = row0 + i;
    int page = 0, slot = 0;
    if (r < a.n_rows) {
      const int req = a.row_req[r], pos = a.row_pos[r];
      page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      slot = pos % S::P;
    }
    row_page[i] = page;
    row_slot[i] = slot;
  }
  if (nk > 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // operand fragments of one stage: B (JT columns blocks) and A (IT row blocks)
  struct Frag {
    bf16x8_v b[G::JT];
    bf16x8_v a[G::IT];
  };
  auto load_frag = [&](int buf, int sub, Frag& f) {
    const uint8_t* st = smem + buf * G::STAGE;
    const int lsw = sub ? lsw1 : lsw0;
#pragma unroll
    for (int j = 0; j < G::JT; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8_v*>(st + G::X_BYTES +
                                                  (G::WN * wn + 16 * j + li) * G::XS + lsw);
#pragma unroll
    for (int i = 0; i < G::IT; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8_v*>(st + (G::WM * wm + 16 * i + li) * G::XS + lsw);
  };
  // step ks (stage ks in buffer ks & 1, its first 32 k in fc): the first 32 k's products
  // with the reads of the second 32 k (same stage, no barrier) between them; then the next
  // stage's bytes are waited for (own loads, then every wavefront's through the barrier,
  // which also orders every wavefront's reads of this stage before the refill issued right
  // after it); then the second 32 k's products with the next stage's first reads between
  // them (the last step re-reads its own stage, unused)
  // the 32 products of 32 k, with the 12 operand reads issued just before them placed one
  // between consecutive products (two at a time measured 227.9 against 224.7 us)
  auto products = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < G::IT; ++i)
#pragma unroll
      for (int j = 0; j < G::JT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int k = 0; k < G::IT + G::JT - 1; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, G::IT * G::JT - (G::IT + G::JT - 1), 0);
  };
  Frag f0, f1;
  load_frag(0, 0, f0);
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    __builtin_amdgcn_sched_barrier(0);
    load_frag(buf, 1, f1);
    products(f0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    if (ks + 1 < nk) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ks + 2 < nk) issue(ks + 2, buf);
    load_frag(ks + 1 < nk ? buf ^ 1 : buf, 0, f0);
    products(f1);
  }

  // result tile -> bf16 [row][column] in LDS, one wavefront row (128 rows) at a time
  // (D[i][j] at lane 16*(i/4) + j, element i%4), then 16-byte chunks to the pages: chunk
  // idx -> row idx % 128, column chunk idx / 128
  uint8_t* ot = smem;
  uint16_t* pool = static_cast<uint16_t*>(a.pool);
#pragma unroll
  for (int half = 0; half < G::BM / G::OUT_ROWS; ++half) {
    __syncthreads();  // the last products (or the last half's chunk reads) are done with LDS
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < G::IT; ++i)
#pragma unroll
        for (int j = 0; j < G::JT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * i + 4 * lg + e;
            const int c = G::WN * wn + 16 * j + li;
            *reinterpret_cast<uint16_t*>(ot + r * G::OS + 2 * c) = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
          }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < (G::OUT_ROWS * G::BN / 8) / G::NT; ++k) {
      const int idx = t + k * G::NT;
      const int r = idx % G::OUT_ROWS;
      const int cc = idx / G::OUT_ROWS;  // column chunk 0..BN/8-1
      const int rt_row = G::OUT_ROWS * half + r;
      if (row0 + rt_row < a.n_rows) {
        const uint4 v = *reinterpret_cast<const uint4*>(ot + r * G::OS + 16 * cc);
        const size_t e = (size_t)row_page[rt_row] * a.page_elems + a.elem_off +
                         append_dest<S>(col0 + 8 * cc, row_slot[rt_row]);
        *reinterpret_cast<uint4*>(pool + e) = v;
      }
    }
  }
}

// Rows at or above this count (bf16, d a multiple of 32) take the MFMA product.
constexpr int kGemmMinRows = 64;

template <class S>
hipError_t launch_append(const AppendArgs& a_in) {
  AppendArgs a = a_in;
  if (a.page_elems == 0) a.page_elems = S::PAGE / S::EB;  // one group: the page is the block
  if constexpr (S::BF) {
    if (a.n_rows >= kGemmMinRows && a.d % GemmCfg<S>::BK == 0) {
      // the kernel addresses X rows by 32-bit byte offsets from X: batches of rows that span
      // less than 4 GiB each
      const size_t row_bytes = (size_t)a.d * 2;
      size_t cap = (size_t)0xffffffffu / row_bytes / GemmCfg<S>::BM * GemmCfg<S>::BM;
      if (cap > (size_t)a.n_rows) cap = a.n_rows;
      for (int r0 = 0; r0 < a.n_rows; r0 += (int)cap) {
        AppendArgs b = a;
        b.X = static_cast<const uint8_t*>(a.X) + (size_t)r0 * row_bytes;
        b.row_req = a.row_req + r0;
        b.row_pos = a.row_pos + r0;
        b.n_rows = a.n_rows - r0 < (int)cap ? a.n_rows - r0 : (int)cap;
        const int row_tiles = (b.n_rows + GemmCfg<S>::BM - 1) / GemmCfg<S>::BM;
        const int blocks = ((row_tiles + 7) / 8) * 8 * GemmCfg<S>::COL_TILES;
        hipLaunchKernelGGL(append_gemm_kernel<S>, dim3(blocks), dim3(GemmCfg<S>::NT), 0,
                           a.stream, b, row_tiles);
      }
      return hipGetLastError();
    }
  }
  constexpr int N = 2 * S::DH + 2 * S::H * S::R;
  if constexpr (S::BF) {
    static_assert(N % 8 == 0, "8-column workgroups");
    if (a.n_rows <= 8)
      hipLaunchKernelGGL(append_eight_rows_mfma_kernel<S>, dim3(N / 8), dim3(256), 0, a.stream, a);
    else
      hipLaunchKernelGGL(append_few_rows_mfma_kernel<S>, dim3(N / 8, (a.n_rows + 15) / 16),
                         dim3(256), 0, a.stream, a);
  } else {
    static_assert(N % 4 == 0, "4-column workgroups");
    hipLaunchKernelGGL(append_few_rows_f32_kernel<S>, dim3(N / 4, (a.n_rows + 7) / 8), dim3(256),
                       0, a.stream, a);
  }
  return hipGetLastError();
}

template <class S>
hipError_t launch_append_pq(const AppendArgs& a_in, const void* q, const void* BK, int rows,
                            void* p) {
  static_assert(S::BF, "the 8-row append is the bf16 kernel");
  AppendArgs a = a_in;
  if (a.page_elems == 0) a.page_elems = S::PAGE / S::EB;
  constexpr int N = 2 * S::DH + 2 * S::H * S::R;
  static_assert(N % 8 == 0, "8-column workgroups");
  if (a.n_rows < 1 || a.n_rows > 8 || rows < 1) return hipErrorInvalidValue;
  static_assert(PrivBlockCfg<S>::NT == 256, "workgroup size");
  const int pq_blocks = (int)private_query_workgroups<S>(rows);
  PrivArgs pa{q, BK, rows, static_cast<uint4*>(p)};
  hipLaunchKernelGGL(append_eight_rows_pq_kernel<S>, dim3(N / 8 + pq_blocks), dim3(256), 0,
                     a.stream, a, pa, N / 8);
  return hipGetLastError();
}

template hipError_t launch_append_pq<ShapeC1>(const AppendArgs&, const void*, const void*, int, void*);
template hipError_t launch_append_pq<ShapeC3>(const AppendArgs&, const void*, const void*, int, void*);
template hipError_t launch_append_pq<ShapeC1N>(const AppendArgs&, const void*, const void*, int, void*);
template hipError_t launch_append_pq<ShapeC3N>(const AppendArgs&, const void*, const void*, int, void*);

template hipError_t launch_append<ShapeC0>(const AppendArgs&);
template hipError_t launch_append<ShapeC1>(const AppendArgs&);
template hipError_t launch_append<ShapeC3>(const AppendArgs&);
template hipError_t launch_append<ShapeC1N>(const AppendArgs&);
template hipError_t launch_append<ShapeC3N>(const AppendArgs&);
template hipError_t launch_append<ShapeC3G>(const AppendArgs&);

}  // namespace lrkv
