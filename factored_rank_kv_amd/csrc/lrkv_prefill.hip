// LRKV multi-query (prefill) attention over the factored paged cache, bf16, on MFMA.
//
// Per head h and query row i at position pos_i (LRKV notes §3, eq 6-7, with the causal
// mask of §2):
//   s_ij = (q_i . S_K[j] + p_i . R_K[h, j]) / sqrt(d_h),  p_i = q_i B_K[h],  j <= pos_i
//   o_i  = (sum_j a_ij S_V[j] + (sum_j a_ij R_V[h, j]) B_V[h]^T) / sum_j a_ij
// with a_ij = exp(s_ij - m_i) and one running max m_i per row (blockwise, as in the fused
// paragraph after Algorithm 2).  Full per-head keys and values are never formed.
//
// Workgroup = (head h, tile of 128 query rows, request b); 8 wavefronts of RW blocks of 16
// rows (RW = 1; with RW > 1 the blocks of a wavefront share every operand read from LDS).
// The key loop walks tiles of 64 positions (four pages): S_K, S_V, R_K[h] and R_V[h] of
// the tile are staged in LDS (token-major rows) and shared by the wavefronts.  Every
// product is computed transposed, tokens (or features) by query rows:
//   S^T  = S_K Q^T + R_K[h] P^T          (P^T = B_K[h]^T Q^T, formed once per tile of rows)
//   O_S^T += S_V^T A^T,  O_R^T += R_V[h]^T A^T,   O^T = O_S^T + B_V[h] O_R^T at the end,
// so that the score tile's MFMA output layout (lane = query row, four consecutive tokens)
// is exactly the B-operand layout of the value products, and each lane owns one query row
// for the softmax rescale.  S_V^T and R_V^T operands come from ds_read_b64_tr_b16 on the
// token-major rows.  P, A and the final O_R are held as bf16; P and O_R as hi + lo pairs.
// Operand reads run ahead of the products in registers: two token blocks of the score
// operands, five of the value operands (the first five issued before the softmax).
//
// MFMA lane layouts used (v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16): A[i][k] at lane
// 16*(k/KL) + i, element k%KL; B[k][j] at lane 16*(k/KL) + j; D[i][j] at lane 16*(i/4) + j,
// element i%4 (KL = 8 for K = 32, 4 for K = 16).
#include "lrkv_device.h"
#include "lrkv_launch.h"

namespace lrkv {

namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef short short4_p __attribute__((ext_vector_type(4)));
typedef short short8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_p lds_s4;

__device__ __forceinline__ f32x4_p mfma32(const bf16x8_p& a, const bf16x8_p& b, f32x4_p c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_p mfma16(const short4_p& a, const short4_p& b, f32x4_p c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 16-lane transposing read: lane j of each 16-lane group reads 4 elements at its address;
// lane i receives element i%4 of lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ short4_p read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
}
// two 4-element halves as one 8-element operand (the K = 32 product pairs two K = 16 blocks:
// any order of k works as long as both operands use the same one)
__device__ __forceinline__ bf16x8_p cat8(const short4_p& lo, const short4_p& hi) {
  return __builtin_bit_cast(bf16x8_p, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ short4_p pack4(float a, float b, float c, float d) {
  return __builtin_bit_cast(short4_p, make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d)));
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi), four at a time
__device__ __forceinline__ void split4(const f32x4_p& x, short4_p& hi, short4_p& lo) {
  float h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = bf16_to_f32((uint16_t)f32_to_bf16_rne(x[e]));
    l[e] = x[e] - h[e];
  }
  hi = pack4(h[0], h[1], h[2], h[3]);
  lo = pack4(l[0], l[1], l[2], l[3]);
}

// max over the four 16-lane rows that hold one query row's tokens: v_permlane16_swap
// pairs rows 0-1 and 2-3, v_permlane32_swap the two halves (VALU, no LDS round trip)
__device__ __forceinline__ float xor_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace

template <class S>
struct PrefillCfg {
  static constexpr int NW = 8, NT = 64 * NW;
  static constexpr int RW = 1;                 // 16-row blocks per wavefront
  static constexpr int BQ = 16 * RW * NW;      // query rows per workgroup
  static constexpr int BT = 64;                // tokens per key tile (four pages)
  static constexpr int PPT = BT / S::P;        // pages per key tile
  static constexpr int RP = 64;                // private width padded to 4 blocks of 16
  // S_K and S_V token rows of 256 bytes with swizzled chunk positions (sk_slot, sv_slot)
  static constexpr int SK_STRIDE = S::DH * 2;
  static constexpr int SV_STRIDE = S::DH * 2;
  static constexpr int R_STRIDE = RP * 2 + 16;       // ... of R_K[h], R_V[h], B_K, B_V rows
  static constexpr int SK_OFF = 0;
  static constexpr int SV_OFF = SK_OFF + BT * SK_STRIDE;
  static constexpr int RK_OFF = SV_OFF + BT * SV_STRIDE;
  static constexpr int RV_OFF = RK_OFF + BT * R_STRIDE;
  static constexpr int LDS = RV_OFF + BT * R_STRIDE;
  static constexpr int IDB = 256;              // page ids held in LDS at a time
  static constexpr int TPB = IDB / PPT;        // key tiles they cover
  static constexpr int KB = S::DH / 32;        // K blocks of the shared score
  static constexpr int FB = S::DH / 16;        // feature blocks of O_S
  static constexpr int RB = RP / 16;           // blocks of the private width
  // 16-byte chunks staged per key tile, and per thread
  static constexpr int S_CH = PPT * S::DHC * S::P;   // of S_K (same for S_V)
  static constexpr int R_CH = PPT * S::RC * S::P;    // of R_K[h] (same for R_V[h])
  static constexpr int S_PT = (S_CH + NT - 1) / NT;
  static constexpr int R_PT = (R_CH + NT - 1) / NT;
  static_assert(S::BF && S::P == 16 && S::R <= RP && S::DH % 32 == 0, "prefill shape");
  static_assert(S::DHC == 16, "16 chunks per S row (the swizzle flips 4 bits)");
  static_assert(S::DH * S::R * 2 <= LDS, "B_K / B_V staging fits");
  static_assert(S::DH * R_STRIDE <= LDS, "padded B_K / B_V rows fit");
};

// Byte offsets of 16-byte chunk c of token row t in the S_K and S_V tiles (256-byte rows):
// chunk position c ^ (t & 15) for S_K and c ^ (9 t & 15) for S_V.  Measured with the LDS
// bank-conflict counter on this part, each tile's two access patterns then run without
// conflicts: for S_K the staging writes and the score reads (16 consecutive rows, one
// chunk per 16 lanes), for S_V the staging writes and the transposing value reads (4 rows
// x 2 neighbouring chunks per 16 lanes).  No one of the swizzles tried (nor padded rows)
// serves all three patterns.
__device__ __forceinline__ int sk_slot(int t, int c) { return t * 256 + 16 * (c ^ (t & 15)); }
__device__ __forceinline__ int sv_slot(int t, int c) { return t * 256 + 16 * (c ^ ((9 * t) & 15)); }

struct PrefillArgs {
  const void* q;
  const void* BK;
  const void* BV;
  const uint8_t* pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* out;
  int max_pages;
  int q_len;
  int q_tiles;
  int n_groups;       // batch * q_tiles
  float score_scale;  // log2(e) / sqrt(d_h)
};

// Stage a [rows x R] bf16 matrix (B_K[h] or B_V[h]) as rows of RP columns (zeros past R).
// Every load of the thread goes out before its first LDS write (as a plain loop, each load
// was waited for before the next went out).
template <class S>
__device__ __forceinline__ void stage_basis(uint8_t* lds, const void* src, int h, int t) {
  using C = PrefillCfg<S>;
  constexpr int N = S::DH * (C::RP / 8), K = (N + C::NT - 1) / C::NT;
  const uint4* g = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(src) +
                                                  (size_t)h * S::DH * S::R * 2);
  uint4 v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int i = min(t + k * C::NT, N - 1);
    const int row = i / (C::RP / 8), c = i % (C::RP / 8);
    const uint4 x = g[row * S::RC + min(c, S::RC - 1)];
    v[k] = c < S::RC ? x : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) asm volatile("" ::"v"(v[k].x), "v"(v[k].y), "v"(v[k].z), "v"(v[k].w));
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int i = t + k * C::NT;
    if (i < N) {
      const int row = i / (C::RP / 8), c = i % (C::RP / 8);
      *reinterpret_cast<uint4*>(lds + row * C::R_STRIDE + 16 * c) = v[k];
    }
  }
}

template <class S>
__global__ void __launch_bounds__(PrefillCfg<S>::NT, 1)
prefill_kernel(const PrefillArgs a) {
  using C = PrefillCfg<S>;
  constexpr int RW = C::RW;
  __shared__ __align__(16) uint8_t lds[C::LDS];
  __shared__ int ids_blk[C::IDB];  // page ids of key tiles [64 k, 64 k + 64)

  // heaviest query tiles (most key tiles under the causal mask) first; the 16 heads of one
  // (request, query tile) run back to back on one XCD, where they share the S tiles in L2
  const int Lb = blockIdx.x;
  const int xcd = Lb & 7, jx = Lb >> 3;
  const int h = jx % S::H;
  const int group = xcd + 8 * (jx / S::H);  // (request, query tile) index
  if (group >= a.n_groups) return;
  const int nb = a.n_groups / a.q_tiles;   // requests
  const int b = group % nb;
  const int qt = a.q_tiles - 1 - group / nb;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int T = a.seq_lens[b];
  // this lane's query rows (one per row block) and their positions (row sees 0..pos)
  int row[RW], pos[RW];
  bool row_ok[RW];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    row[w] = qt * C::BQ + 16 * (RW * wave + w) + li;
    row_ok[w] = row[w] < a.q_len;
    pos[w] = T - a.q_len + row[w];
  }
  // last position any row of the workgroup sees
  const int last_row = min(a.q_len - 1, qt * C::BQ + C::BQ - 1);
  const int pos_max = min(T - a.q_len + last_row, T - 1);
  const int n_tiles = pos_max >= 0 ? pos_max / C::BT + 1 : 0;

  // ---- q rows as MFMA operands: lane (lg, li) holds row li's features 32 kb + 8 lg .. +7
  // (A layout of Q = B layout of Q^T)
  bf16x8_p qv[RW][C::KB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        static_cast<const uint8_t*>(a.q) +
        (((size_t)b * a.q_len + (row_ok[w] ? row[w] : 0)) * S::H + h) * S::DH * 2);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      const uint4 v = row_ok[w] ? qrow[4 * kb + lg] : make_uint4(0u, 0u, 0u, 0u);
      qv[w][kb] = __builtin_bit_cast(bf16x8_p, v);
    }
  }

  // ---- P^T = B_K[h]^T Q^T (private queries of the rows), hi/lo bf16 B operands of the
  // private score: block rb holds P^T[16 rb + 4 lg + e][row li]; pairs of blocks make the
  // K = 32 operands (element e < 4: rank 32 kp + 4 lg + e, element 4 + e: rank
  // 32 kp + 16 + 4 lg + e)
  short4_p pth[RW][C::RB], ptl[RW][C::RB];
  stage_basis<S>(lds, a.BK, h, t);
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    f32x4_p acc[RW];
#pragma unroll
    for (int w = 0; w < RW; ++w) acc[w] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      // A = B_K^T: lane (lg, li) needs B_K[32 kb + 8 lg + e][16 rb + li]
      const uint8_t* base = lds + (32 * kb + 8 * lg + li / 4) * C::R_STRIDE + (16 * rb + 4 * (li & 3)) * 2;
      const bf16x8_p av = cat8(read_tr(base), read_tr(base + 4 * C::R_STRIDE));
#pragma unroll
      for (int w = 0; w < RW; ++w) acc[w] = mfma32(av, qv[w][kb], acc[w]);
    }
#pragma unroll
    for (int w = 0; w < RW; ++w) split4(acc[w], pth[w][rb], ptl[w][rb]);
  }
  __syncthreads();  // B_K staging area is reused by the key tiles
  bf16x8_p pkh[RW][C::RB / 2], pkl[RW][C::RB / 2];
#pragma unroll
  for (int w = 0; w < RW; ++w)
#pragma unroll
    for (int kp = 0; kp < C::RB / 2; ++kp) {
      pkh[w][kp] = cat8(pth[w][2 * kp], pth[w][2 * kp + 1]);
      pkl[w][kp] = cat8(ptl[w][2 * kp], ptl[w][2 * kp + 1]);
    }

  // pad columns of the R_K / R_V rows (never overwritten by staging): zeros, except that
  // R_V column r holds 1.0 for every token, so that row r of O_R^T accumulates the row's
  // exp-sum on the matrix cores, from the very bf16 weights the value products use (B_V's
  // column r is zero, so the expansion drops it)
  static_assert(S::R < C::RP && S::R % 8 == 0, "a pad column for the exp-sum");
  for (int i = t; i < 2 * C::BT * (C::RP / 8 - S::RC); i += C::NT) {
    const int which = i / (C::BT * (C::RP / 8 - S::RC));
    const int rem = i % (C::BT * (C::RP / 8 - S::RC));
    const int tok = rem / (C::RP / 8 - S::RC), c = S::RC + rem % (C::RP / 8 - S::RC);
    *reinterpret_cast<uint4*>(lds + (which ? C::RV_OFF : C::RK_OFF) + tok * C::R_STRIDE + 16 * c) =
        make_uint4(which && c == S::RC ? 0x3F80u : 0u, 0u, 0u, 0u);
  }

  f32x4_p os[RW][C::FB], orr[RW][C::RB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
#pragma unroll
    for (int i = 0; i < C::FB; ++i) os[w][i] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < C::RB; ++i) orr[w][i] = f32x4_p{0.f, 0.f, 0.f, 0.f};
  }
  // m_run: running max of the row (scaled, base-2 units; the exp-sum is row r of O_R^T).
  // The max starts at a finite floor far below any score, so exp2 of a masked score (-inf)
  // minus it is exactly 0 with no select, and the first visible score always moves it.
  float m_run[RW];
#pragma unroll
  for (int w = 0; w < RW; ++w) m_run[w] = -1e30f;

  const int32_t* tab = a.page_table + (size_t)b * a.max_pages;
  auto fill_ids = [&](int kt0) {  // page ids of key tiles kt0 .. kt0 + TPB - 1 (0 past the table)
    for (int i = t; i < C::IDB; i += C::NT) {
      const int pg = kt0 * C::PPT + i;
      ids_blk[i] = pg < a.max_pages ? tab[pg] : 0;
    }
  };
  uint4 sk_r[C::S_PT], sv_r[C::S_PT], rk_r[C::R_PT], rv_r[C::R_PT];
  auto load_tile = [&](int kt) {
    const int* tid_s = ids_blk + (kt % C::TPB) * C::PPT;
#pragma unroll
    for (int k = 0; k < C::S_PT; ++k) {
      const int i = t + k * C::NT;
      const int pg = i / (S::DHC * S::P), rem = i % (S::DHC * S::P);
      const bool live = i < C::S_CH && kt * C::BT + pg * S::P + rem % S::P < T;
      const uint8_t* page = a.pool + (size_t)tid_s[live ? pg : 0] * S::PAGE;
      sk_r[k] = live ? *reinterpret_cast<const uint4*>(page + 16 * rem) : make_uint4(0u, 0u, 0u, 0u);
      sv_r[k] = live ? *reinterpret_cast<const uint4*>(page + S::OFF_SV + 16 * rem) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < C::R_PT; ++k) {
      const int i = t + k * C::NT;
      const int pg = i / (S::RC * S::P), rem = i % (S::RC * S::P);
      const bool live = i < C::R_CH && kt * C::BT + pg * S::P + rem % S::P < T;
      const uint8_t* page = a.pool + (size_t)tid_s[live ? pg : 0] * S::PAGE + h * S::SEC_R;
      rk_r[k] = live ? *reinterpret_cast<const uint4*>(page + S::OFF_RK + 16 * rem) : make_uint4(0u, 0u, 0u, 0u);
      rv_r[k] = live ? *reinterpret_cast<const uint4*>(page + S::OFF_RV + 16 * rem) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < C::S_PT; ++k) {
      const int i = t + k * C::NT;
      if (i < C::S_CH) {
        const int pg = i / (S::DHC * S::P), rem = i % (S::DHC * S::P);
        const int tok = pg * S::P + rem % S::P, c = rem / S::P;
        *reinterpret_cast<uint4*>(lds + C::SK_OFF + sk_slot(tok, c)) = sk_r[k];
        *reinterpret_cast<uint4*>(lds + C::SV_OFF + sv_slot(tok, c)) = sv_r[k];
      }
    }
#pragma unroll
    for (int k = 0; k < C::R_PT; ++k) {
      const int i = t + k * C::NT;
      if (i < C::R_CH) {
        const int pg = i / (S::RC * S::P), rem = i % (S::RC * S::P);
        const int tok = pg * S::P + rem % S::P, c = rem / S::P;
        *reinterpret_cast<uint4*>(lds + C::RK_OFF + tok * C::R_STRIDE + 16 * c) = rk_r[k];
        *reinterpret_cast<uint4*>(lds + C::RV_OFF + tok * C::R_STRIDE + 16 * c) = rv_r[k];
      }
    }
  };
  fill_ids(0);
  __syncthreads();
  if (n_tiles > 0) load_tile(0);

  for (int kt = 0; kt < n_tiles; ++kt) {
    store_tile();
    __syncthreads();

    // ---- scores S^T for the 4 token blocks: lane (lg, li) gets tokens 16 tb + 4 lg + e of
    // row li of each row block; every operand read from LDS serves both row blocks
    f32x4_p sc[RW][4];
    // operands of one token block: its S_K rows (K = 32 blocks) and R_K[h] rows (pairs of
    // 16-rank blocks); two blocks are held ahead so the reads overlap the products
    struct ScoreFrag {
      bf16x8_p kv[C::KB];
      bf16x8_p rk[C::RB / 2];
    };
    auto load_sf = [&](int tb, ScoreFrag& f) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        f.kv[kb] = *reinterpret_cast<const bf16x8_p*>(lds + C::SK_OFF + sk_slot(16 * tb + li, 4 * kb + lg));
#pragma unroll
      for (int kp = 0; kp < C::RB / 2; ++kp) {
        const uint8_t* rkrow = lds + C::RK_OFF + (16 * tb + li) * C::R_STRIDE + 64 * kp + 8 * lg;
        f.rk[kp] = cat8(*reinterpret_cast<const short4_p*>(rkrow),
                        *reinterpret_cast<const short4_p*>(rkrow + 32));
      }
    };
    ScoreFrag sf[2];
    load_sf(0, sf[0]);
    load_sf(1, sf[1]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      __builtin_amdgcn_sched_barrier(0);
      ScoreFrag& f = sf[tb & 1];
      f32x4_p acc[RW];
#pragma unroll
      for (int w = 0; w < RW; ++w) acc[w] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int w = 0; w < RW; ++w) acc[w] = mfma32(f.kv[kb], qv[w][kb], acc[w]);
      // private part, K = 32 per product, ranks ordered as in pkh / pkl
#pragma unroll
      for (int kp = 0; kp < C::RB / 2; ++kp)
#pragma unroll
        for (int w = 0; w < RW; ++w) {
          acc[w] = mfma32(f.rk[kp], pkh[w][kp], acc[w]);
          acc[w] = mfma32(f.rk[kp], pkl[w][kp], acc[w]);
        }
#pragma unroll
      for (int w = 0; w < RW; ++w) sc[w][tb] = acc[w];
      if (tb + 2 < 4) {
        __builtin_amdgcn_sched_barrier(0);
        load_sf(tb + 2, f);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // value operands, in product order: for each pair of token blocks tp, the FB S_V^T
    // feature blocks then the RB R_V[h]^T rank blocks; VD of them are read ahead (the first
    // VD before the softmax, which they do not depend on; 5 measured best of 3 to 8)
    constexpr int VN = 2 * (C::FB + C::RB), VD = 5;
    auto vfrag = [&](int f) -> bf16x8_p {
      const int tp = f / (C::FB + C::RB), k = f % (C::FB + C::RB);
      if (k < C::FB) {
        const int svrow = 32 * tp + 4 * lg + li / 4;
        // features 16 fb + 4 (li & 3) .. +3: chunk 2 fb + (li & 3) / 2, half li & 1
        const uint8_t* v0 = lds + C::SV_OFF + sv_slot(svrow, 2 * k + ((li & 3) >> 1)) + 8 * (li & 1);
        return cat8(read_tr(v0), read_tr(v0 + 16 * C::SV_STRIDE));
      }
      const uint8_t* v0 = lds + C::RV_OFF + (32 * tp + 4 * lg + li / 4) * C::R_STRIDE +
                          (16 * (k - C::FB) + 4 * (li & 3)) * 2;
      return cat8(read_tr(v0), read_tr(v0 + 16 * C::R_STRIDE));
    };
    bf16x8_p vf[VD];
#pragma unroll
    for (int f = 0; f < VD; ++f) vf[f] = vfrag(f);
    __builtin_amdgcn_sched_barrier(0);

    // ---- online softmax per row: scores are tokens j = kt*BT + 16 tb + 4 lg + e of row li
    // probabilities as the B operands of the value products: pp[w][tp] element e < 4 is
    // token 32 tp + 4 lg + e, element 4 + e is token 32 tp + 16 + 4 lg + e
    bf16x8_p pp[RW][2];
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      float mt = -INFINITY;
      // token 16 tb + e of this lane's group is visible iff 16 tb + e <= lim (j < T follows
      // from pos < T)
      const int lim = row_ok[w] ? pos[w] - kt * C::BT - 4 * lg : -1;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = 16 * tb + e <= lim;
          const float s = ok ? sc[w][tb][e] : -INFINITY;  // unscaled
          sc[w][tb][e] = s;
          mt = __builtin_fmaxf(mt, s);
        }
      mt = xor_max(mt) * a.score_scale;
      const bool bump = mt > m_run[w] + 8.0f;
      if (__builtin_expect(__any(bump), 0)) {
        asm volatile("" ::: "memory");
        const float m_new = bump ? mt : m_run[w];
        const float alpha = exp2_fast(m_run[w] - m_new);  // 1 if not bumped, 0 on the first
#pragma unroll
        for (int i = 0; i < C::FB; ++i) os[w][i] *= alpha;
#pragma unroll
        for (int i = 0; i < C::RB; ++i) orr[w][i] *= alpha;
        m_run[w] = m_new;
      }
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sc[w][2 * tp + e / 4][e % 4];
          p[e] = exp2_fast(fmaf(s, a.score_scale, -m_run[w]));  // 0 for a masked score
        }
        const uint4 pw = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
        pp[w][tp] = __builtin_bit_cast(bf16x8_p, pw);
      }
    }

    // ---- values: O_S^T[16 fb + ..][row] += S_V^T A^T, O_R^T likewise, token blocks 2 tp
    // and 2 tp + 1 in one K = 32 product (element e < 4: token 32 tp + 4 lg + e, element
    // 4 + e: token 32 tp + 16 + 4 lg + e, in both operands); the A operand of block
    // (fb, tb) is S_V[16 tb + 4 lg' + e][16 fb + li'] by a transposing read
#pragma unroll
    for (int f = 0; f < VN; ++f) {
      __builtin_amdgcn_sched_barrier(0);
      const int tp = f / (C::FB + C::RB), k = f % (C::FB + C::RB);
#pragma unroll
      for (int w = 0; w < RW; ++w) {
        if (k < C::FB) os[w][k] = mfma32(vf[f % VD], pp[w][tp], os[w][k]);
        else orr[w][k - C::FB] = mfma32(vf[f % VD], pp[w][tp], orr[w][k - C::FB]);
      }
      if (f + VD < VN) vf[f % VD] = vfrag(f + VD);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < n_tiles) {
      if ((kt + 1) % C::TPB == 0) {  // next block of page ids (uniform over the workgroup)
        __syncthreads();
        fill_ids(kt + 1);
        __syncthreads();
      }
      load_tile(kt + 1);
    }
    __syncthreads();  // the tile is overwritten next
  }

  // ---- expansion through B_V[h] and normalisation:
  // O^T[16 fb + 4 lg + e][row li] = O_S^T + sum_rb B_V[16 fb + .][16 rb + .] O_R^T[16 rb + .][row]
  stage_basis<S>(lds, a.BV, h, t);
  __syncthreads();
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    short4_p orh[C::RB], orl[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) split4(orr[w][rb], orh[rb], orl[rb]);
    // the exp-sum of row li: O_R^T[r][li], at lane 16 ((r % 16) / 4) + li, element r % 4 of
    // block r / 16
    const float l_row = __shfl(orr[w][S::R / 16][S::R % 4], 16 * ((S::R % 16) / 4) + li, 64);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const size_t orow = (((size_t)b * a.q_len + row[w]) * S::H + h) * S::DH;
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb) {
      f32x4_p acc = os[w][fb];
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        // A = B_V[h]: lane (lg, li) holds B_V[16 fb + li][16 rb + 4 lg .. +3]
        const short4_p bv = *reinterpret_cast<const short4_p*>(
            lds + (16 * fb + li) * C::R_STRIDE + (16 * rb + 4 * lg) * 2);
        acc = mfma16(bv, orh[rb], acc);
        acc = mfma16(bv, orl[rb], acc);
      }
      if (row_ok[w]) {
        const uint32_t w0 = f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + orow + 16 * fb + 4 * lg) = make_uint2(w0, w1);
      }
    }
  }
}

template <class S>
hipError_t launch_prefill(const DecodeArgs& a) {
  using C = PrefillCfg<S>;
  PrefillArgs p{};
  p.q = a.q;
  p.BK = a.B_K;
  p.BV = a.B_V;
  p.pool = static_cast<const uint8_t*>(a.pool);
  p.page_table = a.page_table;
  p.seq_lens = a.seq_lens;
  p.out = a.out;
  p.max_pages = a.max_pages;
  p.q_len = a.q_len;
  p.q_tiles = (a.q_len + C::BQ - 1) / C::BQ;
  p.score_scale = 1.4426950408889634f / sqrtf((float)S::DH);
  p.n_groups = a.batch * p.q_tiles;
  const int blocks = ((p.n_groups + 7) / 8) * 8 * S::H;
  hipLaunchKernelGGL(prefill_kernel<S>, dim3(blocks), dim3(C::NT), 0, a.stream, p);
  return hipGetLastError();
}

template hipError_t launch_prefill<ShapeC1>(const DecodeArgs&);
template hipError_t launch_prefill<ShapeC3>(const DecodeArgs&);

}  // namespace lrkv
