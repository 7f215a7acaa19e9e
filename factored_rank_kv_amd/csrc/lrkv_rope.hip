// LRKV decode with rotary position encoding for gfx950: the exact path of the LRKV notes §8
// ("can RoPE's rotation pass through the low-rank basis").  The cache holds the unrotated
// shared rows s_j and private coordinates z_j; the key of head h at position j is the
// reconstructed key turned by that position's rotation, k_j = (s_j + z_j B_K[h]^T) D_j, and
// the query q~ arrives already turned at its own position.  Since D_j depends on j, the
// private query q~ D_j^T B_K[h] cannot be formed once for the whole history (eq 6 no longer
// applies); its cost moves into the scan.  With the rotation acting on feature pairs
// (2i, 2i+1) by the angle of position j, the score is
//   q~ . k_j = sum_i cos_ji a_ji + sin_ji b_ji,
//   a_ji = k_{j,2i} q_2i + k_{j,2i+1} q_{2i+1},   b_ji = k_{j,2i} q_{2i+1} - k_{j,2i+1} q_2i,
// with k_j the unrotated key.  Per page and head everything up to (a, b) is dense and runs
// on the matrix cores: the private part of the unrotated keys, transposed, P^T = B_K[h]
// R_K[h]^T (v_mfma_f32_16x16x32_bf16), whose output layout (lane = token, four consecutive
// features) is the B operand of a K = 16 product; then per 16-feature tile (a, b) = M_q
// (S_K^T + P^T) with M_q the query's 2 x 2 pair blocks (v_mfma_f32_16x16x16: S_K^T exactly in
// bf16, P^T in f16).  Only cos a + sin b stays on the VALU, with the (cos, sin) rows of the
// caller's table.  Values carry no rotation: the same online softmax, both value
// accumulators with one weight per position, and the same partial records, merged and
// expanded once through B_V[h]^T by the split decode's merge kernel (the softmax, value and
// output steps of Algorithm 2).
//
// Workgroup = (chunk of pages, group of 8 heads, query row, request), 8 wavefronts, one head
// each for the scores and the private value; the shared value of all 8 heads is one product
// per page and wavefront (wavefront w: features 16w..16w+15), one page behind the scores.
// The chunk's S_K/S_V pages and (cos, sin) rows are staged once in LDS for the 8 heads.
// Pages k+1 and k+2 are in flight in registers while page k is used.
#include "lrkv_device.h"
#include "lrkv_launch.h"

namespace lrkv {

namespace {

typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef short short4_r __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_r __attribute__((ext_vector_type(4)));
typedef float f32x4_r __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_r lds_s4_r;

constexpr int kRopeMaxChunkPages = 256;  // page ids of one chunk held in LDS

template <class S>
struct RopeCfg {
  static constexpr int HG = kRopeHeadsPerWorkgroup;  // heads per workgroup (one per wavefront)
  static constexpr int NT = 64 * HG;
  static constexpr int MIN_BLOCKS = 8 / HG;        // two wavefronts per SIMD
  static constexpr int NG = S::H / HG;             // head groups
  static constexpr int NTILE = S::DH / 16;         // 16-feature tiles of a key row
  static constexpr int KB = (S::R + 31) / 32;      // 32-wide rank blocks (zero past r)
  static constexpr int RVL = (S::RC + 3) / 4;      // R_V chunks per lane (lane = chunk, token)
  static constexpr int S_CHUNKS = 2 * S::DHC * S::P;  // 16-byte chunks of S_K and S_V
  static constexpr int SPT = S_CHUNKS / NT;
  static constexpr int PAIRS = S::DH / 2;          // rotation pairs per row
  static constexpr int CS_CHUNKS = S::P * PAIRS * 8 / 16;  // 16-byte chunks of a page's table rows
  static constexpr int CPT = CS_CHUNKS / NT;
  // LDS strides padded by one 16-byte slot so that a wavefront's reads spread over the
  // banks: S_V chunk columns of P + 1 slots, table rows of d_h/4 + 1 slots
  static constexpr int SV_STRIDE = S::P + 1;
  static constexpr int CS_ROW = PAIRS / 2 + 1;
  static constexpr int SV_BUFS = 3;   // S_V of page k is read in step k + 1
  static constexpr int MQ_ROWS = 17;  // 16 rows of a pair-block operand and a zero row
  static constexpr int FT = S::DH / (16 * HG);  // shared-value feature tiles per wavefront
  static_assert(S::BF && S::P == 16 && S::DH % 16 == 0 && S::H % HG == 0, "bf16 pages of 16");
  static_assert(S_CHUNKS % NT == 0 && CS_CHUNKS % NT == 0, "whole chunks per thread");
  static_assert(S::DH % (16 * HG) == 0, "wavefront w takes shared-value tiles FT w .. FT w + FT - 1");
  static_assert(HG % 4 == 0 && HG <= 16, "heads fill whole 4-row groups of one MFMA tile");
};

struct RopeArgs {
  const void* q;
  const void* BK;
  const uint8_t* pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const float* rope_cs;  // [rope_rows][d_h/2][2] (cos, sin)
  float* part;
  int rope_rows;
  int max_pages;
  int q_len;
  int n_split;
  int chunk;
  int batch;
  float score_scale;
};

template <class S>
struct RopeRegs {
  uint4 st[RopeCfg<S>::SPT];  // S_K / S_V chunks, thread-strided over the two sections
  uint4 cs[RopeCfg<S>::CPT];  // (cos, sin) rows of the page's 16 positions
  uint4 rk[RopeCfg<S>::KB];   // MFMA B operand: R_K[h] chunk 4kb + lane/16, token lane%16
  uint4 rv[RopeCfg<S>::RVL];  // R_V[h] chunk lane/16 + 4j, token lane%16
  uint32_t nrm;               // key-norm layouts: the reciprocal of token lane%16
};

__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_r v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_r*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 and4(const uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Loads of one page into registers.  Every step issues the same loads, live or not, so
// that the number of loads behind each buffer's is the same on every path and the compiler
// waits for exactly the page it needs (a load skipped on some path makes it wait for all of
// them): a step past the chunk's last page (`live` false, uniform) points every lane at the
// first 16 bytes of the page and of the table (one cache line each), and private chunks past
// the rank read a valid chunk whose bytes are masked off where they are used.
template <class S>
__device__ __forceinline__ void rope_issue(const uint8_t* __restrict__ page, const float* __restrict__ cs,
                                           int rope_rows, int pos0, int h, int tid, int lane,
                                           bool live, RopeRegs<S>& r) {
  using C = RopeCfg<S>;
  const uint32_t lm = live ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < C::SPT; ++i) r.st[i] = ld_stream(page + (((uint32_t)(tid + i * C::NT) * 16u) & lm));
  constexpr int ROW_CH = C::PAIRS * 8 / 16;  // 16-byte chunks of one table row
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int c = tid + i * C::NT;
    const int row = min(pos0 + c / ROW_CH, rope_rows - 1);  // rows past the table: never used
    r.cs[i] = *reinterpret_cast<const uint4*>(cs + (((uint32_t)(row * ROW_CH + c % ROW_CH) * 4u) & lm));
  }
  const int g = lane >> 4, t = lane & 15;
  const uint8_t* rk = page + S::OFF_RK + h * S::SEC_R;
  const uint8_t* rv = page + S::OFF_RV + h * S::SEC_R;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const int c = min(4 * kb + g, S::RC - 1);
    r.rk[kb] = ld_stream(rk + (((uint32_t)(c * S::P + t) * 16u) & lm));
  }
#pragma unroll
  for (int j = 0; j < C::RVL; ++j) {
    const int c = min(g + 4 * j, S::RC - 1);
    r.rv[j] = ld_stream(rv + (((uint32_t)(c * S::P + t) * 16u) & lm));
  }
  if constexpr (S::NORM)
    r.nrm = *reinterpret_cast<const uint16_t*>(page + ((uint32_t)(S::OFF_N + (h * S::P + t) * 2) & lm));
}

// Page bytes to LDS: S_K as loaded (chunk-major; bytes of empty slots only reach their own
// token's column, whose score is removed by selection), S_V as loaded with empty slots
// zeroed (their weights are exactly 0, and 0 x NaN would not be), the table rows as loaded.
template <class S>
__device__ __forceinline__ void rope_stage(uint4* __restrict__ skc, uint4* __restrict__ sv,
                                           uint4* __restrict__ csl, int tid,
                                           const RopeRegs<S>& r, int nvalid) {
  using C = RopeCfg<S>;
#pragma unroll
  for (int i = 0; i < C::SPT; ++i) {
    const int c = tid + i * C::NT;
    if (c < S::DHC * S::P) {
      skc[c] = r.st[i];  // features 8 (c / P) .. +7 of token c % P
    } else {
      const int cc = c - S::DHC * S::P;
      sv[(cc / S::P) * C::SV_STRIDE + cc % S::P] =
          (cc % S::P) < nvalid ? r.st[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int c = tid + i * C::NT;  // chunk c % (d_h/4) of table row c / (d_h/4)
    csl[(c / (C::PAIRS / 2)) * C::CS_ROW + c % (C::PAIRS / 2)] = r.cs[i];
  }
}

template <class S>
struct RopeState {
  float m_run;   // reference max (base-2 units), the same in every lane
  float l_lane;  // exp-sum share of this lane's token (each 16-lane row holds every token)
  f32x4_r accS[RopeCfg<S>::FT];  // shared value: heads 4(lane/16) + e of the group, features
                                 // 16 (FT wave + t) + lane%16
  float accR[RopeCfg<S>::RVL][8];  // chunk lane/16 + 4j of acc_R, token lane%16
};

// Scores, softmax and private value of one page for this wavefront's head; the page's
// weights go to LDS (bf16 hi + lo, the A row of the shared-value product) with the head's
// rescale factor.
template <class S>
__device__ __forceinline__ void rope_scores(const uint4* __restrict__ skc,
                                            const uint4* __restrict__ csl,
                                            const uint2* __restrict__ mqb,
                                            const uint2* __restrict__ mqh, int mq_row,
                                            uint16_t* __restrict__ wrow, float* __restrict__ alpha_out,
                                            const uint4 (&bk)[RopeCfg<S>::KB][RopeCfg<S>::NTILE],
                                            int lane, int nvalid, float score_scale,
                                            const RopeRegs<S>& r, RopeState<S>& st) {
  using C = RopeCfg<S>;
  const int n = lane & 15, g = lane >> 4;
  bf16x8_r zb[C::KB];  // R_K[h] rows as the B operand; chunks past the rank zeroed
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
    zb[kb] = __builtin_bit_cast(
        bf16x8_r, 4 * kb + 3 < S::RC ? r.rk[kb] : and4(r.rk[kb], 4 * kb + g < S::RC ? ~0u : 0u));
  float sc = 0.f;
#pragma unroll
  for (int nt = 0; nt < C::NTILE; ++nt) {
    // P^T tile: features 16nt + 4g + e of token n (A = B_K[h] rows, B = R_K[h]^T)
    f32x4_r pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
      pt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_r, bk[kb][nt]), zb[kb],
                                                   pt, 0, 0, 0);
    // (a, b) of the tile's pairs 2(e/4)... for token n: rows 4g + e of M_q (S_K^T + P^T)
    const uint2 skv = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const uint8_t*>(skc + (2 * nt + (g >> 1)) * S::P + n) + 8 * (g & 1));
    f32x4_r ab = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(short4_r, mqb[nt * C::MQ_ROWS + mq_row]),
        __builtin_bit_cast(short4_r, skv), f32x4_r{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    ab = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_r, mqh[nt * C::MQ_ROWS + mq_row]),
                                               __builtin_convertvector(pt, f16x4_r), ab, 0, 0, 0);
    // rows 4g..4g+3 are (a, b) of pairs 8nt + 2g and 8nt + 2g + 1; their (cos, sin) for
    // token n are one 16-byte chunk of its table row
    const float4 c = *reinterpret_cast<const float4*>(csl + n * C::CS_ROW + 4 * nt + g);
    sc = fmaf(c.x, ab[0], sc);
    sc = fmaf(c.y, ab[1], sc);
    sc = fmaf(c.z, ab[2], sc);
    sc = fmaf(c.w, ab[3], sc);
  }
  float scale = score_scale;
  if constexpr (S::NORM) scale *= bf16_lo(r.nrm);  // the key's stored joint-norm reciprocal
  const float full = rows4_sum(sc);                 // over the four pair groups
  const float s = n < nvalid ? full * scale : -INFINITY;  // selection
  const float pm = r16_max(s);
  // online softmax (base 2) with a lazy reference: the reference max moves only when a
  // page's max exceeds it by more than 8, and then l and acc_R are rescaled here and acc_S by
  // every wavefront in the next step (factor in LDS); weights stay <= 2^8
  float alpha = 1.f;
  if (__builtin_expect(pm > st.m_run + 8.0f, 0)) {
    alpha = exp2_fast(st.m_run - pm);  // 0 on the first page
    st.l_lane *= alpha;
#pragma unroll
    for (int j = 0; j < C::RVL; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.accR[j][e] *= alpha;
    st.m_run = pm;
  }
  const float w = exp2_fast(s - st.m_run);
  st.l_lane += w;
  if (g == 0) {  // A row of this head: 16-byte groups of tokens 4k..4k+3, hi then lo
    const uint32_t hi = f32_to_bf16_rne(w);
    const uint32_t lo = f32_to_bf16_rne(w - __uint_as_float(hi << 16));
    wrow[(n >> 2) * 8 + (n & 3)] = (uint16_t)hi;
    wrow[(n >> 2) * 8 + 4 + (n & 3)] = (uint16_t)lo;
    if (n == 0) *alpha_out = alpha;
  }
  // private value: lane (chunk, token) adds its token's weighted R_V row chunk; empty slots
  // and chunks past the rank to zero (their weight is 0, and 0 x NaN is not)
  const uint32_t vm = n < nvalid ? ~0u : 0u;
#pragma unroll
  for (int j = 0; j < C::RVL; ++j) {
    const uint4 v = and4(r.rv[j], g + 4 * j < S::RC ? vm : 0u);
    const uint32_t v4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      st.accR[j][2 * e] = fmaf(w, bf16_lo(v4[e]), st.accR[j][2 * e]);
      st.accR[j][2 * e + 1] = fmaf(w, bf16_hi(v4[e]), st.accR[j][2 * e + 1]);
    }
  }
}

// Shared value of one page for all heads of the group, feature tiles FT wave .. +FT-1:
//   acc_S[h][f] = acc_S[h][f] * alpha[h] + sum_t (hi + lo)[h][t] S_V[t][f]
// as one v_mfma_f32_16x16x32_bf16 per tile (A rows = heads, k = 16 tokens of hi then of lo;
// B = the page's S_V^T tile twice, read by the 16-lane transposing LDS read: lane L of group
// g points at token 4g + L/4, features 16 tile + 4(L%4) .. +3, so lane i receives tokens
// 4g..4g+3 of feature 16 tile + i).
template <class S>
__device__ __forceinline__ void rope_shared_value(const uint4* __restrict__ sv,
                                                  const uint4* __restrict__ wa,
                                                  const float* __restrict__ alpha, int wave,
                                                  int lane, RopeState<S>& st) {
  using C = RopeCfg<S>;
  const int j = lane & 15, g = lane >> 4;
  const bf16x8_r av = __builtin_bit_cast(bf16x8_r, wa[j * 4 + g]);  // head j (zero past the group)
  const float4 al = *reinterpret_cast<const float4*>(alpha + 4 * (g & (C::HG / 4 - 1)));
#pragma unroll
  for (int t = 0; t < C::FT; ++t) {
    const int ft = C::FT * wave + t;
    const uint8_t* bp = reinterpret_cast<const uint8_t*>(sv + (2 * ft + ((j & 3) >> 1)) * C::SV_STRIDE +
                                                         4 * g + (j >> 2)) + 8 * (j & 1);
    const short4_r b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_r*)(bp));
    st.accS[t][0] *= al.x;
    st.accS[t][1] *= al.y;
    st.accS[t][2] *= al.z;
    st.accS[t][3] *= al.w;
    const bf16x8_r bb = __builtin_bit_cast(bf16x8_r, __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3));
    st.accS[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bb, st.accS[t], 0, 0, 0);
  }
}

template <class S>
__global__ void __launch_bounds__(RopeCfg<S>::NT, RopeCfg<S>::MIN_BLOCKS)
decode_rope_kernel(const RopeArgs a) {
  using C = RopeCfg<S>;
  // every argument requested at entry, under one wait
  asm volatile("" ::"s"(a.q), "s"(a.BK), "s"(a.pool), "s"(a.page_table), "s"(a.seq_lens),
               "s"(a.rope_cs), "s"(a.part), "s"(a.rope_rows), "s"(a.max_pages), "s"(a.q_len),
               "s"(a.n_split), "s"(a.chunk), "s"(a.batch), "s"(a.score_scale));
  __shared__ uint4 skc_lds[2][S::DHC * S::P];
  __shared__ uint4 sv_lds[C::SV_BUFS][S::DHC * C::SV_STRIDE];
  __shared__ uint4 cs_lds[2][S::P * C::CS_ROW];
  __shared__ uint4 wa_lds[2][16 * 4];          // weights as A rows: [head][4 x 16 bytes]
  __shared__ __align__(16) float al_lds[2][C::HG];
  __shared__ uint2 mq_lds[C::HG][2][C::NTILE * C::MQ_ROWS];  // pair-block A operands: bf16, f16
  __shared__ uint32_t q_lds[C::HG][S::DH / 2];  // each wavefront's query row (bf16 pairs)
  __shared__ int ids_lds[kRopeMaxChunkPages];

  // (request, row, chunk, head group) in order, each XCD a contiguous range (blocks go to
  // the 8 XCDs round robin), so the head groups of a chunk share an L2
  const int total = a.batch * a.q_len * a.n_split * C::NG;
  const int per_xcd = (total + 7) / 8;
  const int gi = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (gi >= total) return;
  const int hg = gi % C::NG;
  const int split = (gi / C::NG) % a.n_split;
  const int qi = (gi / (C::NG * a.n_split)) % a.q_len;
  const int b = gi / (C::NG * a.n_split * a.q_len);
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = hg * C::HG + wave;

  // the chunk's page ids, this wavefront's query row and its head's B_K rows are requested
  // before the length is known (each valid to read whatever it is), so that one round trip
  // serves them all; the length decides what is kept.  (As loops, each id and query load was
  // waited for before the next load went out: four round trips before the first page.)
  const int pg0 = split * (a.chunk / S::P);
  const int n_ids = min(a.chunk / S::P, a.max_pages - pg0);  // table entries of the chunk
  constexpr int IDK = (kRopeMaxChunkPages + C::NT - 1) / C::NT;
  int id_r[IDK];
  const int32_t* tab = a.page_table + (size_t)b * a.max_pages + pg0;
#pragma unroll
  for (int k = 0; k < IDK; ++k) id_r[k] = tab[min(tid + k * C::NT, n_ids - 1)];
  static_assert(S::DH / 2 == 64, "one query pair per lane");
  const size_t qrow_i = ((size_t)b * a.q_len + qi) * S::H + h;
  const uint32_t q_r =
      reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.q) + qrow_i * S::DH * 2)[lane];
  // this wavefront's head: B_K[h] as the MFMA A operand (lane: feature 16nt + lane%16,
  // rank 32kb + 8(lane/16) .. +8; zero past r)
  const int n = lane & 15, g = lane >> 4;
  uint4 bk[C::KB][C::NTILE];
  const uint8_t* bkh = static_cast<const uint8_t*>(a.BK) + (size_t)h * S::DH * S::R * 2;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt) {
      const int k0 = 32 * kb + 8 * g;
      const uint4 v = *reinterpret_cast<const uint4*>(bkh + ((size_t)(16 * nt + n) * S::R +
                                                             min(k0, S::R - 8)) * 2);
      bk[kb][nt] = k0 < S::R ? v : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
  for (int k = 0; k < IDK; ++k) asm volatile("" ::"v"(id_r[k]));
  asm volatile("" ::"v"(q_r));

  const int vis = visible_tokens(a.seq_lens[b], a.q_len, qi);
  const int tok0 = pg0 * S::P;
  const int tok1 = min(vis, min(pg0 + a.chunk / S::P, a.max_pages) * S::P);
  if (tok0 >= tok1) return;  // uniform: no record for a chunk past the visible tokens
  const int pg1 = (tok1 + S::P - 1) / S::P;
  const int n_pg = pg1 - pg0;
#pragma unroll
  for (int k = 0; k < IDK; ++k)
    if (tid + k * C::NT < n_pg) ids_lds[tid + k * C::NT] = id_r[k];
  q_lds[wave][lane] = q_r;
  // zero rows of the weights' A operand (heads past the group), both buffers
  for (int i = tid; i < 2 * (16 - C::HG) * 4; i += C::NT)
    wa_lds[i / ((16 - C::HG) * 4)][C::HG * 4 + i % ((16 - C::HG) * 4)] = make_uint4(0u, 0u, 0u, 0u);

  const int mq_row = (g == (n >> 2)) ? n : 16;
  __syncthreads();  // page ids, query rows, zero rows in LDS

  auto page_ptr = [&](int pg) { return a.pool + (size_t)ids_lds[pg - pg0] * S::PAGE; };
  auto nvalid = [&](int pg) { return min(S::P, tok1 - pg * S::P); };

  RopeState<S> st;
  st.m_run = -INFINITY;
  st.l_lane = 0.f;
#pragma unroll
  for (int t = 0; t < C::FT; ++t) st.accS[t] = f32x4_r{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C::RVL; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.accR[j][e] = 0.f;

  RopeRegs<S> r0, r1, r2;  // pages k + 1 and k + 2 in flight while page k is used
  auto issue = [&](int pg, RopeRegs<S>& r) {
    rope_issue<S>(page_ptr(min(pg, pg1 - 1)), a.rope_cs, a.rope_rows, pg * S::P, h, tid, lane,
                  pg < pg1, r);
  };
  issue(pg0, r0);
  issue(pg0 + 1, r1);
  issue(pg0 + 2, r2);
  // the query's pair blocks M_q as the A operand of the (a, b) product, per tile, built while
  // the first pages travel: row i is a (even i) or b (odd i) of pair p = i/2 (features 2p,
  // 2p+1 of the tile), stored as the four k = 4(i/4) .. +3 that lane i of group i/4 holds;
  // the other groups read the zero row 16
  {
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(q_lds[wave]);
    for (int x = lane; x < C::NTILE * C::MQ_ROWS; x += 64) {
      const int nt = x / C::MQ_ROWS, i = x % C::MQ_ROWS;
      uint16_t vb[4] = {0, 0, 0, 0}, vh[4] = {0, 0, 0, 0};
      if (i < 16) {
        const int p = i >> 1, pos = 2 * (p & 1);
        const uint16_t q0 = qh[16 * nt + 2 * p], q1 = qh[16 * nt + 2 * p + 1];
        const uint16_t e0 = (i & 1) ? q1 : q0;
        const uint16_t e1 = (i & 1) ? (uint16_t)(q0 ^ 0x8000u) : q1;  // b: -q_2p
        vb[pos] = e0;
        vb[pos + 1] = e1;
        vh[pos] = __builtin_bit_cast(uint16_t, (_Float16)bf16_to_f32(e0));
        vh[pos + 1] = __builtin_bit_cast(uint16_t, (_Float16)bf16_to_f32(e1));
      }
      mq_lds[wave][0][x] = make_uint2(vb[0] | ((uint32_t)vb[1] << 16), vb[2] | ((uint32_t)vb[3] << 16));
      mq_lds[wave][1][x] = make_uint2(vh[0] | ((uint32_t)vh[1] << 16), vh[2] | ((uint32_t)vh[3] << 16));
    }
  }
  rope_stage<S>(skc_lds[0], sv_lds[0], cs_lds[0], tid, r0, nvalid(pg0));
  __syncthreads();

  // One step per page, three per trip (the register buffers rotate); step k also adds the
  // shared value of page k - 1, whose weights every wavefront wrote before the last barrier.
  // Steps past the last page only issue their (collapsed) loads, so the loop has one exit
  // and every path through it issues the same loads.
  auto step = [&](int pg, RopeRegs<S>& cur, RopeRegs<S>& nxt) {
    const int k = pg - pg0;
    if (pg < pg1)
      rope_scores<S>(skc_lds[k & 1], cs_lds[k & 1], mq_lds[wave][0], mq_lds[wave][1], mq_row,
                     reinterpret_cast<uint16_t*>(&wa_lds[k & 1][4 * wave]), &al_lds[k & 1][wave],
                     bk, lane, nvalid(pg), a.score_scale, cur, st);
    if (k > 0 && pg <= pg1)
      rope_shared_value<S>(sv_lds[(k - 1) % C::SV_BUFS], wa_lds[(k - 1) & 1], al_lds[(k - 1) & 1],
                           wave, lane, st);
    if (pg + 1 < pg1)
      rope_stage<S>(skc_lds[(k + 1) & 1], sv_lds[(k + 1) % C::SV_BUFS], cs_lds[(k + 1) & 1], tid, nxt,
                    nvalid(pg + 1));
    issue(pg + 3, cur);
    __syncthreads();
  };
  for (int pg = pg0; pg <= pg1; pg += 3) {
    step(pg, r0, r1);
    step(pg + 1, r1, r2);
    step(pg + 2, r2, r0);
  }

  // ---- partial tuple (m, l, acc_S, acc_R) of this chunk and head, the split decode's layout
  // (the lane geometry derived anew here, so that nothing computed from it is held across
  // the page loop)
  int lane_e = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(lane_e));
  const int g_e = lane_e >> 4, n_e = lane_e & 15;
  const size_t slot = ((size_t)b * a.q_len + qi) * a.n_split + split;
  float* rec = a.part + (slot * S::H + hg * C::HG) * S::PART_PAD;
  float* dst = rec + wave * S::PART_PAD;
  const float l = r16_sum(st.l_lane);  // every 16-lane row holds all tokens
  if (lane_e == 0) {
    dst[0] = st.m_run;
    dst[1] = l;
  }
  if (g_e < C::HG / 4) {  // acc_S rows: heads 4 g_e + e, features 16 (FT wave + t) + n_e
#pragma unroll
    for (int t = 0; t < C::FT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rec[(4 * g_e + e) * S::PART_PAD + 2 + 16 * (C::FT * wave + t) + n_e] = st.accS[t][e];
  }
#pragma unroll
  for (int j = 0; j < C::RVL; ++j) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = r16_sum(st.accR[j][e]);  // over the 16 token lanes
    const int c = g_e + 4 * j;
    if (n_e == 0 && c < S::RC) {
      float4* d4 = reinterpret_cast<float4*>(dst + 2 + S::DH + 8 * c);
      d4[0] = make_float4(v[0], v[1], v[2], v[3]);
      d4[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

}  // namespace

template <class S>
int rope_groups() {
  return RopeCfg<S>::NG;
}

template <class S>
hipError_t launch_decode_rope(const DecodeArgs& a, const float* rope_cs, int rope_rows) {
  using C = RopeCfg<S>;
  RopeArgs r{};
  r.q = a.q;
  r.BK = a.B_K;
  r.pool = static_cast<const uint8_t*>(a.pool);
  r.page_table = a.page_table;
  r.seq_lens = a.seq_lens;
  r.rope_cs = rope_cs;
  r.part = a.part_ws;
  r.rope_rows = rope_rows;
  r.max_pages = a.max_pages;
  r.q_len = a.q_len;
  r.n_split = a.n_split;
  r.chunk = a.chunk;
  r.batch = a.batch;
  r.score_scale = 1.4426950408889634f / sqrtf((float)S::DH);
  const long long total = (long long)a.batch * a.q_len * a.n_split * C::NG;
  hipLaunchKernelGGL((decode_rope_kernel<S>), dim3((unsigned)((total + 7) / 8 * 8)), dim3(C::NT), 0,
                     a.stream, r);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge<S>(a);
}

template int rope_groups<ShapeC1>();
template int rope_groups<ShapeC3>();
template hipError_t launch_decode_rope<ShapeC1>(const DecodeArgs&, const float*, int);
template hipError_t launch_decode_rope<ShapeC3>(const DecodeArgs&, const float*, int);
template hipError_t launch_decode_rope<ShapeC1N>(const DecodeArgs&, const float*, int);
template hipError_t launch_decode_rope<ShapeC3N>(const DecodeArgs&, const float*, int);

}  // namespace lrkv
