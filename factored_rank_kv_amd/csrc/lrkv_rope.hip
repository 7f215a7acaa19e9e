// LRKV decode with rotary position encoding for gfx950: the exact path of the LRKV notes §8
// ("can RoPE's rotation pass through the low-rank basis").  The cache holds the unrotated
// shared rows s_j and private coordinates z_j; the key of head h at position j is the
// reconstructed key turned by that position's rotation, k_j = (s_j + z_j B_K[h]^T) D_j, and
// the query q~ arrives already turned at its own position.  Since D_j depends on j, the
// private query q~ D_j^T B_K[h] cannot be formed once for the whole history (eq 6 no longer
// applies); its cost moves into the scan.  Here it is spent where it is cheapest on CDNA4:
// per page and head, the 16 x d_h block of unrotated keys S_K + R_K[h] B_K[h]^T is formed on
// MFMA (v_mfma_f32_16x16x32_bf16: A = the page's R_K[h] rows, B = B_K[h]^T held in
// registers, the accumulator starting from S_K), and each key row is dotted with the query
// counter-turned by its position, q~ D_j^T, from a caller-supplied (cos, sin) table:
//   score_j = (q~ D_j^T) . (s_j + z_j B_K[h]^T) = (q~ D_j^T) . s_j + ((q~ D_j^T) B_K[h]) . z_j.
// Values carry no rotation: the same online softmax, both value accumulators with one
// weight per position, and the same partial records, merged and expanded once through
// B_V[h]^T by the split decode's merge kernel (the softmax, value and output steps of Algorithm 2).
//
// Workgroup = (chunk of pages, group of 4 heads, query row, request), 4 wavefronts, one head
// each; the chunk's S_K/S_V pages and (cos, sin) rows are staged once in LDS for the 4 heads
// (the other head groups of the chunk run next to it on the same XCD and find the shared
// rows in its L2).  Page k+1 is in flight in registers while page k is used.
#include "lrkv_device.h"
#include "lrkv_launch.h"

namespace lrkv {

namespace {

typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef float f32x4_r __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));
// The B operand of a 16 x 16 x 32 product whose first 16 rows are the identity and the
// rest zero: lane 16 (k/8) + j holds B[k][j] for k = 8 (lane/16) .. +7, j = lane % 16
// (bf16 1.0 = 0x3f80 where k == j).
__device__ __forceinline__ uint4 make_ident8(int lane) {
  const int j = lane & 15, k0 = 8 * (lane >> 4);
  unsigned short b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (unsigned short)(k0 + e == j ? 0x3f80 : 0);
  const uint4 w = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                             b[6] | (b[7] << 16));
  return w;
}

constexpr int kRopeMaxChunkPages = 256;  // page ids of one chunk held in LDS

template <class S>
struct RopeCfg {
  static constexpr int HG = kRopeHeadsPerWorkgroup;  // heads per workgroup (one per wavefront)
  static constexpr int NT = 64 * HG;
  static constexpr int NG = S::H / HG;             // head groups
  static constexpr int NTILE = S::DH / 16;         // 16-feature MFMA tiles of a key row
  static constexpr int KB = (S::R + 31) / 32;      // 32-wide rank blocks (zero past r)
  static constexpr int RVL = (S::RC + 3) / 4;      // R_V chunks per lane (lane = chunk, token)
  static constexpr int S_CHUNKS = 2 * S::DHC * S::P;  // 16-byte chunks of S_K and S_V
  static constexpr int SPT = S_CHUNKS / NT;
  static constexpr int PAIRS = S::DH / 2;          // rotation pairs per row
  static constexpr int CS_CHUNKS = S::P * PAIRS * 8 / 16;  // 16-byte chunks of a page's table rows
  static constexpr int CPT = CS_CHUNKS / NT;
  // LDS strides padded by one 16-byte slot so that a wavefront's reads spread over the
  // banks: S_V chunk columns of P + 1 slots (lanes read 16 columns of one token), table rows
  // of d_h/4 + 1 slots (lanes read four rows of one pair block)
  static constexpr int SV_STRIDE = S::P + 1;
  static constexpr int CS_ROW = PAIRS / 2 + 1;
  static_assert(S::BF && S::P == 16 && S::DH % 16 == 0 && S::H % HG == 0, "bf16 pages of 16");
  static_assert(S_CHUNKS % NT == 0 && CS_CHUNKS % NT == 0, "whole chunks per thread");
  static_assert(S::DH == 2 * 64, "lane l owns value features 2l, 2l+1");
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
  uint4 rk[RopeCfg<S>::KB];   // MFMA A operand: R_K[h] chunk 4kb + lane/16, token lane%16
  uint4 rv[RopeCfg<S>::RVL];  // R_V[h] chunk lane/16 + 4j, token lane%16
};

__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_r v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_r*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads of page `pg` (page index inside the request) into registers.  Private chunks past
// the rank are zeros (never loaded), so padded MFMA rank columns add nothing.
template <class S>
__device__ __forceinline__ void rope_issue(const uint8_t* __restrict__ page, const float* __restrict__ cs,
                                           int rope_rows, int pos0, int h, int tid, int lane,
                                           RopeRegs<S>& r) {
  using C = RopeCfg<S>;
  const uint4* p4 = reinterpret_cast<const uint4*>(page);
#pragma unroll
  for (int i = 0; i < C::SPT; ++i) r.st[i] = ld_stream(p4 + tid + i * C::NT);
  constexpr int ROW_CH = C::PAIRS * 8 / 16;  // 16-byte chunks of one table row
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int c = tid + i * C::NT;
    const int row = min(pos0 + c / ROW_CH, rope_rows - 1);  // rows past the table: never used
    r.cs[i] = *reinterpret_cast<const uint4*>(cs + ((size_t)row * ROW_CH + c % ROW_CH) * 4);
  }
  const int g = lane >> 4, t = lane & 15;
  const uint8_t* rk = page + S::OFF_RK + h * S::SEC_R;
  const uint8_t* rv = page + S::OFF_RV + h * S::SEC_R;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const int c = 4 * kb + g;
    r.rk[kb] = c < S::RC ? ld_stream(rk + (c * S::P + t) * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < C::RVL; ++j) {
    const int c = g + 4 * j;
    r.rv[j] = c < S::RC ? ld_stream(rv + (c * S::P + t) * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Page bytes to LDS: S_K as loaded (chunk-major: the A operand of the product that starts
// the key block's accumulator; bytes of empty slots only reach their own token's row, whose
// score is removed by selection), S_V as loaded with empty slots zeroed (their weights are
// exactly 0, and 0 x NaN would not be), the table rows as loaded.
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
  float m_run;  // running max (base-2 units), the same in every lane
  float l_run;  // running exp-sum of the page weights, the same in every lane
  float accS0, accS1;                         // features 2*lane, 2*lane + 1 of acc_S
  float accR[RopeCfg<S>::RVL][8];             // chunk lane/16 + 4j of acc_R, token lane%16
};

// One page of one head (this wavefront's).
template <class S>
__device__ __forceinline__ void rope_consume(const uint4* __restrict__ skc,
                                             const uint4* __restrict__ sv,
                                             const float2* __restrict__ csl,
                                             float* __restrict__ wl, const uint4* __restrict__ idl,
                                             const uint4 (&bk)[RopeCfg<S>::KB][RopeCfg<S>::NTILE],
                                             const float (&qf)[RopeCfg<S>::NTILE], int lane,
                                             int nvalid, float score_scale, const RopeRegs<S>& r,
                                             uint2 nrm_w, RopeState<S>& st) {
  using C = RopeCfg<S>;
  const int n = lane & 15, g = lane >> 4;
  // ---- unrotated keys of the page: K[t][f] = S_K[t][f] + sum_k R_K[h][t][k] B_K[h][f][k]
  // (lane holds tokens 4g..4g+3 of feature 16nt + n).  The accumulator starts from S_K by a
  // product with the identity, of the same shape as the private products below
  // (v_mfma_f32_16x16x32_bf16, K = 32 of which the last 16 are zero: lanes g < 2 hold
  // A = S_K[token n][features 16nt + 8g .. +7], one 16-byte read of a chunk-major row, and
  // B[k][j] = (k == j)); exact, and with no conversion of S_K on the VALU
  f32x4_r acc[C::NTILE];
  {
    const bf16x8_r ident = __builtin_bit_cast(bf16x8_r, idl[lane]);
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt) {
      const uint4 v = g < 2 ? skc[(2 * nt + g) * S::P + n] : make_uint4(0u, 0u, 0u, 0u);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_r, v), ident,
                                                        f32x4_r{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
  }
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const bf16x8_r a = __builtin_bit_cast(bf16x8_r, r.rk[kb]);
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_r, bk[kb][nt]),
                                                        acc[nt], 0, 0, 0);
  }
  // ---- score: key row t dotted with the query turned back by t's angle, q~ D_t^T:
  // (q~ D^T)_f = cos * q~_f + sin * qp_f, qp_f = q~_(f+1) for even f, -q~_(f-1) for odd f
  // (the pair partner f ^ 1 sits in lane ^ 1: one DPP swap)
  float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < C::NTILE; ++nt) {
    const int m = 8 * nt + (n >> 1);
    const float qn = qf[nt];
    const float partner = dpp_f<kQuadSwap1>(qn);
    const float qp = (n & 1) ? -partner : partner;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 c = csl[(4 * g + e) * (2 * C::CS_ROW) + m];
      const float qr = fmaf(c.x, qn, c.y * qp);
      sc[e] = fmaf(acc[nt][e], qr, sc[e]);
    }
  }
  float s[4];
  float pm = -INFINITY;
  float nrm[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (S::NORM) {  // the keys' stored joint-norm reciprocals (RMSNorm of §8)
    nrm[0] = bf16_lo(nrm_w.x);
    nrm[1] = bf16_hi(nrm_w.x);
    nrm[2] = bf16_lo(nrm_w.y);
    nrm[3] = bf16_hi(nrm_w.y);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float d = r16_sum(sc[e]);  // over the 16 features of each tile row
    s[e] = (4 * g + e) < nvalid ? d * (score_scale * nrm[e]) : -INFINITY;  // selection
    pm = fmaxf(pm, s[e]);
  }
  pm = rows4_max(pm);
  // ---- online softmax (base 2) with a lazy reference: the reference max moves only when a
  // page's max exceeds it by more than 8, and then l, acc_S and acc_R are rescaled together
  // by one factor (a wave-uniform branch, rare after the first page); weights stay <= 2^8
  if (__builtin_expect(pm > st.m_run + 8.0f, 0)) {
    const float alpha = exp2_fast(st.m_run - pm);  // 0 on the first page
    st.l_run *= alpha;
    st.accS0 *= alpha;
    st.accS1 *= alpha;
#pragma unroll
    for (int j = 0; j < C::RVL; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.accR[j][e] *= alpha;
    st.m_run = pm;
  }
  const float m_new = st.m_run;
  float w[4], ws = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e] = exp2_fast(s[e] - m_new);
    ws += w[e];
  }
  st.l_run += rows4_sum(ws);
  if (n == 0) *reinterpret_cast<float4*>(wl + 4 * g) = make_float4(w[0], w[1], w[2], w[3]);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  // ---- shared value: lane owns features 2*lane, 2*lane + 1 (chunk lane/4 of S_V)
  float a0 = st.accS0, a1 = st.accS1;
  const uint32_t* svw =
      reinterpret_cast<const uint32_t*>(sv) + (lane >> 2) * C::SV_STRIDE * 4 + (lane & 3);
#pragma unroll
  for (int t = 0; t < S::P; ++t) {
    const float wt = wl[t];
    const uint32_t v = svw[t * 4];
    a0 = fmaf(wt, bf16_lo(v), a0);
    a1 = fmaf(wt, bf16_hi(v), a1);
  }
  st.accS0 = a0;
  st.accS1 = a1;
  // ---- private value: lane (chunk, token) adds its token's weighted R_V row chunk
  const float wi = wl[lane & 15];
#pragma unroll
  for (int j = 0; j < C::RVL; ++j) {
    const uint4 v = (lane & 15) < nvalid ? r.rv[j] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t v4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      st.accR[j][2 * e] = fmaf(wi, bf16_lo(v4[e]), st.accR[j][2 * e]);
      st.accR[j][2 * e + 1] = fmaf(wi, bf16_hi(v4[e]), st.accR[j][2 * e + 1]);
    }
  }
  __builtin_amdgcn_wave_barrier();  // wl is rewritten by the next page
}

template <class S>
__global__ void __launch_bounds__(RopeCfg<S>::NT, 2) decode_rope_kernel(const RopeArgs a) {
  using C = RopeCfg<S>;
  __shared__ uint4 skc_lds[2][S::DHC * S::P];
  __shared__ uint4 sv_lds[2][S::DHC * C::SV_STRIDE];
  __shared__ uint4 cs_lds[2][S::P * C::CS_ROW];
  __shared__ __align__(16) float w_lds[C::HG][S::P];
  __shared__ int ids_lds[kRopeMaxChunkPages];
  __shared__ uint4 ident_lds[64];  // the identity B operand, read per page (not held)

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

  const int vis = visible_tokens(a.seq_lens[b], a.q_len, qi);
  const int pg0 = split * (a.chunk / S::P);
  const int tok0 = pg0 * S::P;
  const int tok1 = min(vis, min(pg0 + a.chunk / S::P, a.max_pages) * S::P);
  if (tok0 >= tok1) return;  // uniform: no record for a chunk past the visible tokens
  const int pg1 = (tok1 + S::P - 1) / S::P;
  const int n_pg = pg1 - pg0;
  for (int i = tid; i < n_pg; i += C::NT) ids_lds[i] = a.page_table[(size_t)b * a.max_pages + pg0 + i];
  if (tid < 64) ident_lds[tid] = make_ident8(tid);

  // this wavefront's head: B_K[h]^T as the MFMA B operand (lane: feature 16nt + lane%16,
  // rank 32kb + 8(lane/16) .. +8; zero past r), and the turned query's pair elements
  const int n = lane & 15, g = lane >> 4;
  uint4 bk[C::KB][C::NTILE];
  const uint8_t* bkh = static_cast<const uint8_t*>(a.BK) + (size_t)h * S::DH * S::R * 2;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt) {
      const int k0 = 32 * kb + 8 * g;
      bk[kb][nt] = k0 < S::R ? *reinterpret_cast<const uint4*>(bkh + ((size_t)(16 * nt + n) * S::R + k0) * 2)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  float qf[C::NTILE];  // q~ at feature 16nt + lane%16
  {
    const size_t row = (size_t)b * a.q_len + qi;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.q) +
                                                             (row * S::H + h) * S::DH * 2);
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt) qf[nt] = bf16_to_f32(qrow[16 * nt + n]);
  }
  __syncthreads();  // page ids in LDS

  auto page_ptr = [&](int pg) { return a.pool + (size_t)ids_lds[pg - pg0] * S::PAGE; };
  auto nvalid = [&](int pg) { return min(S::P, tok1 - pg * S::P); };

  RopeState<S> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.accS0 = st.accS1 = 0.f;
#pragma unroll
  for (int j = 0; j < C::RVL; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.accR[j][e] = 0.f;

  RopeRegs<S> r0, r1;
  rope_issue<S>(page_ptr(pg0), a.rope_cs, a.rope_rows, tok0, h, tid, lane, r0);
  if (pg0 + 1 < pg1)
    rope_issue<S>(page_ptr(pg0 + 1), a.rope_cs, a.rope_rows, tok0 + S::P, h, tid, lane, r1);
  // key-norm layouts: the stored reciprocals of this lane's tokens 4(lane/16)..+3 of the
  // next page, requested one page ahead (one value held, not one per page buffer), before
  // the loads of the page after, so waiting for them never waits for those
  auto load_norms = [&](int pg) -> uint2 {
    if constexpr (S::NORM)
      return *reinterpret_cast<const uint2*>(page_ptr(pg) + S::OFF_N + (h * S::P + 4 * (lane >> 4)) * 2);
    else
      return make_uint2(0u, 0u);
  };
  uint2 nrm_w = load_norms(pg0);
  rope_stage<S>(skc_lds[0], sv_lds[0], cs_lds[0], tid, r0, nvalid(pg0));
  __syncthreads();

  auto step = [&](int pg, int buf, RopeRegs<S>& cur, RopeRegs<S>& nxt) {
    rope_consume<S>(skc_lds[buf], sv_lds[buf], reinterpret_cast<const float2*>(cs_lds[buf]),
                    w_lds[wave], ident_lds, bk, qf, lane, nvalid(pg), a.score_scale, cur, nrm_w,
                    st);
    const bool more = pg + 1 < pg1;
    if (more) {
      rope_stage<S>(skc_lds[buf ^ 1], sv_lds[buf ^ 1], cs_lds[buf ^ 1], tid, nxt, nvalid(pg + 1));
      if constexpr (S::NORM) nrm_w = load_norms(pg + 1);
    }
    if (pg + 2 < pg1)
      rope_issue<S>(page_ptr(pg + 2), a.rope_cs, a.rope_rows, (pg + 2) * S::P, h, tid, lane, cur);
    __syncthreads();
    return more;
  };
  for (int pg = pg0;; pg += 2) {
    if (!step(pg, 0, r0, r1)) break;
    if (!step(pg + 1, 1, r1, r0)) break;
  }

  // ---- partial tuple (m, l, acc_S, acc_R) of this chunk and head, the split decode's layout
  // (the lane geometry derived anew here, so that nothing computed from it is held across
  // the page loop)
  int lane_e = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(lane_e));
  const int g_e = lane_e >> 4, n_e = lane_e & 15;
  const size_t slot = ((size_t)b * a.q_len + qi) * a.n_split + split;
  float* dst = a.part + (slot * S::H + h) * S::PART_PAD;
  if (lane_e == 0) {
    dst[0] = st.m_run;
    dst[1] = st.l_run;
  }
  *reinterpret_cast<float2*>(dst + 2 + 2 * lane_e) = make_float2(st.accS0, st.accS1);
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
