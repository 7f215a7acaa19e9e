// LRKV decode kernels for gfx950: Algorithm 2 of the LRKV notes (§3) read straight from the
// factored paged cache, as two launches on the caller's stream:
//   1. decode_split_kernel   one workgroup per (chunk of pages, query row, request) covering
//                            all heads.  Prologue: the chunk's page ids, the request length
//                            and the query row are fetched first, then the B_K rows, the
//                            first two pages are put in flight, and the private queries
//                            p = q B_K[h] of every head are formed while they travel (eq 6).
//                            Loop: shared S_K/S_V tiles staged once in LDS for every head,
//                            private R_K/R_V rows streamed per head straight into registers
//                            (page k+1 in flight while page k is used), one online
//                            softmax with a shared and a private value accumulator (fused
//                            blockwise paragraph after Algorithm 2).
//                            Writes the chunk's (max, exp-sum, acc_S, acc_R) tuple per head.
//   2. merge_expand_kernel   merges the chunks' tuples with one rescale factor per chunk,
//                            expands acc_R through B_V[h]^T once and divides by the exp-sum
//                            (the output steps of Algorithm 2, without W_O).
//
// This file is compiled with -fno-honor-nans (max reductions fuse into DPP ops); masked
// page slots are removed by integer selects, so NaN bytes there never reach arithmetic.
#include "lrkv_device.h"
#include "lrkv_launch.h"
#include "lrkv_private.h"

namespace lrkv {

// One stage of a reduce-scatter inside a 16-lane row: v[0..2n) -> v[0..n).  The DPP
// pattern pairs each lane with a partner; the lane keeps the lower or upper half (`upper`,
// its partner the other), sends the other half and adds the partner's copy of its own.
template <int CTRL, int N>
__device__ __forceinline__ void rs_stage(float* v, bool upper) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float send = upper ? v[i] : v[i + N];
    const float keep = upper ? v[i + N] : v[i];
    v[i] = keep + dpp_f<CTRL>(send);
  }
}

// Sums each of 32 values over the 16 lanes of a row; lane j ends with the sums of values
// 2j (in v[0]) and 2j + 1 (in v[1]).  The four stages pair lane j with 15 - j, with
// 7 - j inside its half, with j ^ 2 and with j ^ 1; lane j keeps the upper half at the
// stages where bit 3, 2, 1, 0 of j is set, so the values left are 16 b3 + 8 b2 + 4 b1 +
// 2 b0 = 2j and the next; each pairing joins two disjoint lane sets, so the sums cover
// all 16 lanes.
__device__ __forceinline__ void reduce_scatter_32(float* v, int j);

__device__ __forceinline__ void reduce_scatter_32(float* v, int j) {
  rs_stage<kMirror, 16>(v, j >= 8);
  rs_stage<kHalfMirror, 8>(v, (j & 7) >= 4);
  rs_stage<kQuadSwap2, 4>(v, (j & 2) != 0);
  rs_stage<kQuadSwap1, 2>(v, (j & 1) != 0);
}

// ---------------------------------------------------------------------------------------
// 1. split kernel
//
// Workgroup = (chunk, query row qi, request b), numbered so that each XCD takes a
// contiguous range of (request, row, chunk) (xcd_range_index): a request's records are
// written by one XCD (or a few), and the merge workgroups of that request run there and
// find them in its L2.  NW = H / HPW wavefronts, HPW heads each.
// For the score, the softmax and the private value, lane = hl*(16*SPLIT) + half*16 + j
// covers head h = HPW*wave + hl and token slot j of the page; with SPLIT = 2 the two
// lanes (half = 0, 1) of a (head, token) pair each take half of the features of the dot
// products and of the private value, and add their partial scores with one swizzle.  The
// shared value runs on MFMA for a bf16 cache (shared_value_mfma, one page behind the
// scores); for a float32 cache the wavefront switches to lanes over feature pairs
// (2*lane, 2*lane+1) of its HPW heads, with the weights broadcast by readlane.
//
// Pipeline: two register buffers; page pg+1 is in flight while page pg is consumed, and
// the query row and private query of the lane stay in registers; the S tiles go through a
// double-buffered LDS stage.  Page bytes are read with
// non-temporal loads: the stream is used once and should not evict the small operands that
// every workgroup re-reads (B_K, queries, page tables).
//
// Scores are in base-2 units, s = (q.S_K + p.R_K) * log2(e)/sqrt(d_h), so exp2 is used here
// and in the merge.  The running reference max of a head moves only when a page's max
// exceeds it by more than kRescaleSlack; the exp-sum and both accumulators always share
// that one reference (and are rescaled together when it moves), so l and acc are the
// same quantities the blockwise rule defines, expressed against a different common scale.
// Weights stay <= 2^kRescaleSlack, far from float32 overflow.
// ---------------------------------------------------------------------------------------
constexpr int kMaxChunkPages = 256;     // page ids of one chunk held in LDS
constexpr float kRescaleSlack = 8.0f;   // base-2 units

struct SplitArgs {
  const void* q;
  const void* BK;
  const uint8_t* pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* part;
  int max_pages;
  int q_len;
  int n_split;
  int chunk;
  int batch;
  int groups;  // balanced mode: split workgroups (0: one workgroup per chunk)
  float score_scale;
  // grouped pages: bytes from page to page and to this group's block; heads of a query
  // row and of a partial record in memory (the whole layout's), and this group's first
  // head.  A one-group page: S::PAGE, 0, S::H, S::H, 0.
  long long page_stride;
  long long page_off;
  int q_heads;
  int rec_heads;
  int head0;
  // grouped layouts in one launch: workgroup row blockIdx.y = g takes group g, whose
  // B_K slice, block of the page and first head lie these many bytes / heads further on
  long long group_bk_bytes;
  long long group_page_bytes;
  int group_heads;
  // lrkv_decode_pq: each query row's private-query block (H * P_STRIDE 16-byte slots, as
  // form_private_queries leaves it in LDS), formed beforehand by private_queries_kernel
  const uint4* p_ext;
  int p_row_slots;  // uint4 from one row's private-query blocks to the next
};

// Balanced split (single query row per request): the batch's N pages, request after request,
// are cut into G = min(groups, N) equal ranges, one per split workgroup (workgroups past G
// have no range), whatever the lengths; every range holds at least one page; a range
// crossing requests is processed as one segment per request.  The segment of request b in
// workgroup w writes its partial tuples at record slot w + b: slots are unique (ranges
// are ordered, so w' > w implies b' >= b) and a request's slots are consecutive, in page
// order.  Both kernels derive the ranges from the lengths on the device (at most
// kBalancedMaxBatch requests).

// Blocks of a 1-D grid go to the 8 XCDs round robin (block L to XCD L % 8).  This maps
// block L to index x * ceil(total / 8) + L / 8 (x = L % 8), so each XCD takes one
// contiguous range of [0, total); the grid has 8 * ceil(total / 8) blocks, indices past
// total are left idle.
__device__ __forceinline__ int xcd_range_index(int total) {
  const int per_xcd = (total + 7) / 8;
  return (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
}

// pref[b] = pages of requests 0..b-1 (pref[B] = all pages), one page per P tokens started,
// at most max_pages per request; every thread of the block takes part, the result is in
// LDS after the call.
template <int NT, int P>
__device__ __forceinline__ int page_prefix(const int32_t* __restrict__ seq_lens, int B,
                                           int max_pages, int* pref, int* wsum, int tid) {
  constexpr int PER = (kBalancedMaxBatch + NT - 1) / NT;
  int cnt[PER];
  int s = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    cnt[k] = i < B ? min((max(seq_lens[i], 0) + P - 1) / P, max_pages) : 0;
    s += cnt[k];
  }
  const int lane = tid & 63, wave = tid >> 6;
  int x = s;  // inclusive scan over the wavefront
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int acc = x - s;
  for (int w = 0; w < wave; ++w) acc += wsum[w];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    if (i < B) pref[i] = acc;
    acc += cnt[k];
  }
  if (tid == NT - 1) pref[B] = acc;  // the last thread holds the last requests
  __syncthreads();
  return pref[B];
}

// The workgroup whose range holds page p: the largest w with floor(w N / G) <= p.
__device__ __forceinline__ int group_of_page(int p, int N, int G) {
  return (int)(((long long)(p + 1) * G - 1) / N);
}

template <class S>
struct SplitCfg {
  static constexpr int HPW = PrivCfg<S>::HPW;    // heads per wave
  static constexpr int SPLIT = PrivCfg<S>::SPLIT;  // lanes per (head, token) pair
  static constexpr int NW = S::H / HPW;
  static constexpr int NT = PrivCfg<S>::NT;
  static constexpr int DHC_L = S::DHC / SPLIT;                  // S_K chunks per lane
  static constexpr int RC_L = PrivCfg<S>::RC_L;                 // private chunks per lane
  static constexpr int S_CHUNKS = 2 * S::DHC * S::P;            // 16-byte chunks of S_K + S_V
  static constexpr int SPT = (S_CHUNKS + NT - 1) / NT;          // per thread
  static constexpr int NCH = S::NORM ? S::H * S::P * S::EB / 16 : 0;  // chunks of an N section
  static_assert(NCH <= NT, "one N chunk per thread at most");
  // LDS rows of q and p per head; odd strides (in 16-byte units) spread a wavefront's
  // heads over different banks
  static constexpr int Q_STRIDE = S::DHC + 1;
  // private-query block of a row (its layout and sums: lrkv_private.h)
  static constexpr int P_PER_CHUNK = PrivCfg<S>::P_PER_CHUNK;
  static constexpr int P_STRIDE = PrivCfg<S>::P_STRIDE;
  static constexpr int PREG_N = RC_L * P_PER_CHUNK;  // uint4 of a lane's private query share
  static constexpr int PQ_JOBS = PrivCfg<S>::PQ_JOBS;
  static constexpr int PQ_GROUPS = PrivCfg<S>::PQ_GROUPS;
  static constexpr int PQ_DSPAN = PrivCfg<S>::PQ_DSPAN;
  // bf16 cache: the shared value sum_j w[h][j] S_V[j] runs on MFMA, wave w owning the
  // 16-feature tile [16w, 16w+16) for every head (HT tiles of 16 heads)
  static constexpr bool MFMA_SV = S::BF;
  static constexpr int HT = S::H / 16 > 0 ? S::H / 16 : 1;
  static_assert(!MFMA_SV || (S::H % 16 == 0 && NW * 16 == S::DH && S::P == 16),
                "MFMA shared value: 16-head tiles, one 16-feature tile per wave, 16-token pages");
  static_assert(HPW * SPLIT == 4, "64 lanes = HPW heads x SPLIT x 16 tokens");
  static_assert(S::DHC % SPLIT == 0, "shared chunks split evenly");
  static_assert(NT <= 1024, "workgroup size");
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <class S>
struct PageRegs {
  uint4 rk[SplitCfg<S>::RC_L];
  uint4 rv[SplitCfg<S>::RC_L];
  uint4 st[SplitCfg<S>::SPT];
  uint4 nst;     // key-norm layouts: threads below NCH hold 16 bytes of the page's N section
};

// Lane geometry inside the workgroup.
template <class S>
struct Lane {
  int tid, lane, wave, hl, half, j, h;
  __device__ __forceinline__ Lane(int t) {
    using C = SplitCfg<S>;
    tid = t;
    lane = t & 63;
    wave = t >> 6;
    hl = lane / (16 * C::SPLIT);
    half = (lane >> 4) & (C::SPLIT - 1);
    j = lane & 15;
    h = wave * C::HPW + hl;
  }
};

template <class S>
__device__ __forceinline__ void issue_page(const uint8_t* __restrict__ page, const Lane<S>& L,
                                           PageRegs<S>& r) {
  using C = SplitCfg<S>;
  const uint4* p4 = reinterpret_cast<const uint4*>(page);
#pragma unroll
  for (int i = 0; i < C::SPT; ++i) {
    const int c = L.tid + i * C::NT;
    if (C::S_CHUNKS % C::NT == 0 || c < C::S_CHUNKS) r.st[i] = load_stream(p4 + c);
  }
  const uint4* rkp = reinterpret_cast<const uint4*>(page + S::OFF_RK + L.h * S::SEC_R) + L.j;
  const uint4* rvp = reinterpret_cast<const uint4*>(page + S::OFF_RV + L.h * S::SEC_R) + L.j;
  // private chunks of this lane; a chunk index past the last one re-reads the last chunk
  // (its score term has p = 0 and its value term is never written out)
#pragma unroll
  for (int c = 0; c < C::RC_L; ++c) {
    const int cg = min(L.half * C::RC_L + c, S::RC - 1);
    r.rk[c] = load_stream(rkp + cg * S::P);
  }
#pragma unroll
  for (int c = 0; c < C::RC_L; ++c) {
    const int cg = min(L.half * C::RC_L + c, S::RC - 1);
    r.rv[c] = load_stream(rvp + cg * S::P);
  }
  if constexpr (S::NORM) {  // staged through LDS with the shared rows (see stage_shared)
    if (L.tid < C::NCH) r.nst = load_stream(reinterpret_cast<const uint4*>(page + S::OFF_N) + L.tid);
  }
}

// S_V row t (= S_V[t][0..DH)) keeps its 16-byte chunks in XOR-swizzled order inside the
// row, so the transposing writes below and the row reads of the value loop both avoid
// bank conflicts.
template <class S>
__device__ __forceinline__ int sv_slot(int t, int chunk) {
  return t * S::DHC + (chunk ^ (t & (S::DHC - 1)));
}

// S_K keeps the page's chunk-major order.  float32 cache: S_V is transposed to rows for the
// value loop.  bf16 cache: S_V is transposed to feature rows svt[d][t] (16 tokens of one
// feature contiguous), the B operand layout of the MFMA value product.  Slots past the last
// visible token are written as zeros (their weights are exactly zero, and 0 x NaN would
// not be).
template <class S>
__device__ __forceinline__ void stage_shared(uint4* __restrict__ sk, uint4* __restrict__ sv,
                                             uint16_t* __restrict__ svt, uint4* __restrict__ nl,
                                             int tid, const PageRegs<S>& r, int nvalid) {
  using C = SplitCfg<S>;
  // key-norm layouts: the page's N section (one reciprocal per head and slot) next to the
  // shared rows, read by every lane after the barrier; held in LDS rather than as one value
  // per lane in the page registers, so no wait for it can end up waiting on later loads
  if constexpr (S::NORM)
    if (tid < C::NCH) nl[tid] = r.nst;
#pragma unroll
  for (int i = 0; i < C::SPT; ++i) {
    const int c = tid + i * C::NT;
    if (c < S::DHC * S::P) {
      sk[c] = r.st[i];
    } else if (C::S_CHUNKS % C::NT == 0 || c < C::S_CHUNKS) {
      const int cc = c - S::DHC * S::P;
      const int t = cc % S::P;
      const uint4 v = t < nvalid ? r.st[i] : make_uint4(0u, 0u, 0u, 0u);
      if constexpr (C::MFMA_SV) {
        uint16_t* col = svt + (cc / S::P) * S::CE * S::P + t;  // feature 8*(cc/P), token t
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          col[(2 * e) * S::P] = (uint16_t)(w4[e] & 0xffffu);
          col[(2 * e + 1) * S::P] = (uint16_t)(w4[e] >> 16);
        }
      } else {
        sv[sv_slot<S>(t, cc / S::P)] = v;
      }
    }
  }
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Shared value of one page on MFMA (bf16 cache): for every head tile,
//   acc[h][d] = acc[h][d] * alpha[h] + sum_t W[h][t] S_V[t][d],   d in this wave's tile,
// with W held as bfloat16 hi + lo parts (two products, ~16 significant bits of each
// weight).  v_mfma_f32_16x16x16_bf16 lane layout: A[i][k] at lane 16*(k/4) + i, element
// k%4; B[k][j] at lane 16*(k/4) + j; D[i][j] at lane 16*(i/4) + j, element i%4.
template <class S>
__device__ __forceinline__ void shared_value_mfma(f32x4* acc, const uint16_t* __restrict__ wl,
                                                  const float* __restrict__ al,
                                                  const uint16_t* __restrict__ svt, int wave,
                                                  int lane) {
  using C = SplitCfg<S>;
  const int i = lane & 15, g = lane >> 4;
  const short4v b = *reinterpret_cast<const short4v*>(svt + (16 * wave + i) * S::P + 4 * g);
#pragma unroll
  for (int ht = 0; ht < C::HT; ++ht) {
    const float4 a4 = *reinterpret_cast<const float4*>(al + 16 * ht + 4 * g);
    acc[ht][0] *= a4.x;
    acc[ht][1] *= a4.y;
    acc[ht][2] *= a4.z;
    acc[ht][3] *= a4.w;
    const short4v whi = *reinterpret_cast<const short4v*>(wl + (16 * ht + i) * S::P + 4 * g);
    const short4v wlo =
        *reinterpret_cast<const short4v*>(wl + (S::H + 16 * ht + i) * S::P + 4 * g);
    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(whi, b, acc[ht], 0, 0, 0);
    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wlo, b, acc[ht], 0, 0, 0);
  }
}

// B_K rows of this thread's private-query job: job (head h, 16-byte chunk c of p), rows
// d in group g's span.  Issued before any page load: vector loads return in issue order,
// so rows requested after the pages would wait for the pages.
template <class S>
struct BKRows {
  uint4 v[SplitCfg<S>::PQ_DSPAN];
};

// SKIP_IDLE: wavefronts wholly past the last group load nothing (the balanced split, whose
// loop over segments leaves no registers to spare, keeps the loads unconditional: the
// branch made it spill).  A thread past the last group in a wavefront that loads reads a
// valid row it never uses.
template <class S, bool SKIP_IDLE>
__device__ __forceinline__ void load_bk_rows(const void* __restrict__ BK, int tid, BKRows<S>& r) {
  using C = SplitCfg<S>;
  const int job = tid % C::PQ_JOBS;
  const int g = min(tid / C::PQ_JOBS, C::PQ_GROUPS - 1);
  const int h = job / S::RC;
  const int c = job - h * S::RC;
  const uint8_t* bk = static_cast<const uint8_t*>(BK) +
                      ((size_t)h * S::DH * S::R + (size_t)c * S::CE) * S::EB;
  if (!SKIP_IDLE || __builtin_amdgcn_readfirstlane(tid) < C::PQ_GROUPS * C::PQ_JOBS) {
#pragma unroll
    for (int dd = 0; dd < C::PQ_DSPAN; ++dd)
      r.v[dd] = *reinterpret_cast<const uint4*>(bk + (size_t)(g * C::PQ_DSPAN + dd) * S::R * S::EB);
  }
  asm volatile("" ::: "memory");  // keep them ahead of the page loads that follow
}

// p = q B_K[h] for every head of the row, float32 sums over d_h in a fixed order (the one
// private_query_block follows), packed into LDS for the private score as
// store_private_chunk lays it out.
template <class S>
__device__ __forceinline__ void form_private_queries(const BKRows<S>& bkr,
                                                     const uint4* __restrict__ q_lds,
                                                     float* __restrict__ pacc,
                                                     uint4* __restrict__ p_lds, int tid) {
  using C = SplitCfg<S>;
  const int job = tid % C::PQ_JOBS;
  const int g = tid / C::PQ_JOBS;
  if (g < C::PQ_GROUPS) {
    const int h = job / S::RC;
    float acc[S::CE];
#pragma unroll
    for (int e = 0; e < S::CE; ++e) acc[e] = 0.f;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q_lds + h * C::Q_STRIDE);
#pragma unroll
    for (int dd = 0; dd < C::PQ_DSPAN; ++dd) {
      const int d = g * C::PQ_DSPAN + dd;
      const uint4 b4 = bkr.v[dd];
      if constexpr (S::BF) {
        const float qd = bf16_to_f32(reinterpret_cast<const uint16_t*>(qrow)[d]);
        acc[0] = fmaf(qd, bf16_lo(b4.x), acc[0]);
        acc[1] = fmaf(qd, bf16_hi(b4.x), acc[1]);
        acc[2] = fmaf(qd, bf16_lo(b4.y), acc[2]);
        acc[3] = fmaf(qd, bf16_hi(b4.y), acc[3]);
        acc[4] = fmaf(qd, bf16_lo(b4.z), acc[4]);
        acc[5] = fmaf(qd, bf16_hi(b4.z), acc[5]);
        acc[6] = fmaf(qd, bf16_lo(b4.w), acc[6]);
        acc[7] = fmaf(qd, bf16_hi(b4.w), acc[7]);
      } else {
        const float qd = reinterpret_cast<const float*>(qrow)[d];
        acc[0] = fmaf(qd, __uint_as_float(b4.x), acc[0]);
        acc[1] = fmaf(qd, __uint_as_float(b4.y), acc[1]);
        acc[2] = fmaf(qd, __uint_as_float(b4.z), acc[2]);
        acc[3] = fmaf(qd, __uint_as_float(b4.w), acc[3]);
      }
    }
#pragma unroll
    for (int e = 0; e < S::CE; ++e) pacc[(g * C::PQ_JOBS + job) * S::CE + e] = acc[e];
  }
  constexpr int PAD = C::P_STRIDE - S::RC * C::P_PER_CHUNK;  // zero slots per head
  if constexpr (PAD > 0) {
    for (int i = tid; i < S::H * PAD; i += C::NT)
      p_lds[(i / PAD) * C::P_STRIDE + S::RC * C::P_PER_CHUNK + i % PAD] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  if (tid < C::PQ_JOBS) {
    const int h = tid / S::RC;
    const int c = tid - h * S::RC;
    float p[S::CE];
#pragma unroll
    for (int e = 0; e < S::CE; ++e) {
      float v = 0.f;
#pragma unroll
      for (int gg = 0; gg < C::PQ_GROUPS; ++gg) v += pacc[(gg * C::PQ_JOBS + tid) * S::CE + e];
      p[e] = v;
    }
    store_private_chunk<S>(p_lds + h * C::P_STRIDE + c * C::P_PER_CHUNK, p);
  }
}

template <class S>
struct SplitState {
  float m_run;                                // reference max of the lane's head
  float l_run;                                // this lane's share of the exp-sum
  float accR[SplitCfg<S>::RC_L * S::CE];      // its share of sum_j w_j R_V[h, j] (its half)
  float accS[SplitCfg<S>::HPW][2];            // float32 cache: sum_j w_j S_V[j][2*lane + e]
  f32x4 accT[SplitCfg<S>::HT];                // bf16 cache: MFMA tiles of acc_S (see above)
};

// the partner lane of a (head, token) pair (lane ^ 16) holds the other half of the
// features; v_permlane16_swap hands each lane of the pair both values (VALU, no LDS round
// trip), and both lanes form the same sum
__device__ __forceinline__ float add_partner(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <class S, bool PREG>
__device__ __forceinline__ void consume_page(const uint4* __restrict__ sk,
                                             const uint4* __restrict__ sv,
                                             const uint4 (&qreg)[SplitCfg<S>::DHC_L],
                                             const uint4 (&preg)[SplitCfg<S>::PREG_N],
                                             const uint4* __restrict__ p_lds,
                                             uint16_t* __restrict__ wl, float* __restrict__ al,
                                             const Lane<S>& L, int nvalid, float score_scale,
                                             const uint4* __restrict__ nl, PageRegs<S>& r,
                                             SplitState<S>& st) {
  using C = SplitCfg<S>;
  const int j = L.j;
  const bool valid = j < nvalid;
  // ---- score: q . S_K[j] + p . R_K[h, j]   (eq 6), this lane's half of the features
  float acc0 = 0.f, acc1 = 0.f;
  const uint4* skh = sk + L.half * C::DHC_L * S::P;
#pragma unroll
  for (int c = 0; c < C::DHC_L; ++c) {
    const uint4 s4 = skh[c * S::P + j];
    const uint4 q4 = qreg[c];
    if constexpr (S::BF) {
      acc0 = dot2_bf16(q4.x, s4.x, acc0);
      acc1 = dot2_bf16(q4.y, s4.y, acc1);
      acc0 = dot2_bf16(q4.z, s4.z, acc0);
      acc1 = dot2_bf16(q4.w, s4.w, acc1);
    } else {
      acc0 = fmaf(__uint_as_float(q4.x), __uint_as_float(s4.x), acc0);
      acc1 = fmaf(__uint_as_float(q4.y), __uint_as_float(s4.y), acc1);
      acc0 = fmaf(__uint_as_float(q4.z), __uint_as_float(s4.z), acc0);
      acc1 = fmaf(__uint_as_float(q4.w), __uint_as_float(s4.w), acc1);
    }
  }
  const uint4* ph = p_lds + L.h * C::P_STRIDE;
#pragma unroll
  for (int c = 0; c < C::RC_L; ++c) {
    const int cg = L.half * C::RC_L + c;  // slots past RC hold p = 0
    const uint4 k4 = r.rk[c];
    if constexpr (S::BF) {
      const uint4 hi = PREG ? preg[2 * c] : ph[2 * cg];
      const uint4 lo = PREG ? preg[2 * c + 1] : ph[2 * cg + 1];
      acc0 = dot2_bf16(hi.x, k4.x, acc0);
      acc1 = dot2_bf16(hi.y, k4.y, acc1);
      acc0 = dot2_bf16(hi.z, k4.z, acc0);
      acc1 = dot2_bf16(hi.w, k4.w, acc1);
      acc0 = dot2_bf16(lo.x, k4.x, acc0);
      acc1 = dot2_bf16(lo.y, k4.y, acc1);
      acc0 = dot2_bf16(lo.z, k4.z, acc0);
      acc1 = dot2_bf16(lo.w, k4.w, acc1);
    } else {
      const uint4 p4 = PREG ? preg[c] : ph[cg];
      acc0 = fmaf(__uint_as_float(p4.x), __uint_as_float(k4.x), acc0);
      acc1 = fmaf(__uint_as_float(p4.y), __uint_as_float(k4.y), acc1);
      acc0 = fmaf(__uint_as_float(p4.z), __uint_as_float(k4.z), acc0);
      acc1 = fmaf(__uint_as_float(p4.w), __uint_as_float(k4.w), acc1);
    }
  }
  float full = acc0 + acc1;
  if constexpr (C::SPLIT == 2) full = add_partner(full);
  float scale = score_scale;
  if constexpr (S::NORM)  // the key's stored joint-norm reciprocal multiplies the summed score
    scale *= S::BF ? bf16_to_f32(reinterpret_cast<const uint16_t*>(nl)[L.h * S::P + j])
                   : reinterpret_cast<const float*>(nl)[L.h * S::P + j];
  // masked slots leave by selection, never by multiplying with zero
  const float s = valid ? full * scale : -INFINITY;

  // ---- online softmax: the reference moves (and rescales l, acc_S, acc_R by one factor)
  // only when the page's max clears it by more than the slack
  const float pm = r16_max(s);
  const bool bump = pm > st.m_run + kRescaleSlack;
  float alpha = 1.f;
  if (__builtin_expect(__any(bump), 0)) {  // rare after the first page: a real branch
    asm volatile("" ::: "memory");
    const float m_new = bump ? pm : st.m_run;
    alpha = exp2_fast(st.m_run - m_new);  // 0 on the first page, 1 if not bumped
    st.l_run *= alpha;
#pragma unroll
    for (int k = 0; k < C::RC_L * S::CE; ++k) st.accR[k] *= alpha;
    if constexpr (!C::MFMA_SV) {
#pragma unroll
      for (int x = 0; x < C::HPW; ++x) {
        const float a = readlane_f(alpha, x * 16 * C::SPLIT);
        st.accS[x][0] *= a;
        st.accS[x][1] *= a;
      }
    }
    st.m_run = m_new;
  }
  const float w = exp2_fast(s - st.m_run);  // exactly 0 for masked slots
  st.l_run += w;
  if constexpr (C::MFMA_SV) {
    // weights as bfloat16 hi + lo for the MFMA shared value of this page (run by every
    // wave after the next barrier), and the head's rescale factor for its accumulator
    if (L.half == 0) {
      const uint32_t hi = f32_to_bf16_rne(w);
      const uint32_t lo = f32_to_bf16_rne(w - bf16_to_f32((uint16_t)hi));
      wl[L.h * S::P + L.j] = (uint16_t)hi;
      wl[(S::H + L.h) * S::P + L.j] = (uint16_t)lo;
      if (L.j == 0) al[L.h] = alpha;
    }
  }
  // only the last page of a request has empty slots: their R_V bytes are replaced by
  // zeros there (selection), full pages skip the selects
  if (__builtin_expect(nvalid < S::P, 0)) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < C::RC_L; ++c)
      if (!valid) r.rv[c] = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int c = 0; c < C::RC_L; ++c) {
    const uint32_t v4[4] = {r.rv[c].x, r.rv[c].y, r.rv[c].z, r.rv[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (S::BF) {
        const int k = 8 * c + 2 * e;
        st.accR[k] = fmaf(w, bf16_lo(v4[e]), st.accR[k]);
        st.accR[k + 1] = fmaf(w, bf16_hi(v4[e]), st.accR[k + 1]);
      } else {
        const int k = 4 * c + e;
        st.accR[k] = fmaf(w, __uint_as_float(v4[e]), st.accR[k]);
      }
    }
  }

  // ---- shared value (float32 cache): lanes over feature pairs, weights broadcast by
  // readlane.  The bf16 cache does this on MFMA (shared_value_mfma).
  if constexpr (!C::MFMA_SV) {
    float sA[C::HPW], sB[C::HPW];
#pragma unroll
    for (int x = 0; x < C::HPW; ++x) {
      sA[x] = st.accS[x][0];
      sB[x] = st.accS[x][1];
    }
    const int dl = (2 * L.lane < S::DH) ? L.lane : (S::DH / 2 - 1);
    const int e0 = 2 * dl;  // first feature of the pair
#pragma unroll
    for (int t = 0; t < S::P; ++t) {
      const int slot = sv_slot<S>(t, e0 / S::CE) * S::CE + (e0 % S::CE);  // element index
      const float2 pr = reinterpret_cast<const float2*>(sv)[slot / 2];
      const float sv0 = pr.x, sv1 = pr.y;
#pragma unroll
      for (int x = 0; x < C::HPW; ++x) {
        const float wt = readlane_f(w, x * 16 * C::SPLIT + t);
        sA[x] = fmaf(wt, sv0, sA[x]);
        sB[x] = fmaf(wt, sv1, sB[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < C::HPW; ++x) {
      st.accS[x][0] = sA[x];
      st.accS[x][1] = sB[x];
    }
  }
}

template <class S, bool BAL, bool EXTP = false>
__global__ void __launch_bounds__(SplitCfg<S>::NT, 1)
decode_split_kernel(const SplitArgs a) {
  using C = SplitCfg<S>;
  constexpr int SV_ROWS = C::MFMA_SV ? 1 : S::P * S::DHC;
  constexpr int SVT_BUFS = C::MFMA_SV ? 3 : 1;
  constexpr int SVT_ELEMS = C::MFMA_SV ? S::DH * S::P : 8;
  constexpr int W_ELEMS = C::MFMA_SV ? 2 * S::H * S::P : 8;
  __shared__ uint4 sk_lds[2][S::DHC * S::P];  // chunk-major [c][t], double buffered
  __shared__ uint4 sv_lds[2][SV_ROWS];        // float32 cache: rows [t][swizzled c]
  // bf16 cache: S_V feature rows [d][t] (three buffers: page k is read by the MFMA during
  // step k+1 while page k+2 is staged), weights hi/lo [2][H][t] and rescale factors [H]
  // of the last consumed page (two buffers)
  __shared__ __align__(16) uint16_t svt_lds[SVT_BUFS][SVT_ELEMS];
  __shared__ __align__(16) uint16_t w_lds[2][W_ELEMS];
  __shared__ __align__(16) float al_lds[2][S::H];
  __shared__ uint4 q_lds[S::H * C::Q_STRIDE];
  __shared__ uint4 p_lds[S::H * C::P_STRIDE];
  __shared__ float pacc[C::PQ_GROUPS * C::PQ_JOBS * S::CE];
  __shared__ int ids_lds[kMaxChunkPages];
  __shared__ int pref_lds[BAL ? kBalancedMaxBatch + 1 : 1];
  __shared__ int wsum_lds[BAL ? C::NW : 1];
  __shared__ uint4 n_lds[2][C::NCH > 0 ? C::NCH : 1];  // key-norm layouts: N sections

  const int grp = (int)blockIdx.y;  // 0 unless a grouped layout runs in one launch
  const uint8_t* BKg = static_cast<const uint8_t*>(a.BK) + (size_t)grp * a.group_bk_bytes;
  const long long page_off = a.page_off + (long long)grp * a.group_page_bytes;
  const int head0 = a.head0 + grp * a.group_heads;
  // segment: request b, query row qi, pages [pg0, pg_end) of the request, record slot
  int b, qi, pg0, pg_end;
  size_t slot;
  int g_hi = 0;  // balanced: end of this workgroup's range (page index over the batch)
  if constexpr (BAL) {
    const int N = page_prefix<C::NT, S::P>(a.seq_lens, a.batch, a.max_pages, pref_lds, wsum_lds,
                                           (int)threadIdx.x);
    // ranges over at most N workgroups, so that every range holds at least one page (the
    // merge takes every slot between a request's first and last range as written)
    const int G = min(a.groups, N);
    if ((int)blockIdx.x >= G) return;  // uniform for the whole workgroup
    const int g_lo = (int)((long long)blockIdx.x * N / G);
    g_hi = (int)((long long)(blockIdx.x + 1) * N / G);
    int lo = 0, hi = a.batch - 1;  // the request holding page g_lo
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (pref_lds[mid + 1] > g_lo) hi = mid;
      else lo = mid + 1;
    }
    b = lo;
    qi = 0;
    pg0 = g_lo - pref_lds[b];
    pg_end = min(g_hi, pref_lds[b + 1]) - pref_lds[b];
    slot = (size_t)blockIdx.x + b;
  } else {
    // (request, row, chunk) index g in order; XCD x (blocks go to the 8 XCDs round robin)
    // takes the contiguous range of g starting at x * per_xcd, so a request's records are
    // written by as few XCDs as possible and the merge reads them there
    const int total = a.batch * a.q_len * a.n_split;
    const int g = xcd_range_index(total);
    if (g >= total) return;  // uniform
    const int split = g % a.n_split;
    qi = (g / a.n_split) % a.q_len;
    b = g / (a.n_split * a.q_len);
    pg0 = split * (a.chunk / S::P);
    pg_end = pg0 + a.chunk / S::P;
    slot = (size_t)g;
  }
  for (;;) {
  // the lane's geometry is derived anew for each segment: values computed from it are then
  // not kept live across the segment loop (which made the balanced kernel spill)
  int t_in = (int)threadIdx.x;
  if constexpr (BAL) asm volatile("" : "+v"(t_in));
  const Lane<S> L(t_in);
  const int tid = L.tid;
  const size_t row = (size_t)b * a.q_len + qi;

  // the request length (scalar load) and this segment's page ids and query row (vector
  // loads) travel together
  const int nid = min(pg_end - pg0, a.max_pages - pg0);  // table entries of this segment
  const int32_t* tab = a.page_table + (size_t)b * a.max_pages + pg0;
  int id_r[(kMaxChunkPages + C::NT - 1) / C::NT];
#pragma unroll
  for (int k = 0; k < (kMaxChunkPages + C::NT - 1) / C::NT; ++k) {
    const int i = tid + k * C::NT;
    if (i < nid) id_r[k] = tab[i];
  }
  constexpr int QCH = (S::H * S::DHC + C::NT - 1) / C::NT;
  uint4 q_r[QCH];
  const uint4* qsrc = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) +
                                                     (row * a.q_heads + head0) * S::DH * S::EB);
#pragma unroll
  for (int k = 0; k < QCH; ++k) {
    const int i = tid + k * C::NT;
    if (i < S::H * S::DHC) q_r[k] = qsrc[i];
  }
  // lrkv_decode_pq: the row's private-query block travels with them, in place of the B_K
  // rows and the formation below
  constexpr int PBL = S::H * C::P_STRIDE;  // 16-byte slots of a row's block
  constexpr int PCH = EXTP ? (PBL + C::NT - 1) / C::NT : 1;
  uint4 p_r[PCH];
  if constexpr (EXTP) {
#pragma unroll
    for (int k = 0; k < PCH; ++k) {
      const int i = tid + k * C::NT;
      if (i < PBL) p_r[k] = a.p_ext[row * a.p_row_slots + (size_t)grp * PBL + i];
    }
  }
  // the request length is read first (a scalar load)
  const int len_b = a.seq_lens[b];
  const int vis = visible_tokens(len_b, a.q_len, qi);
  const int tok0 = pg0 * S::P;
  // pages past the table row are never read, whatever the lengths say
  const int tok1 = min(vis, min(pg_end, a.max_pages) * S::P);
  if (tok0 < tok1) {  // uniform for the whole workgroup
#pragma unroll
  for (int k = 0; k < (kMaxChunkPages + C::NT - 1) / C::NT; ++k) {
    const int i = tid + k * C::NT;
    if (i < nid) ids_lds[i] = id_r[k];
  }
  // q (and the private queries, given) go to LDS: before the barrier where the private
  // queries are formed here, after the first pages are requested where they are given
  auto store_q_p = [&]() {
#pragma unroll
    for (int k = 0; k < QCH; ++k) {
      const int i = tid + k * C::NT;
      if (i < S::H * S::DHC) q_lds[(i / S::DHC) * C::Q_STRIDE + i % S::DHC] = q_r[k];
    }
    if constexpr (EXTP) {
#pragma unroll
      for (int k = 0; k < PCH; ++k) {
        const int i = tid + k * C::NT;
        if (i < PBL) p_lds[i] = p_r[k];
      }
    }
  };
  if constexpr (!EXTP) store_q_p();
  __syncthreads();  // page ids (and q where the private queries are formed here) in LDS
  // B_K rows go out once the page ids are in (ahead of them they delay the ids: every
  // workgroup reads all of B_K, 58 MB of L2 traffic at C1 sizes) and ahead of every page
  // load, since loads return in issue order
  BKRows<S> bkr;
  if constexpr (!EXTP) load_bk_rows<S, !BAL>(BKg, tid, bkr);

  const int pg1 = (tok1 + S::P - 1) / S::P;
  const uint8_t* pool = a.pool;
  auto page_ptr = [&](int pg) {
    return pool + (size_t)ids_lds[pg - pg0] * (size_t)a.page_stride + (size_t)page_off;
  };
  auto nvalid = [&](int pg) { return min(S::P, tok1 - pg * S::P); };

  // two register buffers of pages: page k+1 travels while page k is consumed, and page
  // k+2 goes in flight into k's buffer once k is consumed (measured faster than three or
  // four buffers: the registers hold the query row and the private query instead)
  PageRegs<S> r0, r1;
  // pages pg0, pg0+1 go in flight while the private queries are formed
  issue_page<S>(page_ptr(pg0), L, r0);
  if (pg0 + 1 < pg1) issue_page<S>(page_ptr(pg0 + 1), L, r1);
  if constexpr (EXTP) store_q_p();  // the barrier after the first page's staging covers them
  if constexpr (!EXTP) form_private_queries<S>(bkr, q_lds, pacc, p_lds, tid);
  stage_shared<S>(sk_lds[0], sv_lds[0], svt_lds[0], n_lds[0], tid, r0, nvalid(pg0));
  __syncthreads();

  // this lane's half of its head's query row, and its share of the private query (hi and
  // lo parts for bf16), in registers for the whole segment; the balanced split and the
  // key-norm layout of the 32-head shape have no room for the private share, which stays
  // in LDS there
  constexpr bool PREG = (!BAL && !S::NORM) || S::H <= 16;
  uint4 qreg[C::DHC_L];
#pragma unroll
  for (int c = 0; c < C::DHC_L; ++c) qreg[c] = q_lds[L.h * C::Q_STRIDE + L.half * C::DHC_L + c];
  uint4 preg[C::PREG_N];
  if constexpr (PREG) {
#pragma unroll
    for (int c = 0; c < C::PREG_N; ++c) preg[c] = p_lds[L.h * C::P_STRIDE + L.half * C::PREG_N + c];
  }

  SplitState<S> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int k = 0; k < C::RC_L * S::CE; ++k) st.accR[k] = 0.f;
#pragma unroll
  for (int x = 0; x < C::HPW; ++x) st.accS[x][0] = st.accS[x][1] = 0.f;
#pragma unroll
  for (int x = 0; x < C::HT; ++x) st.accT[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one pipeline step: page pg is in `cur` and LDS buffer `buf`, page pg+1 in `nxt`; page
  // pg+2 goes in flight into `cur` once pg is consumed.  bf16 cache: the shared value of
  // page pg-1 (weights written last step) goes through MFMA first.  Returns false when pg
  // was the last page.
  auto step = [&](int pg, int buf, PageRegs<S>& cur, PageRegs<S>& nxt) {
    const int k = pg - pg0;
    if constexpr (C::MFMA_SV) {
      if (k > 0)
        shared_value_mfma<S>(st.accT, w_lds[buf ^ 1], al_lds[buf ^ 1], svt_lds[(k + 2) % 3],
                             L.wave, L.lane);
    }
    consume_page<S, PREG>(sk_lds[buf], sv_lds[buf], qreg, preg, p_lds, w_lds[buf], al_lds[buf],
                          L, nvalid(pg), a.score_scale, n_lds[buf], cur, st);
    const bool more = pg + 1 < pg1;
    if (more)
      stage_shared<S>(sk_lds[buf ^ 1], sv_lds[buf ^ 1], svt_lds[C::MFMA_SV ? (k + 1) % 3 : 0],
                      n_lds[buf ^ 1], tid, nxt, nvalid(pg + 1));
    if (pg + 2 < pg1) issue_page<S>(page_ptr(pg + 2), L, cur);
    __syncthreads();
    return more;
  };
  for (int pg = pg0;; pg += 2) {
    if (!step(pg, 0, r0, r1)) break;
    if (!step(pg + 1, 1, r1, r0)) break;
  }
  if constexpr (C::MFMA_SV) {  // shared value of the last page
    const int kl = pg1 - 1 - pg0;
    shared_value_mfma<S>(st.accT, w_lds[kl & 1], al_lds[kl & 1], svt_lds[kl % 3], L.wave, L.lane);
  }

  // ---- partial tuple of this chunk: m, l, acc_S[DH], acc_R[R] per head
  const float l_tot = r16_sum(st.l_run);
  float* dst = a.part + (slot * a.rec_heads + head0 + L.h) * S::PART_PAD;
  if (L.j == 0 && L.half == 0) {
    dst[0] = st.m_run;
    dst[1] = l_tot;
  }
  constexpr int NR = C::RC_L * S::CE;  // acc_R values per lane (its half of the features)
  if constexpr (NR == 32) {
    // reduce-scatter over the 16 token lanes of the row: lane j ends with the sums of
    // values 2j and 2j + 1, stored as one float2
    reduce_scatter_32(st.accR, L.j);
    const int kg = L.half * NR + 2 * L.j;  // feature of R_V
    if (kg < S::R)
      *reinterpret_cast<float2*>(dst + 2 + S::DH + kg) = make_float2(st.accR[0], st.accR[1]);
  } else {
#pragma unroll
    for (int k = 0; k < NR; ++k) st.accR[k] = r16_sum(st.accR[k]);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int kg = L.half * NR + k;  // feature of R_V
      if ((k & 15) == L.j && kg < S::R) dst[2 + S::DH + kg] = st.accR[k];
    }
  }
  if constexpr (C::MFMA_SV) {
    // MFMA tile: lane holds heads 16*ht + 4*(lane/16) + e, feature 16*wave + lane%16
    float* rec = a.part + (slot * a.rec_heads + head0) * S::PART_PAD;
#pragma unroll
    for (int ht = 0; ht < C::HT; ++ht)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rec[(16 * ht + 4 * (L.lane >> 4) + e) * S::PART_PAD + 2 + 16 * L.wave + (L.lane & 15)] =
            st.accT[ht][e];
  } else if (2 * L.lane < S::DH) {
#pragma unroll
    for (int x = 0; x < C::HPW; ++x) {
      float2* d2 = reinterpret_cast<float2*>(
          a.part + (slot * a.rec_heads + head0 + C::HPW * L.wave + x) * S::PART_PAD + 2 +
          2 * L.lane);
      *d2 = make_float2(st.accS[x][0], st.accS[x][1]);
    }
  }
  }  // tok0 < tok1
  if constexpr (!BAL) {
    break;
  } else {  // the next request of this workgroup's range, if any
    if (++b >= a.batch || pref_lds[b] >= g_hi) break;
    pg0 = 0;
    pg_end = min(g_hi, pref_lds[b + 1]) - pref_lds[b];
    slot = (size_t)blockIdx.x + b;
    __syncthreads();  // LDS of the last segment is reused
  }
  }  // segments
}

// ---------------------------------------------------------------------------------------
// 2. merge + expand.  Workgroup = (head, query row, request), 256 threads, on the XCD that
// wrote the request's records (chunked split; see xcd_range_index).  Thread t owns
// one column of the partial record: t < DH -> acc_S[t], t < DH + R -> acc_R[t - DH],
// t == DH + R -> l.  When every chunk fits in LDS (the usual case) one memory round trip
// does: the records of all n_split chunks (16-byte loads issued together, before the request
// length is known; records past the visible chunks are ignored) and the thread's B_V row.
// Then m* and the weights exp2(m_s - m*) come from the LDS copy, columns are summed over the
// chunks in chunk order, and o[d] = (A_S[d] + A_R . B_V[h][d]) / L.  Balanced split: the
// request's records are those of the workgroups whose page ranges meet it (slot w + b),
// found from the lengths first; a workgroup skips nothing and the count is exact.
// ---------------------------------------------------------------------------------------
template <class S, bool BAL>
__global__ void __launch_bounds__(256)
merge_expand_kernel(const float* __restrict__ part, const void* __restrict__ BV,
                    const int32_t* __restrict__ seq_lens, int q_len, int n_split, int chunk,
                    int batch, int groups, int max_pages, void* __restrict__ out) {
  static_assert(S::DH + S::R + 1 <= 256, "one thread per column");
  constexpr int PP = S::PART_PAD;
  constexpr int MS_LDS = (48 * 1024) / (PP * 4);
  constexpr int MS = MS_LDS < 256 ? MS_LDS : 256;  // chunks per pass held in LDS
  constexpr int LP = (MS * (PP / 4) + 255) / 256;  // 16-byte loads per thread and pass
  __shared__ float4 tile[LP * 256];                // records, then padding
  __shared__ float wts[MS];
  __shared__ float red[4];
  __shared__ float accR_s[S::R];
  __shared__ float l_s;
  int h, qi, b;
  if constexpr (BAL) {
    h = blockIdx.x;
    qi = blockIdx.y;
    b = blockIdx.z;
  } else {  // (request, row, head) ranges per XCD, as the split kernel's chunks
    const int total = batch * q_len * S::H;
    const int g = xcd_range_index(total);
    if (g >= total) return;
    h = g % S::H;
    qi = (g / S::H) % q_len;
    b = g / (S::H * q_len);
  }
  const int t = threadIdx.x;
  const size_t row = (size_t)b * q_len + qi;
  const size_t out_off = (row * S::H + h) * S::DH;
  const int col = t < S::DH + S::R ? 2 + t : (t == S::DH + S::R ? 1 : -1);
  const float* base = part + (row * n_split * S::H + h) * PP;
  const size_t stride = (size_t)S::H * PP;  // floats between chunks of the same head
  const float* tf = reinterpret_cast<const float*>(tile);
  int cap = n_split;  // records that may be read
  int n_bal = 0;      // balanced: this request's records
  if constexpr (BAL) {
    __shared__ int pref_s[kBalancedMaxBatch + 1];
    __shared__ int wsum_s[4];
    const int N = page_prefix<256, S::P>(seq_lens, batch, max_pages, pref_s, wsum_s, t);
    const int G = min(groups, N);  // the split kernel's ranges: each holds a page
    const int p0 = pref_s[b], p1 = pref_s[b + 1];
    const int w0 = p1 > p0 ? group_of_page(p0, N, G) : 0;
    n_bal = p1 > p0 ? group_of_page(p1 - 1, N, G) - w0 + 1 : 0;
    base = part + (((size_t)w0 + b) * S::H + h) * PP;
    cap = n_bal;
  }

  // a pass of cnt <= MS records into LDS: every load of the thread goes out before the
  // first LDS write (one memory round trip, not one per 16 bytes); lanes past the pass
  // read its last 16 bytes again and write them past its records (never read), so
  // neither the loads nor the writes need a branch
  auto load_pass = [&](int s0, int cnt) {
    const int last = cnt * (PP / 4) - 1;
    float4 v[LP];
#pragma unroll
    for (int k = 0; k < LP; ++k) {
      const int i = min(t + 256 * k, last);
      const int s = i / (PP / 4), c4 = i - s * (PP / 4);
      v[k] = reinterpret_cast<const float4*>(base + (size_t)(s0 + s) * stride)[c4];
    }
#pragma unroll
    for (int k = 0; k < LP; ++k) tile[t + 256 * k] = v[k];
  };
  // B_V row and first pass go out before the length is known
  constexpr int BVW = S::R * S::EB / 16;
  uint4 bvr[BVW];
  if (t < S::DH) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(BV) +
                                                      ((size_t)h * S::DH + t) * S::R * S::EB);
#pragma unroll
    for (int c = 0; c < BVW; ++c) bvr[c] = src[c];
  }
  if (cap > 0 && cap <= MS) load_pass(0, cap);
  const int vis = visible_tokens(seq_lens[b], q_len, qi);
  const int n = BAL ? n_bal : (vis + chunk - 1) / chunk;
  if (n == 0) {  // no visible token: zeros
    if (t < S::DH) {
      if constexpr (S::BF) static_cast<uint16_t*>(out)[out_off + t] = 0;
      else static_cast<float*>(out)[out_off + t] = 0.f;
    }
    return;
  }
  auto block_max = [&](float m) {
    m = r16_max(m);  // DPP inside each 16-lane row, then the rows by permlane swaps
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = __builtin_fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = __builtin_fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  };

  float m_star;
  if (cap <= MS) {
    __syncthreads();
    m_star = block_max(t < n ? tf[t * PP] : -INFINITY);
  } else {
    float m = -INFINITY;
    for (int s = t; s < n; s += 256) m = __builtin_fmaxf(m, base[s * stride]);
    m_star = block_max(m);
  }

  float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
  for (int s0 = 0; s0 < n; s0 += MS) {
    const int cnt = min(MS, n - s0);
    if (cap > MS) {
      __syncthreads();  // previous pass done with tile
      load_pass(s0, cnt);
      __syncthreads();
    }
    if (t < cnt) wts[t] = exp2_fast(tf[t * PP] - m_star);
    __syncthreads();
    if (col >= 0) {
      int s = 0;
      // unrolled: the reads of 16 records go out before the first sum waits on them
#pragma unroll 4
      for (; s + 4 <= cnt; s += 4) {
        v0 = fmaf(wts[s], tf[s * PP + col], v0);
        v1 = fmaf(wts[s + 1], tf[(s + 1) * PP + col], v1);
        v2 = fmaf(wts[s + 2], tf[(s + 2) * PP + col], v2);
        v3 = fmaf(wts[s + 3], tf[(s + 3) * PP + col], v3);
      }
      for (; s < cnt; ++s) v0 = fmaf(wts[s], tf[s * PP + col], v0);
    }
    __syncthreads();  // wts reused by the next pass
  }
  const float v = (v0 + v1) + (v2 + v3);
  if (col == 1) l_s = v;
  else if (t >= S::DH && t < S::DH + S::R) accR_s[t - S::DH] = v;
  __syncthreads();

  if (t < S::DH) {
    float o = v;  // A_S[t]
#pragma unroll
    for (int c = 0; c < BVW; ++c) {
      if constexpr (S::BF) {
        o = fmaf(accR_s[8 * c + 0], bf16_lo(bvr[c].x), o);
        o = fmaf(accR_s[8 * c + 1], bf16_hi(bvr[c].x), o);
        o = fmaf(accR_s[8 * c + 2], bf16_lo(bvr[c].y), o);
        o = fmaf(accR_s[8 * c + 3], bf16_hi(bvr[c].y), o);
        o = fmaf(accR_s[8 * c + 4], bf16_lo(bvr[c].z), o);
        o = fmaf(accR_s[8 * c + 5], bf16_hi(bvr[c].z), o);
        o = fmaf(accR_s[8 * c + 6], bf16_lo(bvr[c].w), o);
        o = fmaf(accR_s[8 * c + 7], bf16_hi(bvr[c].w), o);
      } else {
        o = fmaf(accR_s[4 * c + 0], __uint_as_float(bvr[c].x), o);
        o = fmaf(accR_s[4 * c + 1], __uint_as_float(bvr[c].y), o);
        o = fmaf(accR_s[4 * c + 2], __uint_as_float(bvr[c].z), o);
        o = fmaf(accR_s[4 * c + 3], __uint_as_float(bvr[c].w), o);
      }
    }
    if constexpr (S::BF)
      static_cast<uint16_t*>(out)[out_off + t] = (uint16_t)f32_to_bf16_rne(o / l_s);
    else
      static_cast<float*>(out)[out_off + t] = o / l_s;
  }
}

// ---------------------------------------------------------------------------------------
// Private queries once per query row (eq 6 of the LRKV notes), for lrkv_decode_pq: one
// workgroup per (head, block of query rows), private_query_block (the split kernel's own
// sums, in its order, and its hi + lo packing; B_K[h] read once per workgroup).  A split
// workgroup that reads the block instead of forming it holds bit for bit the same private
// queries.
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(256)
private_queries_kernel(const void* __restrict__ q, const void* __restrict__ BK, int rows,
                       uint4* __restrict__ p_out) {
  // workgroup row blockIdx.y = g: group g of a grouped layout (gridDim.y groups)
  const int g = (int)blockIdx.y, G = (int)gridDim.y;
  private_query_block<S>(q, BK, rows, p_out + (size_t)g * PrivCfg<S>::ROW_SLOTS, blockIdx.x,
                         G * S::H, g * S::H, G * PrivCfg<S>::ROW_SLOTS);
}

// ---------------------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------------------
template <class S>
size_t private_query_row_bytes() {
  return (size_t)PrivCfg<S>::ROW_SLOTS * 16;
}

template <class S>
hipError_t launch_private_queries(const void* q, const void* BK, int rows, void* p, hipStream_t stream,
                                  int groups) {
  static_assert(PrivBlockCfg<S>::NT == 256, "workgroup size");
  hipLaunchKernelGGL((private_queries_kernel<S>), dim3((unsigned)private_query_workgroups<S>(rows), groups),
                     dim3(256), 0, stream, q, BK, rows, static_cast<uint4*>(p));
  return hipGetLastError();
}

template <class S>
SplitArgs split_args(const DecodeArgs& a) {
  SplitArgs s{};
  s.q = a.q;
  s.BK = a.B_K;
  s.pool = static_cast<const uint8_t*>(a.pool);
  s.page_table = a.page_table;
  s.seq_lens = a.seq_lens;
  s.part = a.part_ws;
  s.max_pages = a.max_pages;
  s.q_len = a.q_len;
  s.n_split = a.n_split;
  s.chunk = a.chunk;
  s.batch = a.batch;
  s.groups = a.groups;
  s.score_scale = 1.4426950408889634f / sqrtf((float)S::DH);
  s.page_stride = S::PAGE;
  s.page_off = 0;
  s.q_heads = S::H;
  s.rec_heads = S::H;
  s.head0 = 0;
  return s;
}

template <class S, bool EXTP = false>
void launch_split(const DecodeArgs& a, const SplitArgs& s, int group_rows = 1) {
  if (a.groups > 0)
    hipLaunchKernelGGL((decode_split_kernel<S, true, EXTP>), dim3(a.groups, group_rows),
                       dim3(SplitCfg<S>::NT), 0, a.stream, s);
  else
    hipLaunchKernelGGL((decode_split_kernel<S, false, EXTP>),
                       dim3((a.batch * a.q_len * a.n_split + 7) / 8 * 8, group_rows),
                       dim3(SplitCfg<S>::NT), 0, a.stream, s);
}

template <class S>
hipError_t launch_decode(const DecodeArgs& a) {
  if (a.p_ext) {  // lrkv_decode_pq: private queries formed beforehand (split path only)
    SplitArgs s = split_args<S>(a);
    s.p_ext = static_cast<const uint4*>(a.p_ext);
    s.p_row_slots = PrivCfg<S>::ROW_SLOTS;
    launch_split<S, true>(a, s);
  } else {
    if constexpr (S::BF && !S::NORM) {  // key-norm layouts: every row through the split
      if (a.q_len >= kPrefillMinRows) return launch_prefill<S>(a);
    }
    launch_split<S>(a, split_args<S>(a));
  }
  if (a.groups > 0) {  // balanced split, one query row per request
    hipLaunchKernelGGL((merge_expand_kernel<S, true>), dim3(S::H, 1, a.batch), dim3(256), 0,
                       a.stream, a.part_ws, a.B_V, a.seq_lens, 1, 0, 0, a.batch, a.groups,
                       a.max_pages, a.out);
    return hipGetLastError();
  }
  return launch_merge<S>(a);
}

template <class Sg, class S>
hipError_t launch_decode_grouped(const DecodeArgs& a, int G) {
  static_assert(Sg::DH == S::DH && Sg::R == S::R && Sg::BF == S::BF && !S::NORM, "group blocks");
  {  // every group in one launch: workgroup row g takes group g
    SplitArgs s = split_args<Sg>(a);
    s.page_stride = (long long)G * Sg::PAGE;
    s.q_heads = S::H;
    s.rec_heads = S::H;
    s.group_bk_bytes = (long long)Sg::H * Sg::DH * Sg::R * Sg::EB;
    s.group_page_bytes = Sg::PAGE;
    s.group_heads = Sg::H;
    if (a.p_ext) {  // lrkv_decode_pq: group g's private-query blocks follow group g - 1's
      s.p_ext = static_cast<const uint4*>(a.p_ext);
      s.p_row_slots = G * PrivCfg<Sg>::ROW_SLOTS;
      launch_split<Sg, true>(a, s, G);
    } else {
      launch_split<Sg>(a, s, G);
    }
  }
  if (a.groups > 0) {
    hipLaunchKernelGGL((merge_expand_kernel<S, true>), dim3(S::H, 1, a.batch), dim3(256), 0,
                       a.stream, a.part_ws, a.B_V, a.seq_lens, 1, 0, 0, a.batch, a.groups,
                       a.max_pages, a.out);
    return hipGetLastError();
  }
  return launch_merge<S>(a);
}

template hipError_t launch_decode_grouped<ShapeC3G, ShapeC3>(const DecodeArgs&, int);

template <class S>
hipError_t launch_merge(const DecodeArgs& a) {
  hipLaunchKernelGGL((merge_expand_kernel<S, false>), dim3((a.batch * a.q_len * S::H + 7) / 8 * 8),
                     dim3(256), 0, a.stream, a.part_ws, a.B_V, a.seq_lens, a.q_len, a.n_split,
                     a.chunk, a.batch, 0, a.max_pages, a.out);
  return hipGetLastError();
}

template hipError_t launch_merge<ShapeC1>(const DecodeArgs&);
template hipError_t launch_merge<ShapeC3>(const DecodeArgs&);
template hipError_t launch_merge<ShapeC1N>(const DecodeArgs&);
template hipError_t launch_merge<ShapeC3N>(const DecodeArgs&);

template size_t private_query_row_bytes<ShapeC0>();
template size_t private_query_row_bytes<ShapeC1>();
template size_t private_query_row_bytes<ShapeC3>();
template hipError_t launch_private_queries<ShapeC0>(const void*, const void*, int, void*, hipStream_t, int);
template hipError_t launch_private_queries<ShapeC1>(const void*, const void*, int, void*, hipStream_t, int);
template hipError_t launch_private_queries<ShapeC3>(const void*, const void*, int, void*, hipStream_t, int);
template hipError_t launch_private_queries<ShapeC3G>(const void*, const void*, int, void*, hipStream_t, int);
template size_t private_query_row_bytes<ShapeC3G>();
template hipError_t launch_decode<ShapeC0>(const DecodeArgs&);
template hipError_t launch_decode<ShapeC1>(const DecodeArgs&);
template hipError_t launch_decode<ShapeC3>(const DecodeArgs&);
template hipError_t launch_decode<ShapeC1N>(const DecodeArgs&);
template hipError_t launch_decode<ShapeC3N>(const DecodeArgs&);

}  // namespace lrkv
