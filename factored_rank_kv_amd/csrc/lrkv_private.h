// Private queries p = q B_K[h] (LRKV notes §2: the query carried into each head's rank-r
// space), their block layout and one formation job per thread, shared by the split decode,
// the stand-alone formation kernel and the append launch that forms them beside the new
// rows (gfx950 only).
#pragma once

#include "lrkv_device.h"

namespace lrkv {

// Geometry of the split decode workgroup that the block layout follows, and of the sums.
template <class S>
struct PrivCfg {
  static constexpr int HPW = S::H <= 4 ? 4 : (S::H / 8 > 2 ? S::H / 8 : 2);  // heads per wave
  static constexpr int SPLIT = 4 / HPW;        // lanes per (head, token) pair
  static constexpr int NT = (S::H / HPW) * 64;  // threads of a split workgroup
  static constexpr int RC_L = (S::RC + SPLIT - 1) / SPLIT;  // private chunks per lane
  static constexpr int P_PER_CHUNK = S::BF ? 2 : 1;  // uint4 per chunk (bf16: hi, lo)
  // uint4 slots per head: room for SPLIT*RC_L chunks, the slots past RC hold zeros (a lane
  // whose half runs past the last chunk adds nothing for it); the odd count spreads a
  // wavefront's heads over different LDS banks
  static constexpr int P_STRIDE = (SPLIT * RC_L * P_PER_CHUNK) | 1;
  static constexpr int PAD = P_STRIDE - S::RC * P_PER_CHUNK;  // zero slots per head
  static constexpr int ROW_SLOTS = S::H * P_STRIDE;            // uint4 of a row's block
  // one job per (head, 16-byte chunk of p); d_h cut into PQ_GROUPS spans summed apart
  static constexpr int PQ_JOBS = S::H * S::RC;
  static constexpr int PQ_GROUPS = NT / PQ_JOBS > 0 ? NT / PQ_JOBS : 1;
  static constexpr int PQ_DSPAN = S::DH / PQ_GROUPS;
  static_assert(S::DH % PQ_GROUPS == 0, "d_h split evenly");
};

// Packs one 8-value (bf16) or 4-value (float32) chunk of p into its slots: bf16 as 4 words
// of bfloat16 pairs of hi(p) then 4 words of lo(p) = bf16(p - hi(p)), so that
// p.R_K[h,j] = dot2(hi, r) + dot2(lo, r) keeps about 16 significant bits of p; float32 as
// it is.
template <class S>
__device__ __forceinline__ void store_private_chunk(uint4* __restrict__ dst, const float* p) {
  if constexpr (S::BF) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h0 = f32_to_bf16_rne(p[2 * e]), h1 = f32_to_bf16_rne(p[2 * e + 1]);
      hi[e] = h0 | (h1 << 16);
      lo[e] = f32_to_bf16_rne(p[2 * e] - bf16_to_f32((uint16_t)h0)) |
              (f32_to_bf16_rne(p[2 * e + 1] - bf16_to_f32((uint16_t)h1)) << 16);
    }
    dst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    dst[1] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  } else {
    dst[0] = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]),
                        __float_as_uint(p[3]));
  }
}

// Workgroup form of the formation: workgroup blk takes head h = blk % H for a block of
// PQ_ROWS_WG query rows (rows (blk / H) PQ_ROWS_WG, ...), 256 threads.  B_K[h] is read from
// memory once per workgroup, in whole 16-byte chunks, into LDS, with the block's query rows
// of head h; thread t then holds job (row, chunk c) and span g = t % PQ_GROUPS.  The span's
// partial sum over d in [g DSPAN, (g+1) DSPAN) is one fused multiply-add chain from zero,
// and the spans are added in order g = 0, 1, ... to a zero start: the same float32
// arithmetic, in the same order, as the split decode's own formation, so either gives the
// same bits.  The PQ_GROUPS threads of a job sit in one wavefront (PQ_GROUPS divides 64).
// q: [rows][q_heads][d_h], heads head0 .. head0 + H - 1 taken; BK: [..][d_h][r] from head
// head0; p_out: a row's block of ROW_SLOTS uint4 every row_slots, every slot written (the
// pad slots zero).  (A grouped layout forms group g's blocks with head0 = g H and
// row_slots = G ROW_SLOTS, p_out advanced by g ROW_SLOTS.)  Every thread of the workgroup
// must make the call.
template <class S>
struct PrivBlockCfg {
  using C = PrivCfg<S>;
  static constexpr int NT = 256;
  static constexpr int JOB_THREADS = S::RC * C::PQ_GROUPS;  // threads per (row, head)
  static constexpr int ROWS_WG = NT / JOB_THREADS;          // query rows per workgroup
  // B_K[h] in LDS, span g's rows after g spans of DSPAN + 1 rows: the extra row of chunks
  // shifts each span by RC 16-byte slots, so the 4 spans' reads of one row spread over the
  // banks
  static constexpr int BK_SLOTS = C::PQ_GROUPS * (C::PQ_DSPAN + 1) * S::RC;
  static_assert(ROWS_WG >= 1, "one row's jobs fit a workgroup");
};

template <class S>
__host__ __device__ constexpr long long private_query_workgroups(long long rows) {
  return (long long)S::H * ((rows + PrivBlockCfg<S>::ROWS_WG - 1) / PrivBlockCfg<S>::ROWS_WG);
}

template <class S>
__device__ __forceinline__ void private_query_block(const void* __restrict__ q,
                                                    const void* __restrict__ BK, int rows,
                                                    uint4* __restrict__ p_out, long long blk,
                                                    int q_heads = S::H, int head0 = 0,
                                                    int row_slots = PrivCfg<S>::ROW_SLOTS) {
  using C = PrivCfg<S>;
  using W = PrivBlockCfg<S>;
  static_assert(64 % C::PQ_GROUPS == 0 && C::PQ_GROUPS >= 2, "a job's spans in one wavefront");
  static_assert(C::PAD <= C::PQ_GROUPS - 1, "the pad slots fit the spans past the first");
  __shared__ uint4 bk_lds[W::BK_SLOTS];
  __shared__ uint4 q_lds[W::ROWS_WG * S::DHC];
  const int t = (int)threadIdx.x;
  const int h = (int)(blk % S::H);
  const long long row0 = (blk / S::H) * W::ROWS_WG;
  // B_K[h] (d_h rows of RC chunks, contiguous) and the block's query rows of head h: every
  // load of the thread goes out before its first LDS write (as a loop, each load was
  // waited for before the next went out)
  constexpr int BKN = S::DH * S::RC, BKI = (BKN + W::NT - 1) / W::NT;
  constexpr int QN = W::ROWS_WG * S::DHC, QI = (QN + W::NT - 1) / W::NT;
  const uint4* bkg = reinterpret_cast<const uint4*>(BK) + (size_t)(head0 + h) * S::DH * S::RC;
  uint4 bkv[BKI], qvv[QI];
#pragma unroll
  for (int k = 0; k < BKI; ++k) {
    const int e = min(t + k * W::NT, BKN - 1);  // lanes past the end re-read the last chunk
    bkv[k] = bkg[e];
  }
#pragma unroll
  for (int k = 0; k < QI; ++k) {
    const int e = min(t + k * W::NT, QN - 1);
    const int rl = e / S::DHC, kk = e - rl * S::DHC;
    const long long row = row0 + rl < rows ? row0 + rl : rows - 1;  // past the end: a valid row
    qvv[k] = reinterpret_cast<const uint4*>(q)[((size_t)row * q_heads + head0 + h) * S::DHC + kk];
  }
  // (an empty statement taking each value keeps the loads from sinking into the
  // conditional stores below, one round trip each)
#pragma unroll
  for (int k = 0; k < BKI; ++k) asm volatile("" ::"v"(bkv[k].x), "v"(bkv[k].y), "v"(bkv[k].z), "v"(bkv[k].w));
#pragma unroll
  for (int k = 0; k < QI; ++k) asm volatile("" ::"v"(qvv[k].x), "v"(qvv[k].y), "v"(qvv[k].z), "v"(qvv[k].w));
#pragma unroll
  for (int k = 0; k < BKI; ++k) {
    const int e = t + k * W::NT;
    if (e < BKN) {
      const int d = e / S::RC, c = e - d * S::RC;
      const int g = d / C::PQ_DSPAN, dd = d - g * C::PQ_DSPAN;
      bk_lds[(g * (C::PQ_DSPAN + 1) + dd) * S::RC + c] = bkv[k];
    }
  }
#pragma unroll
  for (int k = 0; k < QI; ++k)
    if (t + k * W::NT < QN) q_lds[t + k * W::NT] = qvv[k];
  __syncthreads();
  const int g = t % C::PQ_GROUPS;
  const int c = (t / C::PQ_GROUPS) % S::RC;
  const int rl = min(t / W::JOB_THREADS, W::ROWS_WG - 1);  // threads past the jobs: idle
  const uint8_t* qs = reinterpret_cast<const uint8_t*>(q_lds + rl * S::DHC) +
                      (size_t)g * C::PQ_DSPAN * S::EB;
  const uint4* bks = bk_lds + g * (C::PQ_DSPAN + 1) * S::RC + c;
  // the chain's operands in registers, every LDS read before the first product (left to
  // the scheduler, each read waited for right before its product)
  constexpr int QV = (C::PQ_DSPAN * S::EB) % 16 == 0 ? C::PQ_DSPAN * S::EB / 16 : 0;
  uint4 qv[QV > 0 ? QV : 1];
  float qsc[QV > 0 ? 1 : C::PQ_DSPAN];
  if constexpr (QV > 0) {
#pragma unroll
    for (int k = 0; k < QV; ++k) qv[k] = reinterpret_cast<const uint4*>(qs)[k];
  } else {
#pragma unroll
    for (int dd = 0; dd < C::PQ_DSPAN; ++dd)
      qsc[dd] = S::BF ? bf16_to_f32(reinterpret_cast<const uint16_t*>(qs)[dd])
                      : reinterpret_cast<const float*>(qs)[dd];
  }
  uint4 b4[C::PQ_DSPAN];
#pragma unroll
  for (int dd = 0; dd < C::PQ_DSPAN; ++dd) b4[dd] = bks[dd * S::RC];
#pragma unroll
  for (int dd = 0; dd < C::PQ_DSPAN; ++dd)
    asm volatile("" ::"v"(b4[dd].x), "v"(b4[dd].y), "v"(b4[dd].z), "v"(b4[dd].w));
  float acc[S::CE];
#pragma unroll
  for (int e = 0; e < S::CE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int dd = 0; dd < C::PQ_DSPAN; ++dd) {
    float qd;
    if constexpr (QV > 0) {
      const uint4 w4 = qv[dd * S::EB / 16];
      const int wi = (dd * S::EB / 4) % 4;
      const uint32_t w = wi == 0 ? w4.x : wi == 1 ? w4.y : wi == 2 ? w4.z : w4.w;
      if constexpr (S::BF)
        qd = (dd & 1) ? bf16_hi(w) : bf16_lo(w);
      else
        qd = __uint_as_float(w);
    } else {
      qd = qsc[dd];
    }
    const uint4 b = b4[dd];
    if constexpr (S::BF) {
      acc[0] = fmaf(qd, bf16_lo(b.x), acc[0]);
      acc[1] = fmaf(qd, bf16_hi(b.x), acc[1]);
      acc[2] = fmaf(qd, bf16_lo(b.y), acc[2]);
      acc[3] = fmaf(qd, bf16_hi(b.y), acc[3]);
      acc[4] = fmaf(qd, bf16_lo(b.z), acc[4]);
      acc[5] = fmaf(qd, bf16_hi(b.z), acc[5]);
      acc[6] = fmaf(qd, bf16_lo(b.w), acc[6]);
      acc[7] = fmaf(qd, bf16_hi(b.w), acc[7]);
    } else {
      acc[0] = fmaf(qd, __uint_as_float(b.x), acc[0]);
      acc[1] = fmaf(qd, __uint_as_float(b.y), acc[1]);
      acc[2] = fmaf(qd, __uint_as_float(b.z), acc[2]);
      acc[3] = fmaf(qd, __uint_as_float(b.w), acc[3]);
    }
  }
  // the job's first lane adds the spans in order
  const int lane = t & 63;
  const int first = lane - g;
  float p[S::CE];
#pragma unroll
  for (int e = 0; e < S::CE; ++e) {
    float v = 0.f;
#pragma unroll
    for (int gg = 0; gg < C::PQ_GROUPS; ++gg) v += __shfl(acc[e], first + gg, 64);
    p[e] = v;
  }
  const long long row = row0 + t / W::JOB_THREADS;
  if (t >= W::ROWS_WG * W::JOB_THREADS || row >= rows) return;
  uint4* dst = p_out + (size_t)row * row_slots + (size_t)h * C::P_STRIDE;
  if (g == 0) store_private_chunk<S>(dst + c * C::P_PER_CHUNK, p);
  if (c == 0 && g >= 1 && g <= C::PAD)
    dst[S::RC * C::P_PER_CHUNK + g - 1] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace lrkv
