// LRKV decode kernels for gfx950: Algorithm 2 of the LRKV notes (§3) read from the
// factored paged cache, as three launches on the caller's stream:
//   1. private_query_kernel  p = q B_K[h], once per (request, query row, head)   (eq 6)
//   2. decode_split_kernel   one workgroup per (request, query row, chunk of pages), all
//                            heads: shared S_K/S_V tiles staged once in LDS for every head,
//                            private R_K/R_V rows streamed per head, one online softmax with
//                            a shared and a private value accumulator (the fused blockwise
//                            paragraph after Algorithm 2), partial tuples written out
//   3. merge_expand_kernel   merge the chunks' (max, exp-sum, acc_S, acc_R) tuples with one
//                            rescale factor per chunk, expand acc_R through B_V[h]^T once,
//                            divide by the exp-sum (Algorithm 2 steps 08-09 without W_O)
#include "lrkv_device.h"
#include "lrkv_launch.h"

namespace lrkv {

// ---------------------------------------------------------------------------------------
// 1. private query
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(1024)
private_query_kernel(const void* __restrict__ q, const void* __restrict__ BK,
                     float* __restrict__ p) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  if (t >= S::H * S::R) return;
  const int h = t / S::R;
  const int k = t - h * S::R;
  float acc = 0.f;
  if constexpr (S::BF) {
    const uint16_t* qh = static_cast<const uint16_t*>(q) + ((size_t)row * S::H + h) * S::DH;
    const uint16_t* bk = static_cast<const uint16_t*>(BK) + (size_t)h * S::DH * S::R + k;
#pragma unroll 8
    for (int d = 0; d < S::DH; ++d) acc = fmaf(bf16_to_f32(qh[d]), bf16_to_f32(bk[d * S::R]), acc);
  } else {
    const float* qh = static_cast<const float*>(q) + ((size_t)row * S::H + h) * S::DH;
    const float* bk = static_cast<const float*>(BK) + (size_t)h * S::DH * S::R + k;
#pragma unroll 8
    for (int d = 0; d < S::DH; ++d) acc = fmaf(qh[d], bk[d * S::R], acc);
  }
  p[((size_t)row * S::H + h) * S::R + k] = acc;
}

// ---------------------------------------------------------------------------------------
// 2. split kernel
//
// Workgroup = (chunk, query row i, request b); H/4 wavefronts; lane = 16*hl + j handles
// head h = 4*wave + hl and token slot j of the current page for the score, the softmax and
// the private value accumulator.  For the shared value accumulator the same wavefront
// switches to lanes over feature pairs (dims 2*lane, 2*lane+1) for its four heads.
//
// Scores are kept in base-2 units: s = (q.S_K + p.R_K) * log2(e) / sqrt(d_h), so the
// softmax uses exp2; the merge uses the same units.
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(S::H * 16)
decode_split_kernel(const void* __restrict__ q, const float* __restrict__ p,
                    const uint8_t* __restrict__ pool, const int32_t* __restrict__ page_table,
                    int max_pages, const int32_t* __restrict__ seq_lens, int q_len, int n_split,
                    int chunk, float* __restrict__ part, float score_scale) {
  constexpr int NT = S::H * 16;
  __shared__ uint4 sk_lds[S::DHC * S::P];  // chunk-major [c][t], as in the page
  __shared__ uint4 sv_lds[S::P * S::DHC];  // row-major [t][c]: row t is S_V[t][0..DH)

  const int split = blockIdx.x;
  const int qi = blockIdx.y;
  const int b = blockIdx.z;
  const int T = seq_lens[b];
  const int vis = visible_tokens(T, q_len, qi);
  const int tok0 = split * chunk;
  const int tok1 = min(vis, tok0 + chunk);
  if (tok0 >= tok1) return;  // uniform for the whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 4;
  const int j = lane & 15;
  const int h = wave * 4 + hl;
  const size_t row = (size_t)b * q_len + qi;

  // query of head h: DH elements as 32-bit words (bf16 pairs or floats)
  constexpr int QW = S::DH * S::EB / 4;
  uint32_t qv[QW];
  {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q) +
                                                      (row * S::H + h) * S::DH * S::EB);
#pragma unroll
    for (int c = 0; c < S::DHC; ++c) {
      const uint4 v = src[c];
      qv[4 * c + 0] = v.x;
      qv[4 * c + 1] = v.y;
      qv[4 * c + 2] = v.z;
      qv[4 * c + 3] = v.w;
    }
  }
  // private query of head h.  bf16 cache: split each float32 p into hi + lo bfloat16 parts
  // so the private dot product runs on v_dot2_f32_bf16 with ~16 significant bits of p.
  constexpr int PW = S::BF ? S::R / 2 : S::R;
  uint32_t phi[PW];
  uint32_t plo[S::BF ? PW : 1];
  {
    const float* ph = p + (row * S::H + h) * S::R;
    if constexpr (S::BF) {
#pragma unroll
      for (int k2 = 0; k2 < PW; ++k2) {
        const float a = ph[2 * k2], c = ph[2 * k2 + 1];
        const uint32_t ah = f32_to_bf16_rne(a), ch = f32_to_bf16_rne(c);
        phi[k2] = ah | (ch << 16);
        plo[k2] = f32_to_bf16_rne(a - bf16_to_f32((uint16_t)ah)) |
                  (f32_to_bf16_rne(c - bf16_to_f32((uint16_t)ch)) << 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < S::R; ++k) phi[k] = __float_as_uint(ph[k]);
    }
  }

  float m_run = -INFINITY;  // running max (same in the 16 lanes of a head)
  float l_run = 0.f;        // this lane's share of the exp-sum
  float accR[S::R];         // this lane's share of sum_j w_j R_V[h, j]
#pragma unroll
  for (int k = 0; k < S::R; ++k) accR[k] = 0.f;
  float accS[4][2];  // sum_j w_j S_V[j][2*lane + e] for the wavefront's four heads
#pragma unroll
  for (int x = 0; x < 4; ++x) accS[x][0] = accS[x][1] = 0.f;
  const int dl = (2 * lane < S::DH) ? lane : (S::DH / 2 - 1);  // feature pair of this lane

  const int32_t* tab = page_table + (size_t)b * max_pages;
  const int pg0 = tok0 / S::P;
  const int pg1 = (tok1 + S::P - 1) / S::P;
  for (int pg = pg0; pg < pg1; ++pg) {
    const uint8_t* page = pool + (size_t)tab[pg] * S::PAGE;
    const int nvalid = min(S::P, tok1 - pg * S::P);

    __syncthreads();  // the previous page's LDS tiles are no longer read
    for (int c = tid; c < 2 * S::DHC * S::P; c += NT) {
      const uint4 v = reinterpret_cast<const uint4*>(page)[c];
      if (c < S::DHC * S::P) {
        sk_lds[c] = v;
      } else {
        const int cc = c - S::DHC * S::P;
        sv_lds[(cc % S::P) * S::DHC + cc / S::P] = v;
      }
    }
    uint4 rk[S::RC], rv[S::RC];
    {
      const uint4* rkp = reinterpret_cast<const uint4*>(page + S::OFF_RK + h * S::SEC_R) + j;
      const uint4* rvp = reinterpret_cast<const uint4*>(page + S::OFF_RV + h * S::SEC_R) + j;
#pragma unroll
      for (int c = 0; c < S::RC; ++c) {
        rk[c] = rkp[c * S::P];
        rv[c] = rvp[c * S::P];
      }
    }
    __syncthreads();

    const bool valid = j < nvalid;
    // ---- score: q . S_K[j] + p . R_K[h, j]  (eq 6)
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < S::DHC; ++c) {
      const uint4 s4 = sk_lds[c * S::P + j];
      if constexpr (S::BF) {
        acc = dot2_bf16(qv[4 * c + 0], s4.x, acc);
        acc = dot2_bf16(qv[4 * c + 1], s4.y, acc);
        acc = dot2_bf16(qv[4 * c + 2], s4.z, acc);
        acc = dot2_bf16(qv[4 * c + 3], s4.w, acc);
      } else {
        acc = fmaf(__uint_as_float(qv[4 * c + 0]), __uint_as_float(s4.x), acc);
        acc = fmaf(__uint_as_float(qv[4 * c + 1]), __uint_as_float(s4.y), acc);
        acc = fmaf(__uint_as_float(qv[4 * c + 2]), __uint_as_float(s4.z), acc);
        acc = fmaf(__uint_as_float(qv[4 * c + 3]), __uint_as_float(s4.w), acc);
      }
    }
#pragma unroll
    for (int c = 0; c < S::RC; ++c) {
      const uint32_t r4[4] = {rk[c].x, rk[c].y, rk[c].z, rk[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (S::BF) {
          acc = dot2_bf16(phi[4 * c + e], r4[e], acc);
          acc = dot2_bf16(plo[4 * c + e], r4[e], acc);
        } else {
          acc = fmaf(__uint_as_float(phi[4 * c + e]), __uint_as_float(r4[e]), acc);
        }
      }
    }
    // masked slots are removed by selection, never multiplied by zero
    const float s = valid ? acc * score_scale : -INFINITY;

    // ---- online softmax, one factor rescales exp-sum and both accumulators
    const float m_new = fmaxf(m_run, row16_max(s));
    const float alpha = exp2f(m_run - m_new);
    const float w = exp2f(s - m_new);
    l_run = l_run * alpha + w;
    if (!valid) {
#pragma unroll
      for (int c = 0; c < S::RC; ++c) rv[c] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < S::RC; ++c) {
      const uint32_t r4[4] = {rv[c].x, rv[c].y, rv[c].z, rv[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (S::BF) {
          const int k = 8 * c + 2 * e;
          accR[k] = fmaf(w, bf16_lo(r4[e]), accR[k] * alpha);
          accR[k + 1] = fmaf(w, bf16_hi(r4[e]), accR[k + 1] * alpha);
        } else {
          const int k = 4 * c + e;
          accR[k] = fmaf(w, __uint_as_float(r4[e]), accR[k] * alpha);
        }
      }
    }
    m_run = m_new;

    // ---- shared value accumulator: lanes over feature pairs, weights broadcast by readlane
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float a = readlane_f(alpha, 16 * x);
      accS[x][0] *= a;
      accS[x][1] *= a;
    }
    for (int t = 0; t < nvalid; ++t) {
      float sv0, sv1;
      if constexpr (S::BF) {
        const uint32_t pr = reinterpret_cast<const uint32_t*>(sv_lds)[t * (S::DH / 2) + dl];
        sv0 = bf16_lo(pr);
        sv1 = bf16_hi(pr);
      } else {
        const float2 pr = reinterpret_cast<const float2*>(sv_lds)[t * (S::DH / 2) + dl];
        sv0 = pr.x;
        sv1 = pr.y;
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float wt = readlane_f(w, 16 * x + t);
        accS[x][0] = fmaf(wt, sv0, accS[x][0]);
        accS[x][1] = fmaf(wt, sv1, accS[x][1]);
      }
    }
  }

  // ---- partial tuple of this chunk: m, l, acc_S[DH], acc_R[R] per head
  const float l_tot = row16_sum(l_run);
#pragma unroll
  for (int k = 0; k < S::R; ++k) accR[k] = row16_sum(accR[k]);
  float* dst = part + ((row * n_split + split) * S::H + h) * S::PART;
  if (j == 0) {
    dst[0] = m_run;
    dst[1] = l_tot;
  }
#pragma unroll
  for (int k = 0; k < S::R; ++k)
    if ((k & 15) == j) dst[2 + S::DH + k] = accR[k];
  if (2 * lane < S::DH) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      float* d2 = part + ((row * n_split + split) * S::H + 4 * wave + x) * S::PART + 2 + 2 * lane;
      d2[0] = accS[x][0];
      d2[1] = accS[x][1];
    }
  }
}

// ---------------------------------------------------------------------------------------
// 3. merge + expand
// Workgroup = (head, query row, request); thread t owns column 1 + t of the partial tuple
// (l, acc_S[DH], acc_R[R]) and sums it over the chunks with weights exp2(m_s - m*).
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(256)
merge_expand_kernel(const float* __restrict__ part, const void* __restrict__ BV,
                    const int32_t* __restrict__ seq_lens, int q_len, int n_split, int chunk,
                    void* __restrict__ out) {
  static_assert(1 + S::DH + S::R <= 256, "one thread per column");
  __shared__ float accR_s[S::R];
  __shared__ float l_s;
  const int h = blockIdx.x;
  const int qi = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const size_t row = (size_t)b * q_len + qi;
  const int vis = visible_tokens(seq_lens[b], q_len, qi);
  const int n = (vis + chunk - 1) / chunk;
  const size_t out_off = (row * S::H + h) * S::DH;

  if (n == 0) {  // no visible token: zeros
    if (t < S::DH) {
      if constexpr (S::BF) static_cast<uint16_t*>(out)[out_off + t] = 0;
      else static_cast<float*>(out)[out_off + t] = 0.f;
    }
    return;
  }
  const float* base = part + (row * n_split * S::H + h) * S::PART;
  const size_t stride = (size_t)S::H * S::PART;  // next chunk, same head
  float m_star = -INFINITY;
  for (int s = 0; s < n; ++s) m_star = fmaxf(m_star, base[s * stride]);
  const int col = 1 + t;
  float v = 0.f;
  if (col < S::PART) {
    for (int s = 0; s < n; ++s) v = fmaf(exp2f(base[s * stride] - m_star), base[s * stride + col], v);
    if (col == 1) l_s = v;
    else if (col >= 2 + S::DH) accR_s[col - 2 - S::DH] = v;
  }
  __syncthreads();
  if (col >= 2 && col < 2 + S::DH) {
    const int d = col - 2;
    float o = v;  // acc_S[d]
    if constexpr (S::BF) {
      const uint16_t* bv = static_cast<const uint16_t*>(BV) + ((size_t)h * S::DH + d) * S::R;
#pragma unroll 8
      for (int k = 0; k < S::R; ++k) o = fmaf(accR_s[k], bf16_to_f32(bv[k]), o);
      static_cast<uint16_t*>(out)[out_off + d] = (uint16_t)f32_to_bf16_rne(o / l_s);
    } else {
      const float* bv = static_cast<const float*>(BV) + ((size_t)h * S::DH + d) * S::R;
#pragma unroll 4
      for (int k = 0; k < S::R; ++k) o = fmaf(accR_s[k], bv[k], o);
      static_cast<float*>(out)[out_off + d] = o / l_s;
    }
  }
}

// ---------------------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------------------
template <class S>
hipError_t launch_decode(const DecodeArgs& a) {
  const int rows = a.batch * a.q_len;
  const int pq_threads = ((S::H * S::R + 63) / 64) * 64;
  hipLaunchKernelGGL(private_query_kernel<S>, dim3(rows), dim3(pq_threads), 0, a.stream, a.q,
                     a.B_K, a.p_ws);
  const float score_scale = 1.4426950408889634f / sqrtf((float)S::DH);
  hipLaunchKernelGGL(decode_split_kernel<S>, dim3(a.n_split, a.q_len, a.batch), dim3(S::H * 16),
                     0, a.stream, a.q, a.p_ws, static_cast<const uint8_t*>(a.pool), a.page_table,
                     a.max_pages, a.seq_lens, a.q_len, a.n_split, a.chunk, a.part_ws, score_scale);
  hipLaunchKernelGGL(merge_expand_kernel<S>, dim3(S::H, a.q_len, a.batch), dim3(256), 0, a.stream,
                     a.part_ws, a.B_V, a.seq_lens, a.q_len, a.n_split, a.chunk, a.out);
  return hipGetLastError();
}

template hipError_t launch_decode<ShapeC0>(const DecodeArgs&);
template hipError_t launch_decode<ShapeC1>(const DecodeArgs&);
template hipError_t launch_decode<ShapeC3>(const DecodeArgs&);

}  // namespace lrkv
