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
// product columns (8 bf16 / 4 f32) x up to 8 rows; 256 threads = 8 rows x 32 k-lanes.
// Reading the weights once dominates, so the grid has one workgroup per chunk; chunks that
// share a 128-byte line are given to blocks on the same XCD (blocks go to XCDs round robin).
// bf16: pairs of k go through v_dot2_f32_bf16 (products exact, float32 sums); v_perm_b32
// packs (W[k][c], W[k+1][c]) from two weight rows.
// ---------------------------------------------------------------------------------------
template <class S>
__global__ void __launch_bounds__(256)
append_few_rows_kernel(AppendArgs a, int n_chunks) {
  constexpr int CE = S::CE;
  constexpr int KS = S::BF ? 2 : 1;  // k values per step
  __shared__ float red[4][8][CE];
  const int bx = blockIdx.x;
  const int chunk = (n_chunks % 8 == 0) ? (bx % 8) * (n_chunks / 8) + bx / 8 : bx;
  const int col0 = chunk * CE;
  int ldw, wc;
  const uint8_t* W = weight_column<S>(a, col0, ldw, wc);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int n = t & 7;
  const int kl = t >> 3;  // 0..31
  const int row = blockIdx.y * 8 + n;
  const bool active = row < a.n_rows;

  float acc[CE];
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  if (active) {
    const size_t wrow = (size_t)ldw * S::EB;  // bytes per weight row
    const uint8_t* wcol = W + (size_t)wc * S::EB;
    if constexpr (S::BF) {
      const uint32_t* xr = reinterpret_cast<const uint32_t*>(
          static_cast<const uint16_t*>(a.X) + (size_t)row * a.d);
#pragma unroll 4
      for (int k = kl * KS; k < a.d; k += 32 * KS) {
        const uint4 w0 = *reinterpret_cast<const uint4*>(wcol + (size_t)k * wrow);
        const uint4 w1 = *reinterpret_cast<const uint4*>(wcol + (size_t)(k + 1) * wrow);
        const uint32_t x = xr[k >> 1];
        const uint32_t a0[4] = {w0.x, w0.y, w0.z, w0.w};
        const uint32_t a1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);  // col 2e
          const uint32_t hi = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);  // col 2e+1
          acc[2 * e] = dot2_bf16(x, lo, acc[2 * e]);
          acc[2 * e + 1] = dot2_bf16(x, hi, acc[2 * e + 1]);
        }
      }
    } else {
      const float* xr = static_cast<const float*>(a.X) + (size_t)row * a.d;
#pragma unroll 4
      for (int k = kl; k < a.d; k += 32) {
        const float4 w = *reinterpret_cast<const float4*>(wcol + (size_t)k * wrow);
        const float x = xr[k];
        acc[0] = fmaf(x, w.x, acc[0]);
        acc[1] = fmaf(x, w.y, acc[1]);
        acc[2] = fmaf(x, w.z, acc[2]);
        acc[3] = fmaf(x, w.w, acc[3]);
      }
    }
  }
  // sum over the 32 k-lanes: 8 per wavefront (lane bits 3..5), then 4 wavefronts
#pragma unroll
  for (int e = 0; e < CE; ++e) {
    acc[e] += __shfl_xor(acc[e], 8);
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < CE; ++e) red[wave][n][e] = acc[e];
  }
  __syncthreads();
  if (t < 8 * CE) {
    const int rn = t / CE, e = t % CE;
    const int r = blockIdx.y * 8 + rn;
    if (r < a.n_rows) {
      const float v = (red[0][rn][e] + red[1][rn][e]) + (red[2][rn][e] + red[3][rn][e]);
      const int req = a.row_req[r];
      const int pos = a.row_pos[r];
      const int page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
      store_elem<S>(a.pool, (size_t)page * (S::PAGE / S::EB) + append_dest<S>(col0 + e, pos % S::P),
                    v);
    }
  }
}

template <class S>
hipError_t launch_append(const AppendArgs& a) {
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
