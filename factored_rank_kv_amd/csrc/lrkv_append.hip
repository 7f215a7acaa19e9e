// LRKV append (Algorithm 1 of the LRKV notes, §3): project new rows into the shared and
// per-head private coordinates and scatter them into their pages.
//
// The projection is one product X [n x d] . [W_SK | W_SV | U_K | U_V] [d x N] with
// N = 2 d_h + 2 H r columns; column c of the product is written, rounded to nearest even,
// at the row's (page, slot) in the section that column belongs to.
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

template <class S>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (S::BF) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Workgroup = 256 output columns x ROWS rows; each thread owns one column for ROWS rows and
// runs the dot products over d in float32.
template <class S, int ROWS>
__global__ void __launch_bounds__(256)
append_rows_kernel(AppendArgs a) {
  constexpr int N = 2 * S::DH + 2 * S::H * S::R;
  const int col = blockIdx.x * 256 + threadIdx.x;
  const int n0 = blockIdx.y * ROWS;
  if (col >= N) return;
  const void* W;
  int ldw, wc;
  if (col < S::DH) {
    W = a.W_SK; ldw = S::DH; wc = col;
  } else if (col < 2 * S::DH) {
    W = a.W_SV; ldw = S::DH; wc = col - S::DH;
  } else if (col < 2 * S::DH + S::H * S::R) {
    W = a.U_K; ldw = S::H * S::R; wc = col - 2 * S::DH;
  } else {
    W = a.U_V; ldw = S::H * S::R; wc = col - 2 * S::DH - S::H * S::R;
  }
  const int nr = min(ROWS, a.n_rows - n0);
  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.f;
  for (int k = 0; k < a.d; ++k) {
    const float w = load_elem<S>(W, (size_t)k * ldw + wc);
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      if (r < nr) acc[r] = fmaf(load_elem<S>(a.X, (size_t)(n0 + r) * a.d + k), w, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (r >= nr) break;
    const int n = n0 + r;
    const int req = a.row_req[n];
    const int pos = a.row_pos[n];
    const int page = a.page_table[(size_t)req * a.max_pages + pos / S::P];
    const size_t e = (size_t)page * (S::PAGE / S::EB) + append_dest<S>(col, pos % S::P);
    if constexpr (S::BF) static_cast<uint16_t*>(a.pool)[e] = (uint16_t)f32_to_bf16_rne(acc[r]);
    else static_cast<float*>(a.pool)[e] = acc[r];
  }
}

template <class S>
hipError_t launch_append(const AppendArgs& a) {
  constexpr int N = 2 * S::DH + 2 * S::H * S::R;
  constexpr int ROWS = 8;
  dim3 grid((N + 255) / 256, (a.n_rows + ROWS - 1) / ROWS);
  hipLaunchKernelGGL((append_rows_kernel<S, ROWS>), grid, dim3(256), 0, a.stream, a);
  return hipGetLastError();
}

template hipError_t launch_append<ShapeC0>(const AppendArgs&);
template hipError_t launch_append<ShapeC1>(const AppendArgs&);
template hipError_t launch_append<ShapeC3>(const AppendArgs&);

}  // namespace lrkv
