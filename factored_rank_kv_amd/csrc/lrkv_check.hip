// Index validation for the LRKV library: counts the device-side index values (request
// lengths, page ids, appended rows' request and position) that lrkv_append and
// lrkv_decode would trust without looking.  Those calls read them on the device and never
// check them (a check there would need a synchronization); a caller who is not sure of
// its tables runs this first, on the same stream.  The rules follow the factored page
// layout of the LRKV notes §3 (one page table for the shared and the private rows, token
// j of request b in page page_table[b][j / P]).
#include "lrkv_launch.h"

namespace lrkv {

namespace {

__global__ void check_zero_kernel(int32_t* errors) {
  if (threadIdx.x == 0) errors[0] = 0;
}

// Work item i: i < batch checks a length; then batch * max_pages page-table entries (each
// checked if a valid length of its request covers it); then n_rows appended rows.
__global__ void __launch_bounds__(256)
check_kernel(const CheckArgs a, long long items) {
  int bad = 0;
  const long long entries = (long long)a.batch * a.max_pages;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += stride) {
    if (a.seq_lens && i < a.batch) {
      const int s = a.seq_lens[i];
      bad += s < 0 || s > a.max_seq_len;
    } else if (a.seq_lens && i < a.batch + entries) {
      const long long e = i - a.batch;
      const int b = (int)(e / a.max_pages), p = (int)(e % a.max_pages);
      const int s = a.seq_lens[b];
      if (s >= 0 && s <= a.max_seq_len && (long long)p * a.page_size < s) {
        const int id = a.page_table[e];
        bad += id < 0 || id >= a.num_pages;
      }
    } else if (a.row_req) {
      const long long n = i - (a.seq_lens ? a.batch + entries : 0);
      const int req = a.row_req[n], pos = a.row_pos[n];
      if (req < 0 || req >= a.batch || pos < 0 || pos >= a.max_pages * a.page_size) {
        ++bad;
      } else {
        const int id = a.page_table[(long long)req * a.max_pages + pos / a.page_size];
        bad += id < 0 || id >= a.num_pages;
      }
    }
  }
  // block sum, then one atomic add per block that found something
  __shared__ int red[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bad += __shfl_xor(bad, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int total = red[0] + red[1] + red[2] + red[3];
    if (total) atomicAdd(a.errors, total);
  }
}

}  // namespace

hipError_t launch_check(const CheckArgs& a) {
  const long long entries = (long long)a.batch * a.max_pages;
  const long long items = (a.seq_lens ? a.batch + entries : 0) + (a.row_req ? a.n_rows : 0);
  hipLaunchKernelGGL(check_zero_kernel, dim3(1), dim3(64), 0, a.stream, a.errors);
  if (items > 0) {
    const long long want = (items + 255) / 256;
    const int blocks = (int)(want < 2048 ? want : 2048);
    hipLaunchKernelGGL(check_kernel, dim3(blocks), dim3(256), 0, a.stream, a, items);
  }
  return hipGetLastError();
}

}  // namespace lrkv
