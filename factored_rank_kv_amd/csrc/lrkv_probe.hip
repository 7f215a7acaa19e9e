// Streaming-read probe: the bandwidth a plain read of a buffer reaches on this device, the
// bound a kernel that must read the same bytes once can hope for (as opposed to the
// published HBM peak).  Measurement infrastructure, not an operation of the method.
//
// Workgroups of 256 threads; workgroup w reads the 16-byte words w * 256 * 4 + k * stride
// ... in groups of 4 per thread (all 4 loads in flight before any is used), folds them
// with XOR and writes its 16-byte fold to sink[w], so no load can be dropped.
#include "../../include/lrkv.h"
#include "lrkv_launch.h"

namespace lrkv {

namespace {

constexpr int kProbeUnroll = 4;

__global__ void __launch_bounds__(256)
read_probe_kernel(const uint4* __restrict__ src, size_t n16, uint4* __restrict__ sink) {
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  const size_t stride = (size_t)gridDim.x * 256 * kProbeUnroll;
  for (size_t base = (size_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x; base < n16;
       base += stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  // fold the workgroup's lanes: thread 0 of each wave writes, waves 1..3 into their slots
  // of a 4-entry LDS array, thread 0 combines
  __shared__ uint4 part[4];
  for (int o = 32; o > 0; o >>= 1) {
    acc.x ^= __shfl_xor(acc.x, o);
    acc.y ^= __shfl_xor(acc.y, o);
    acc.z ^= __shfl_xor(acc.z, o);
    acc.w ^= __shfl_xor(acc.w, o);
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint4 r = part[0];
    for (int w = 1; w < 4; ++w) {
      r.x ^= part[w].x;
      r.y ^= part[w].y;
      r.z ^= part[w].z;
      r.w ^= part[w].w;
    }
    sink[blockIdx.x] = r;
  }
}

}  // namespace

}  // namespace lrkv

extern "C" int lrkv_read_probe(const void* buf, uint64_t bytes, int32_t workgroups, void* sink,
                               void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || workgroups <= 0 || workgroups > (1 << 20) ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 15u))
    return LRKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(lrkv::read_probe_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf),
                     (size_t)(bytes / 16), static_cast<uint4*>(sink));
  return hipGetLastError() == hipSuccess ? LRKV_OK : LRKV_ERR_HIP;
}
