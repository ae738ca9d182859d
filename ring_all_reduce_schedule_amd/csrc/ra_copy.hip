// ra_copy.hip -- plain streaming copy, a measurement helper: the streaming
// ceiling the all-reduce kernels are compared with, and the known-size kernel
// HBM byte counters are calibrated against.  Not part of the all-reduce.
#include "ra_elem.h"
#include "ra_internal.h"

namespace ra {

__global__ __launch_bounds__(kBlock) void k_copy(u32x4* __restrict__ dst,
                                                 const u32x4* __restrict__ src, int64_t nvec) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * kBlock * U;
  for (int64_t base = (int64_t)blockIdx.x * kBlock * U; base < nvec; base += stride) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = base + u * kBlock + threadIdx.x;
      if (v < nvec) x[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = base + u * kBlock + threadIdx.x;
      if (v < nvec) dst[v] = x[u];
    }
  }
}


hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s) {
  const int64_t nvec = bytes / 16;
  if (nvec == 0) return hipSuccess;
  const int64_t per = (int64_t)kBlock * 4;
  const int grid = (int)std::min<int64_t>((nvec + per - 1) / per, kMaxGrid);
  hipLaunchKernelGGL(k_copy, dim3(grid), dim3(kBlock), 0, s, reinterpret_cast<u32x4*>(dst),
                     reinterpret_cast<const u32x4*>(src), nvec);
  return hipGetLastError();
}


}  // namespace ra
