// ra_copy.hip -- plain streaming copy, a measurement helper: the streaming
// ceiling the all-reduce kernels are compared with, and the known-size kernel
// HBM byte counters are calibrated against.  Not part of the all-reduce.
#include "ra_elem.h"
#include "ra_internal.h"

namespace ra {

// One 16-byte vector per thread, the most workgroups in flight: the shape that
// streamed best in a sweep on MI355X (6.2 TB/s plain, 6.5 TB/s with the
// streaming hint at 16 GiB, against 5.6 TB/s with four vectors per thread).
template <bool NT>
__global__ __launch_bounds__(kBlock) void k_copy(u32x4* __restrict__ dst,
                                                 const u32x4* __restrict__ src, int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t v = (int64_t)blockIdx.x * kBlock + threadIdx.x; v < nvec; v += stride)
    st16<NT>(dst, v, ld16<NT>(src, v));
}

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s) {
  const int64_t nvec = bytes / 16;
  if (nvec == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((nvec + kBlock - 1) / kBlock, kMaxGrid);
  if (bytes > kStreamingBytes)
    hipLaunchKernelGGL(k_copy<true>, dim3(grid), dim3(kBlock), 0, s, reinterpret_cast<u32x4*>(dst),
                       reinterpret_cast<const u32x4*>(src), nvec);
  else
    hipLaunchKernelGGL(k_copy<false>, dim3(grid), dim3(kBlock), 0, s, reinterpret_cast<u32x4*>(dst),
                       reinterpret_cast<const u32x4*>(src), nvec);
  return hipGetLastError();
}

}  // namespace ra
