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

// The same copy on a resident grid of `grid` workgroups that loop over 16 KiB
// tiles (four vectors per thread), tile t = b, b + grid, ... for workgroup b:
// the shape of the persistent step kernels, and the ceiling they are rated
// against.  The 16-byte vectors past the last whole tile go one per thread.
__global__ __launch_bounds__(kBlock) void k_copy_resident(u32x4* __restrict__ dst,
                                                          const u32x4* __restrict__ src,
                                                          int64_t nvec) {
  constexpr int U = 4;
  const int64_t tiles = nvec / (kBlock * U);
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t base = t * kBlock * U + threadIdx.x;
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = ld16<true>(src, base + u * kBlock);
#pragma unroll
    for (int u = 0; u < U; ++u) st16<true>(dst, base + u * kBlock, x[u]);
  }
  for (int64_t v = tiles * kBlock * U + (int64_t)blockIdx.x * kBlock + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * kBlock)
    st16<true>(dst, v, ld16<true>(src, v));
}

hipError_t launch_copy_resident(void* dst, const void* src, int64_t bytes, int grid, hipStream_t s) {
  const int64_t nvec = bytes / 16;
  if (nvec == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_resident, dim3(grid), dim3(kBlock), 0, s, reinterpret_cast<u32x4*>(dst),
                     reinterpret_cast<const u32x4*>(src), nvec);
  return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t* dst, uint32_t value, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kBlock)
    dst[i] = value;
}

hipError_t launch_fill_u32(uint32_t* dst, uint32_t value, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((count + kBlock - 1) / kBlock, 1024);
  hipLaunchKernelGGL(k_fill_u32, dim3(grid), dim3(kBlock), 0, s, dst, value, count);
  return hipGetLastError();
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
