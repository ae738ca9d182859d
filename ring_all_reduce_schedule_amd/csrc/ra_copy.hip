// ra_copy.hip -- plain streaming copy, a measurement helper: the streaming
// ceiling the all-reduce kernels are compared with, and the known-size kernel
// HBM byte counters are calibrated against.  Not part of the all-reduce.
#include "ra_elem.h"
#include "ra_sync.h"
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
// tiles (four vectors per thread), taken as the persistent step kernels take a
// large step's tiles: workgroup b belongs to group b mod qn (its XCD), each
// group takes a contiguous range of tiles, sized to its share of the grid, in
// order from a counter of its own (ctr[32*x], zeroed before the launch).  The
// ceiling those kernels are rated against.  The 16-byte vectors past the last
// whole tile go one per thread.
__global__ __launch_bounds__(kBlock) void k_copy_resident(u32x4* __restrict__ dst,
                                                          const u32x4* __restrict__ src,
                                                          int64_t nvec, uint32_t* ctr, int qn) {
  constexpr int U = 4;
  const int64_t tiles = nvec / (kBlock * U);
  const int64_t nb = gridDim.x, b = blockIdx.x;
  const int xq = (int)(b % qn);
  const int64_t per = nb / qn, more = nb % qn;
  const int64_t w0 = xq * per + (xq < more ? xq : more), wq = per + (xq < more ? 1 : 0);
  const int64_t t0 = tiles * w0 / nb, t1 = tiles * (w0 + wq) / nb;
  __shared__ uint32_t grab;
  for (;;) {
    if (threadIdx.x == 0)
      grab = __hip_atomic_fetch_add(ctr + 32 * xq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t t = t0 + grab;
    __syncthreads();
    if (t >= t1) break;
    const int64_t base = t * kBlock * U + threadIdx.x;
    u32x4 x[U];
    for (int u = 0; u < U; ++u) x[u] = ld16<true>(src, base + u * kBlock);
    for (int u = 0; u < U; ++u) st16<true>(dst, base + u * kBlock, x[u]);
  }
  for (int64_t v = tiles * kBlock * U + b * kBlock + threadIdx.x; v < nvec; v += nb * kBlock)
    st16<true>(dst, v, ld16<true>(src, v));
}

hipError_t launch_copy_resident(void* dst, const void* src, int64_t bytes, int grid,
                                uint32_t* ctr, hipStream_t s) {
  const int64_t nvec = bytes / 16;
  if (nvec == 0) return hipSuccess;
  const int qn = grid < kXcds ? grid : kXcds;
  hipError_t e = launch_fill_u32(ctr, 0u, (int64_t)qn * 32, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_copy_resident, dim3(grid), dim3(kBlock), 0, s, reinterpret_cast<u32x4*>(dst),
                     reinterpret_cast<const u32x4*>(src), nvec, ctr, qn);
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
