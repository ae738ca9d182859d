// ra_sync.h -- synchronisation between workgroups for the step-by-step and
// pipelined kernels (gfx950): per-stream workspace, a self-resetting grid barrier
// and per-slice ready counters, all with bounded waits that report a timeout
// instead of hanging ("Ring All-Reduce, in depth", section "Failure modes": a
// stalled rank must fail fast).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// ---------------------------------------------------------------- workspace

constexpr int kMaxChannels = 64;

// Device workspace shared by the calls on one (device, stream).  Every word
// that workgroups poll sits on a 128-byte line of its own.
struct WsHeader {
  uint32_t status;                   // sticky: 0 ok, else an ra_status code set on device
  uint32_t pad[31];
  uint32_t bar[kMaxChannels][32];    // barrier word of channel h in bar[h][0]
                                     // (self-resetting, see grid_barrier)
};

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Make every wave's earlier global stores visible device-wide (to the L2 of
// every XCD), then let thread 0 continue to publish a flag.  The workgroup
// barrier alone does not wait for other waves' stores (it compiles to a bare
// s_barrier), so each wave first waits until its own stores are acknowledged by
// its XCD's L2; thread 0 then writes that L2 back (agent-scope release) on
// behalf of the whole workgroup -- one write-back per workgroup, not per wave --
// and waits for that write-back to finish before anything is published (the
// compiler does not always keep a wait between the write-back and a following
// flag store, and a flag seen before the data is written back would be stale).
__device__ __forceinline__ void workgroup_release_agent() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    release_agent();
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// Barrier over the `nblocks` co-resident workgroups that share the word `bar`
// (the whole grid, or one channel of it).
//
// Every workgroup adds 1 to the barrier word except one leader, which adds
// 2^31 - (nblocks - 1); one full round therefore adds exactly 2^31, so the top
// bit flips precisely when the last workgroup arrives and the low bits return to
// where they were -- the word never needs resetting between rounds or calls.  A
// waiter watches for the top bit to differ from what it saw when it arrived.
//
// `expect_extra` = 1 makes the round wait for one arrival that never comes (a
// test hook for the timeout path).  Waits are bounded by `limit` ticks of the
// constant-rate device clock; on expiry the waiter records RA_ERR_TIMEOUT (6)
// in the sticky status word.  A workgroup also gives up as soon as it sees a
// nonzero status.  Returns false when the caller must exit.
__device__ __forceinline__ bool grid_barrier(WsHeader* ws, uint32_t* bar, bool leader,
                                             uint32_t nblocks, uint32_t expect_extra,
                                             uint64_t limit) {
  __shared__ int go;
  workgroup_release_agent();
  if (threadIdx.x == 0) {
    uint32_t inc = leader ? 0x80000000u - (nblocks + expect_extra - 1u) : 1u;
    uint32_t old = __hip_atomic_fetch_add(bar, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t t0 = now_ticks();
    int ok = 1;
    while (((ld_relaxed(bar) ^ old) & 0x80000000u) == 0) {
      if (ld_relaxed(&ws->status) != 0) { ok = 0; break; }
      if (now_ticks() - t0 > limit) {
        __hip_atomic_store(&ws->status, 6u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    acquire_agent();
    go = ok;
  }
  __syncthreads();
  return go != 0;
}

// Wait until *flag >= target (thread 0 spins, the workgroup follows).  Same
// timeout and abort rules as grid_barrier.  Returns false when the caller must exit.
__device__ __forceinline__ bool wait_flag(WsHeader* ws, const uint32_t* flag, uint32_t target,
                                          uint64_t limit) {
  __shared__ int go;
  if (threadIdx.x == 0) {
    int ok = 1;
    if ((int32_t)(ld_relaxed(flag) - target) < 0) {
      uint64_t t0 = now_ticks();
      while ((int32_t)(ld_relaxed(flag) - target) < 0) {
        if (ld_relaxed(&ws->status) != 0) { ok = 0; break; }
        if (now_ticks() - t0 > limit) {
          __hip_atomic_store(&ws->status, 6u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    acquire_agent();
    go = ok;
  }
  __syncthreads();
  return go != 0;
}

// Publish *flag = value after every wave's stores of this workgroup.
__device__ __forceinline__ void post_flag(uint32_t* flag, uint32_t value) {
  workgroup_release_agent();
  if (threadIdx.x == 0)
    __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool ws_failed(WsHeader* ws) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = ld_relaxed(&ws->status) != 0;
  __syncthreads();
  return bad != 0;
}

}  // namespace ra
