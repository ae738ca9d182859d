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
constexpr int kXcds = 8;             // accelerator complex dies of one MI355X

// Device workspace shared by the calls on one (device, stream).  Every word
// that workgroups poll sits on a 128-byte line of its own.
struct WsHeader {
  uint32_t status;                   // sticky: 0 ok, else an ra_status code set on device
  uint32_t pad[31];
  uint32_t bar[kMaxChannels][32];    // barrier word of channel h in bar[h][0]
                                     // (self-resetting, see grid_barrier)
  uint32_t xbar[kXcds][32];          // two-level barrier: arrivals of XCD group x
  uint32_t xflag[kXcds][32];         // two-level barrier: release count of XCD group x
  uint32_t tiles[kMaxChannels][32];  // persistent step grids: tile counters that hand
                                     // out a step's tiles in order (zeroed per launch)
};

// How workgroups that synchronise share the chip's caches.
//   kSyncDevice: anywhere on the chip -- every workgroup writes its XCD's L2 back
//                before it arrives and invalidates it after it leaves
//   kSyncXcdGroups: the whole grid, with workgroup b on XCD b mod 8 -- one
//                workgroup per XCD writes the L2 back (two-level barrier)
//   kSyncOneXcd: every workgroup that shares data sits on one XCD, hence one L2 --
//                no write-back at all
// Every waiting workgroup still takes the agent-scope acquire: it is the only
// invalidate that reaches the CU's L1 for lines other CUs wrote.
// The host chooses the last two only after checking, once per device, that the
// dispatcher places workgroup b on XCD b mod 8.
// How the workgroups of a step kernel wait for each other between steps:
// device-wide barrier, two-level (per XCD, then across XCDs) barrier, barrier of
// workgroups that share one XCD, or a single workgroup's own barrier.
enum SyncScope { kSyncDevice = 0, kSyncXcdGroups = 1, kSyncOneXcd = 2, kSyncBlock = 3 };

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// Wait (thread 0) until the top bit of *w differs from ref's, or until *w
// differs from ref (whole word); bounded like every wait here.  False when the
// caller must exit.
template <bool kTopBit>
__device__ __forceinline__ bool spin_until(WsHeader* ws, const uint32_t* w, uint32_t ref,
                                           uint64_t limit) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (kTopBit ? ((v ^ ref) & 0x80000000u) != 0 : v != ref) return true;
    if (__hip_atomic_load(&ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > limit) {
      __hip_atomic_store(&ws->status, 6u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

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

// Two-level barrier over a whole grid of G co-resident workgroups, workgroup b
// on XCD b mod 8 (kSyncXcdGroups).  Each XCD group x counts its own arrivals on
// xbar[x] (the 2^31 scheme of grid_barrier, led by workgroup x); the last
// arrival of the group -- the one whose add carries the count across 2^31 --
// writes the XCD's L2 back once, for every workgroup of the group, and arrives
// at the grid word `bar` (led by group 0's last arrival).  When all groups are
// in, that workgroup bumps xflag[x]; the others of the group wait for the bump.
// Everyone then takes the agent-scope acquire.  One L2 write-back per XCD per
// barrier, and no word takes more than G/8 arrivals, where the one-level
// barrier pays G of each (measured at 1024 workgroups: about 11-18 us against
// 66-123 us).
__device__ __forceinline__ bool xcd_barrier(WsHeader* ws, uint32_t* bar, uint32_t expect_extra,
                                            uint64_t limit) {
  __shared__ int go;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t G = gridDim.x, b = blockIdx.x;
    const uint32_t x = b % kXcds, nx = (G - x + kXcds - 1) / kXcds;
    const uint32_t groups = G < (uint32_t)kXcds ? G : (uint32_t)kXcds;
    // the release count before this workgroup arrives: it cannot move before
    // the whole group, this workgroup included, has arrived
    const uint32_t f0 = __hip_atomic_load(&ws->xflag[x][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t inc = b == x ? 0x80000000u - (nx - 1u) : 1u;
    const uint32_t old = __hip_atomic_fetch_add(&ws->xbar[x][0], inc, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    int ok;
    if (((old ^ (old + inc)) & 0x80000000u) != 0) {
      release_agent();
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t ginc = x == 0 ? 0x80000000u - (groups + expect_extra - 1u) : 1u;
      const uint32_t gold = __hip_atomic_fetch_add(bar, ginc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = spin_until<true>(ws, bar, gold, limit);
      __hip_atomic_fetch_add(&ws->xflag[x][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      ok = spin_until<false>(ws, &ws->xflag[x][0], f0, limit);
    }
    acquire_agent();
    go = ok;
  }
  __syncthreads();
  return go != 0;
}

// Barrier among workgroups that all sit on one XCD (kSyncOneXcd): their stores
// meet in the XCD's L2, so arriving needs only the workgroup's own stores to be
// acknowledged there -- no L2 write-back.  Same counting, acquire, timeout and
// abort rules as grid_barrier.
__device__ __forceinline__ bool xcd_local_barrier(WsHeader* ws, uint32_t* bar, bool leader,
                                                  uint32_t nblocks, uint32_t expect_extra,
                                                  uint64_t limit) {
  __shared__ int go;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t inc = leader ? 0x80000000u - (nblocks + expect_extra - 1u) : 1u;
    const uint32_t old = __hip_atomic_fetch_add(bar, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    go = spin_until<true>(ws, bar, old, limit);
    acquire_agent();
  }
  __syncthreads();
  return go != 0;
}

// Wait until *flag >= target (thread 0 spins, the workgroup follows).  Same
// timeout and abort rules as grid_barrier.  Returns false when the caller must exit.
// The comparison is unsigned: ready counters only grow between the host's
// resets (every call numbers its hops above anything an earlier call left, and
// the host zeroes the counters before the numbering would pass 2^32), so a
// counter is below its target exactly when its unsigned value is -- also for a
// counter left at zero by a fresh buffer while the numbering is past 2^31.
__device__ __forceinline__ bool wait_flag(WsHeader* ws, const uint32_t* flag, uint32_t target,
                                          uint64_t limit) {
  __shared__ int go;
  if (threadIdx.x == 0) {
    int ok = 1;
    if (ld_relaxed(flag) < target) {
      uint64_t t0 = now_ticks();
      while (ld_relaxed(flag) < target) {
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

// Publish *flag = value after every wave's stores of this workgroup.  kLocal:
// the readers sit on this workgroup's XCD, so the stores only have to reach its
// L2 (no write-back).
template <bool kLocal = false>
__device__ __forceinline__ void post_flag(uint32_t* flag, uint32_t value) {
  if (kLocal) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    workgroup_release_agent();
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Test hook: when `seed` is nonzero, hold this workgroup for a pseudo-random
// 0-23 x 2048 clocks (about 0-25 us), different for every workgroup, point and
// call.  Arrival orders at barriers and flags get shuffled; a correct protocol
// gives the same bits whatever the order.
__device__ __forceinline__ void stress_delay(uint32_t seed, uint32_t point) {
  if (seed == 0) return;
  if (threadIdx.x == 0) {
    uint32_t h = (blockIdx.x + 1u) * 2654435761u ^ (point + 1u) * 40503u ^ seed * 2246822519u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    for (uint32_t i = (h >> 8) % 24u; i > 0; --i) __builtin_amdgcn_s_sleep(32);
  }
  __syncthreads();
}

__device__ __forceinline__ bool ws_failed(WsHeader* ws) {
  if (ws == nullptr) return false;          // a launch without workspace has no waits
  __shared__ int bad;
  if (threadIdx.x == 0) bad = ld_relaxed(&ws->status) != 0;
  __syncthreads();
  return bad != 0;
}

}  // namespace ra
