// ra_internal.h -- interface between the host API (ra_api.cpp) and the kernel
// launchers (ra_kernels.hip).  Not installed; the public ABI is include/ra.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ra {

struct WsHeader;
struct RankPtrs;

// Kernel families of the step-by-step schedule run by launch_steps().
enum StepMode { kModeRing = 0, kModeBidir = 1, kModeTree = 2 };

// What every persistent (grid-synchronised) launch needs besides the data.
struct SyncCfg {
  WsHeader* ws;           // device workspace of this (device, stream)
  uint64_t limit_ticks;   // bound of one device-side wait, device clock ticks
  uint32_t expect_extra;  // 1 = first wait expects an arrival that never comes (test hook)
  uint64_t* step_ts;      // optional device array of step timestamps
  int grid;               // 0 = as many workgroups as are co-resident
};

// Launch descriptions return the number of workgroups used through *grid_used.

// One pass: each element folded in its chunk's ring order, result stored to all ranks.
hipError_t launch_fused(const RankPtrs& P, int p, int64_t n, int dtype, hipStream_t s,
                        int* grid_used);

// Steps [step_begin, step_end) of a step-by-step schedule, one cooperative launch,
// a grid barrier between steps.  Ring/bidir: steps 0..p-2 reduce-scatter,
// p-1..2p-3 all-gather.  Tree: L reduce levels then L broadcast levels.
hipError_t launch_steps(const RankPtrs& P, int p, int64_t n, int dtype, StepMode mode,
                        int step_begin, int step_end, const SyncCfg& sc, hipStream_t s,
                        int* grid_used);

// Hops [hop_begin, hop_end) of the forward ring with chunks cut into slices of
// `slice` elements and per-slice ready counters in `flags` (p * kmax entries,
// all <= `base` on entry).
hipError_t launch_pipelined(const RankPtrs& P, int p, int64_t n, int dtype, int hop_begin,
                            int hop_end, int64_t slice, int64_t kmax, uint32_t* flags,
                            uint32_t base, const SyncCfg& sc, hipStream_t s, int* grid_used);

// Slices per chunk for the pipelined kernel (the host sizes `flags` with it).
int64_t pipelined_slices_per_chunk(int p, int64_t n, int dtype, int64_t slice);

// Plain streaming copy (measurement helper).
hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s);

int elem_bytes(int dtype);

}  // namespace ra
