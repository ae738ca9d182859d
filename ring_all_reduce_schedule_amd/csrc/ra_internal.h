// ra_internal.h -- interface between the host API (ra_api.cpp) and the kernel
// launchers (ra_fused.hip, ra_steps.hip, ra_copy.hip), plus small host helpers.
// Not installed; the public ABI is include/ra.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ra_elem.h"

namespace ra {

struct WsHeader;

// Kernel families of the step-by-step schedule run by launch_steps().
enum StepMode { kModeRing = 0, kModeBidir = 1, kModeTree = 2, kModeHier = 3 };

// What the step and pipelined launchers need besides the data.
struct SyncCfg {
  WsHeader* ws;           // device workspace of this (device, stream); null when the call
                          // cannot run a persistent grid (its launches have no waits)
  uint64_t limit_ticks;   // bound of one device-side wait, device clock ticks
  uint32_t expect_extra;  // 1 = first wait expects an arrival that never comes (test hook)
  uint32_t stress;        // nonzero: pseudo-random delays before arrivals and hops (test hook)
  uint64_t* step_ts;      // optional device array of step timestamps
  int grid;               // 0 = as many workgroups as are co-resident
  int channels;           // step kernels: independent channels (1 = whole grid, 0 = automatic)
  int group;              // kModeHier: ranks per node g (g divides p)
  bool may_probe;         // may run (and allocate for) the one-time XCD placement probe;
                          // false: an unprobed device counts as unplaced
};

// Launch descriptions return the number of workgroups used through *grid_used.

// Whether a one-pass call runs with read and write phases (k_fused_phased):
// where the library finds it pays, always where the grid fits, or never.
enum PhaseMode { kPhasesAuto = 0, kPhasesForce = 1, kPhasesOff = 2 };

// One pass: each element folded in its chunk's ring order with reduction `op`
// (wide: accumulated in the wider type).  mode 0 stores the result to all ranks
// (all-reduce), 1 only to the chunk's owner (reduce-scatter), 2 copies each
// owner's chunk to the other ranks (all-gather; op and wide unused).  phases: a
// PhaseMode.
hipError_t launch_fused(const RankPtrs& P, int p, int64_t n, int dtype, int op, bool wide,
                        int mode, int phases, hipStream_t s, int* grid_used);

// Steps [step_begin, step_end) of a step-by-step schedule, in order.  Steps
// that move at most 256 vectors run on one workgroup (its own barrier between
// steps); larger ones as one launch per step, or -- when sc asks for a grid,
// channels, step timestamps or a test hook -- as one persistent cooperative
// launch with a grid barrier between steps.  Ring/bidir: steps 0..p-2
// reduce-scatter, p-1..2p-3 all-gather.  Tree: L reduce levels then L broadcast
// levels.  Hier (g = sc.group, m = p / g): g-1 intra-node reduce-scatter steps,
// 2(m-1) inter-node all-reduce steps on the shards, g-1 intra-node all-gather
// steps.
hipError_t launch_steps(const RankPtrs& P, int p, int64_t n, int dtype, int op, StepMode mode,
                        int step_begin, int step_end, const SyncCfg& sc, hipStream_t s,
                        int* grid_used, int* launches);

// One pass in the two-level order: node partials folded over local ranks,
// then folded over nodes (g ranks per node), stored to every rank.
hipError_t launch_fused_hier(const RankPtrs& P, int p, int64_t n, int dtype, int op, int g,
                             hipStream_t s, int* grid_used);

// Hops [hop_begin, hop_end) of the forward ring with chunks cut into slices of
// `slice` elements and per-slice ready counters in `flags` (p * kmax entries,
// all <= `base` on entry).
hipError_t launch_pipelined(const RankPtrs& P, int p, int64_t n, int dtype, int op, int hop_begin,
                            int hop_end, int64_t slice, int64_t kmax, uint32_t* flags,
                            uint32_t base, const SyncCfg& sc, hipStream_t s, int* grid_used);

// The pipelined ring with every slice carried through all its hops by one
// workgroup (no flags, no barriers).  mode 0: all-reduce, 1: reduce-scatter
// (leaves the step-by-step partials), 2: all-gather.  slice_elems 0 = one tile
// (kBlock vectors) per slice; stress != 0 adds the test hook's delays.
hipError_t launch_rider(const RankPtrs& P, int p, int64_t n, int dtype, int op, int mode,
                        int64_t slice_elems, uint32_t stress, hipStream_t s, int* grid_used);

// Slices per chunk for the pipelined kernel (the host sizes `flags` with it).
int64_t pipelined_slices_per_chunk(int p, int64_t n, int dtype, int64_t slice);

// Slice length used when the caller does not choose one.
int64_t pipelined_default_slice(int p, int64_t n, int dtype, int grid_override);

// dst[0 .. count) = value, a kernel on stream s (a fill that a graph capture
// records as a kernel, not as a memset).
hipError_t launch_fill_u32(uint32_t* dst, uint32_t value, int64_t count, hipStream_t s);

// Plain streaming copy (measurement helpers): one-shot grid, and a resident
// grid of `grid` workgroups looping over tiles handed out in order from tile
// counters at ctr (8 of them, 32 words apart; zeroed here, on s).
hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s);
hipError_t launch_copy_resident(void* dst, const void* src, int64_t bytes, int grid,
                                uint32_t* ctr, hipStream_t s);

// Workgroups a persistent step kernel runs by default on the current device.
int default_persistent_workgroups();

// ---------------------------------------------------------------- host helpers

inline int elem_bytes(int dtype) {
  switch (dtype) {
    case 2: case 3: return 2;
    case 4: case 5: return 8;
    default: return 4;
  }
}

inline int elems_per_vec(int dtype) { return 16 / elem_bytes(dtype); }

// Whole 16-byte vectors inside [lo, hi) (host mirror of split_span).
inline int64_t vecs_in(int64_t lo, int64_t hi, int V) {
  int64_t a0 = (lo + V - 1) / V * V;
  int64_t a1 = hi / V * V;
  return a1 > a0 ? (a1 - a0) / V : 0;
}

// Vectors the tiles of [lo, hi) span, counted from the line their first tile
// starts on (Span::vb): the whole vectors plus up to kLineVecs - 1 before them.
inline int64_t tiled_vecs_in(int64_t lo, int64_t hi, int V) {
  int64_t a0 = (lo + V - 1) / V, a1 = hi / V;
  return a1 > a0 ? a1 - a0 / kLineVecs * kLineVecs : 0;
}

// Whether a segment of `vecs` tiled vectors ends in a tile (of `tile` vectors)
// at most half full: then launches number every segment's last tile after the
// others (tile_of in ra_elem.h).  Fuller last tiles gain nothing from it (p = 64
// with 15,625 bfloat16 per chunk, last tiles 62% full: 53.4 against 52.2 us).
inline int short_tail(int64_t vecs, int64_t tile) {
  const int64_t rem = vecs % tile;
  return rem != 0 && 2 * rem <= tile;
}

// The most workgroups of 256 threads an MI355X holds at once (256 compute units,
// 8 each).  Up to that many, a launch's workgroups are all placed in the first
// rounds of the dispatcher, and which compute unit gets which tile is decided by
// their order; beyond it, workgroups wait for free slots and the order of the
// short tiles no longer decides anything (launches keep the plain order).
constexpr int64_t kResidentTiles = 2048;

// Where a launch's edge workgroups sit in its workgroup order (e0):
// first, so their chains of round trips start at once, or -- when the segments'
// last tiles are short (tail_last) -- right after the other tiles and before the
// short ones, so that the first round of compute units gets whole tiles and the
// edge workgroups share the second round with the short tiles.  Measured at
// p = 64 (one-pass all-reduce, us): 524,365 bfloat16 per rank (short last tiles)
// 30.4-30.8 with the edge workgroups placed so (31.4 with them first, and the
// short tiles numbered like the others); 1,000,003 (last tiles 62% full) 52.6-54.5
// with them first against 55.4-56.7 with them last.
inline int64_t edge_start(int64_t ntiles, int64_t nseg, int tail_last, int edges, int64_t grid) {
  const int64_t after_whole = ntiles - nseg;          // the tiles before the short ones
  return tail_last && after_whole + edges <= grid ? after_whole : 0;
}

inline int64_t host_chunk_lo(int64_t off, int64_t len, int p, int c) {
  int64_t base = len / p, extra = len % p;
  return off + (int64_t)c * base + std::min<int64_t>(c, extra);
}

inline ChunkGeo make_geo(int64_t off, int64_t len, int p) {
  ChunkGeo g;
  g.off = off;
  g.base = len / p;
  g.extra = len % p;
  return g;
}

// Buffers larger than this in total (p * S) are streamed with non-temporal
// loads and stores: they are far beyond the 256 MB Infinity Cache, and the
// streaming hint measured +3.7% for the fused kernel at 8 x 16 GiB.  Smaller
// working sets keep normal caching so that repeated calls can hit the cache.
constexpr int64_t kStreamingBytes = 512ll << 20;

inline bool streaming(int p, int64_t n, int dtype) {
  return (int64_t)p * n * elem_bytes(dtype) > kStreamingBytes;
}

// Non-persistent grids are capped here; beyond it, workgroups loop over tiles.
// The dispatch counts the grid in work-items in 32 bits, so this is the largest
// grid of kBlock-thread workgroups there is.  A grid that covers the data once
// streams faster than one that loops: the tree at 8 x 16 GB (whole-buffer steps
// of up to 15.6 million tiles) took 89.9 ms against 91.1 with a cap of 2^22.
constexpr int64_t kMaxGrid = 0xFFFFFFFFll / kBlock;

}  // namespace ra
