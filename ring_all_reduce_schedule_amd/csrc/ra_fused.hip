// ra_fused.hip -- the fused one-pass all-reduce kernel (gfx950) and its launcher.
//
// One launch per all-reduce.  Every element is folded in exactly the order the
// ring accumulates it ("Ring All-Reduce, in depth", section "The schedule":
// chunk c leaves rank c at reduce-scatter step 0 and picks up ranks c+1, c+2,
// ... one hop per step, the all-gather then copies the finished sum), rounding
// to the buffer type at every hop, and the result is stored to all p ranks.
// Every rank buffer is read once and written once: 2*p*S bytes, the least any
// one-GPU all-reduce can move.  All element traffic uses 16-byte vector
// loads/stores with consecutive lanes on consecutive vectors; chunk edges that
// fall inside a vector are handled element by element.  Indices are 64-bit.
#include <cstdlib>
#include <mutex>
#include <unordered_map>

#include "ra_elem.h"
#include "ra_internal.h"

namespace ra {

// What one fused pass produces.
//   kAllReduce      every element folded in its ring order, stored to every rank
//   kReduceScatter  the same fold, stored only to the chunk's owner: chunk c ends
//                   the reduce-scatter on rank c - 1 ("Ring All-Reduce, in
//                   depth", section "The schedule": rank r owns chunk r + 1);
//                   the other chunks of every rank are left as they were
//   kAllGather      the owner's copy of chunk c (rank c - 1) stored to the
//                   other p - 1 ranks, no arithmetic
// Bytes moved: 2pS, (p+1)S and pS.  A reduce-scatter and all-gather used on
// their own, as sharded optimisers do ("Ring All-Reduce, in depth", section
// "Trade-offs"), each move the least their output needs.
enum FusedMode { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2 };

// The chunks' edge elements (those that share a 16-byte vector with the
// neighbouring chunk), one chunk per wave (edge_wave): edge workgroup w carries
// chunks 4w .. 4w + 3.  Lane k folds element k of chunk c in ring order and
// leaves what each rank stores.
template <int DT, int OP, bool WIDE, int MODE>
__device__ __forceinline__ void fused_edges(const RankPtrs& P, const ChunkGeo& g, int p,
                                            int64_t w) {
  typedef Elem<DT> E;
  typedef Fold<DT, OP, WIDE> F;
  EdgeLds<DT>& L = edge_lds<DT>();
  void** lp = L.lp;
  load_rank_table(lp, P, p);
  const int wave = (int)(threadIdx.x / kWave);
  const int64_t cw = w * kWavesPerBlock + wave;
  const int c = cw < p ? (int)cw : 0;
  const int64_t lo = cw < p ? chunk_lo(g, c) : 0, hi = cw < p ? chunk_hi(g, c) : 0;
  const int owner = c == 0 ? p - 1 : c - 1;
  edge_wave<DT>(lp, p, lo, hi, L.slab[wave], [&](EdgeSlab<DT>& sl, int k) {
    typename E::S out;
    if (MODE == kAllGather) {
      out = sl.x[k][owner];
    } else {
      typename F::A1 acc = F::start1(sl.x[k][c], p);
      for (int j = 1; j < p; ++j) {
        const int r = c + j < p ? c + j : c + j - p;
        acc = F::step1(acc, sl.x[k][r], p);
      }
      out = F::finish1(acc);
    }
    if (MODE == kReduceScatter) {
      sl.x[k][owner] = out;
      sl.mask[k] = 1ull << owner;
    } else {
      for (int r = 0; r < p; ++r) sl.x[k][r] = out;
      sl.mask[k] = all_ranks(p) & ~(MODE == kAllGather ? 1ull << owner : 0ull);
    }
  });
}

// Tile t = (chunk c, tile j of that chunk), one 16-byte vector per thread,
// numbered by tile_of.  For every element of the tile: acc = x_c;
// acc = acc + x_{c+1}; ...; acc = acc + x_{c+p-1} (indices mod p, rounding each
// addition), the order in which the step-by-step ring accumulates chunk c, so
// the bits match.  OP and WIDE choose the reduction and the accumulation type
// (Fold in ra_elem.h).  When the chunks have edge elements, edge workgroups
// e0 .. e0 + edges - 1 (placed by edge_start) fold them, one chunk per wave,
// while the tiles run, and the other workgroups take the tiles in order: left in
// each chunk's first tile they were a second memory round trip after its
// vectors, and in a launch whose workgroups all run at once the slowest
// workgroup sets the time (p = 9, 1,000,003 int32 per rank: 19.4 us against
// 17.4 with chunk starts on lines, before the move).
template <int DT, int OP, bool WIDE, bool NT, int MODE>
__global__ __launch_bounds__(kBlock) void k_fused(RankPtrs P, ChunkGeo g, int p, int64_t T,
                                                  int64_t ntiles, int edges, int64_t e0,
                                                  int tail_last) {
  typedef Fold<DT, OP, WIDE> F;
  constexpr int V = Elem<DT>::V;
  const int64_t b = blockIdx.x;
  auto tile = [&](int c, int64_t j) {
    const int owner = c == 0 ? p - 1 : c - 1;
    const int64_t lo = chunk_lo(g, c), hi = chunk_hi(g, c);
    const Span sp = split_span<V>(lo, hi);
    const int64_t vt = sp.vb + j * kBlock;          // the tile's first vector
    const unsigned lane = threadIdx.x;
    if (vt + lane >= sp.v0 && vt + lane < sp.v1) {
      u32x4 out;
      if (MODE == kAllGather) {
        out = ld16t<NT>(P.b[owner], vt, lane);
      } else {
        typename F::A acc = F::start(ld16t<NT>(P.b[c], vt, lane), p);
        fold_run<NT, F>(acc, P, 0, p, c + 1, p - 1, vt, lane, p);
        out = F::finish(acc);
      }
      if (MODE == kReduceScatter)
        st16t<NT>(P.b[owner], vt, lane, out);
      else
        store_all<NT>(P, p, vt, lane, out, MODE == kAllGather ? owner : -1);
    }
  };
  // launches with no edge elements and whole last tiles take a loop with none
  // of the placement arithmetic: at one tile per workgroup it was a visible part
  // of a small call (p = 64 with 8,192 bfloat16 per chunk: 25.9 us with this
  // loop, 26.3 through the general one)
  if (edges == 0 && !tail_last) {
    const uint32_t T32 = (uint32_t)T;
    for (int64_t t = b; t < ntiles; t += gridDim.x) {
      const uint32_t c = (uint32_t)t / T32;
      tile((int)c, (int64_t)((uint32_t)t - c * T32));
    }
    return;
  }
  // the edge workgroups' work outside the tile loop: inside it, values the
  // compiler keeps live across the loop added to the edge code's registers
  if (b >= e0 && b < e0 + edges) fused_edges<DT, OP, WIDE, MODE>(P, g, p, b - e0);
  for (int64_t v = b; v < ntiles + edges; v += gridDim.x) {
    if (v >= e0 && v < e0 + edges) continue;
    int c;
    int64_t j;
    tile_of((uint32_t)(v < e0 ? v : v - edges), (uint32_t)T, (uint32_t)p, tail_last, &c, &j);
    tile(c, j);
  }
}


// ---------------------------------------------------------------- read and write phases
//
// The same fold as k_fused on a resident grid whose reads and writes take turns
// across the whole chip.  Iteration k of every wave (tile b + k * grid) loads
// and folds in read window k and stores in write window k; the windows follow
// each other every `period` ticks of the device's constant 100 MHz clock, the
// read window taking kPhaseReadShare/256 of it.  Every wave places its first
// window at the first multiple of the period (counted on the clock's low 32
// bits) at least kPhaseLead ticks after its own start, so all waves keep one
// grid of windows without exchanging anything: the launch needs no workspace
// and can be captured in a HIP graph.  A wave whose loads land late stores at
// once, and one that starts late simply joins a later window.
//
// Why: HBM streams 8 ranks' reads alone at 7.09 TB/s and their writes alone at
// 6.67, but the one-shot pass, whose workgroups each read eight vectors and
// then write eight, mixes the two at every instant and runs at 6.1-6.35 TB/s
// (8 x 16 GB bfloat16); on a resident grid left to itself the mix is worse
// (about 5.6).  With the turns enforced the same bytes moved at 6.39-6.45 TB/s
// on every box measured, as long as the period leaves the memory enough time:
// at 8 x 16 GB bfloat16 (134 MB per window pair) 2080-2100 ticks held window
// for window in every run, 2075 fell behind in one run of three, 2050 in every
// run, and a wave grid that falls behind runs like the resident grid left to
// itself.  kPhaseRate sets the period from the bytes of one window pair, with
// a margin over that edge; RA_PHASE_GBPS overrides it (measurements only).
// The rate the memory sustains in phases depends on the rank count and on where
// the buffers lie.  At 16 GB per rank (ms, phases against the one-shot pass, two
// boxes): p = 8 39.95 / 40.84 and 39.92 / 42.06, p = 7 38.28 / 38.45 and 38.39 /
// 38.94, p = 6 30.26 / 30.61 and 36.59 / 35.10, p = 5 28.81 / 26.14, p = 4
// 20.42 / 19.98; at 7 ranks and fewer the windows fell behind on some box, so
// the library picks the phases for 8 ranks only, where they held on every box.
// The standalone all-gather (one read, p - 1 writes per tile) gains as well at
// p = 8: 20.03 and 20.22 ms sized for 6.4 and 6.35 TB/s against 21.02 and 21.37
// (6.6 fell behind); it takes them, sized for 6.35.
// Smaller buffers lie closer together, and eight streams at the same offsets of
// buffers less than about 12 GiB apart meet on the same HBM channels: the
// one-shot pass slows down, but the phases fall behind their windows and lose
// more.  At 8 ranks (ms, phases / one-shot, one box): 512 MiB per rank 1.761 /
// 1.559, 1 GiB 3.546 / 3.161, 2 GiB 7.110 / 6.405, 4 GiB 13.27 / 12.57, 8 GiB
// 21.79 / 21.36, 16 GB 39.94 / 41.57; so the library picks them from 12 GiB per
// rank.
// The standalone reduce-scatter (p reads, one write) does not: at best 24.48
// against 24.66 ms, and behind its windows from 6.6 TB/s up -- its short write
// windows cost a memory round trip each -- so it takes them only when forced.
constexpr int kPhasedPerCU = 8;                  // 256-thread workgroups: 8 waves per SIMD
// bytes per second a window pair is sized for, and the read window's share of
// the period (of 256), per mode: all-reduce (reads land up to a round trip
// late), all-gather (one read in p), reduce-scatter (forced only)
constexpr int64_t kPhaseRate = 6420000000000ll, kPhaseReadShare = 136;
constexpr int64_t kPhaseRateAG = 6350000000000ll, kPhaseReadShareAG = 38;
constexpr int64_t kPhaseRateRS = 6000000000000ll, kPhaseReadShareRS = 226;
constexpr int64_t kPhasedMinRankBytes = 12ll << 30;   // bytes per rank the library picks them from
constexpr uint32_t kPhaseLead = 500;             // ticks: the grid's dispatch fits in 5 us
constexpr uint64_t kMaxClockWait = 1000000;      // ticks (10 ms): a bound on any one wait
constexpr int kPhasedRanks = 8;                  // the rank count the library picks them for

__device__ __forceinline__ void wait_clock(uint64_t t) {
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  if (t <= now || t - now > kMaxClockWait) return;
  while (__builtin_amdgcn_s_memrealtime() < t) __builtin_amdgcn_s_sleep(1);
}

template <int DT, int OP, bool WIDE, bool NT, int MODE>
__global__ __launch_bounds__(kBlock, kPhasedPerCU) void k_fused_phased(RankPtrs P, ChunkGeo g,
                                                                      int p, int64_t T,
                                                                      int64_t ntiles, int edges,
                                                                      uint32_t period,
                                                                      uint32_t rwin) {
  typedef Fold<DT, OP, WIDE> F;
  constexpr int V = Elem<DT>::V;
  const int64_t b = blockIdx.x;
  if (b < edges) fused_edges<DT, OP, WIDE, MODE>(P, g, p, b);
  uint64_t R = __builtin_amdgcn_s_memrealtime() + kPhaseLead;
  R += period - (uint32_t)R % period;
  const uint32_t T32 = (uint32_t)T;
  const unsigned lane = threadIdx.x;
  for (int64_t t = b; t < ntiles; t += gridDim.x, R += period) {
    // the tile index passes through a register the compiler cannot see into:
    // otherwise it keeps a running pointer per rank across iterations, and the
    // kernel no longer fits 8 waves per SIMD without spilling
    uint32_t tt = (uint32_t)t;
    asm volatile("" : "+s"(tt));
    const uint32_t c = tt / T32;
    const int64_t j = (int64_t)(tt - c * T32);
    const Span sp = split_span<V>(chunk_lo(g, (int)c), chunk_hi(g, (int)c));
    const int64_t vt = sp.vb + j * kBlock;          // the tile's first vector
    const bool in = vt + lane >= sp.v0 && vt + lane < sp.v1;
    const int owner = c == 0 ? p - 1 : (int)c - 1;
    wait_clock(R);
    u32x4 out = {0u, 0u, 0u, 0u};
    if (in) {
      if (MODE == kAllGather) {
        out = ld16t<NT>(P.b[owner], vt, lane);
      } else {
        typename F::A acc = F::start(ld16t<NT>(P.b[c], vt, lane), p);
        fold_run<NT, F>(acc, P, 0, p, (int)c + 1, p - 1, vt, lane, p);
        out = F::finish(acc);
      }
    }
    wait_clock(R + rwin);
    if (in) {
      if (MODE == kReduceScatter)
        st16t<NT>(P.b[owner], vt, lane, out);
      else
        store_all<NT>(P, p, vt, lane, out, MODE == kAllGather ? owner : -1);
    }
  }
}

// Compute units and clock ticks per second of the current device (cached).
static hipError_t phase_device(int* cus, int64_t* tick_hz) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::unordered_map<int, std::pair<int, int64_t>> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int n = 0, khz = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess || khz <= 0) khz = 100000;    // the gfx9 constant clock
    it = cache.emplace(dev, std::make_pair(n, (int64_t)khz * 1000)).first;
  }
  *cus = it->second.first;
  *tick_hz = it->second.second;
  return hipSuccess;
}

// The rate a window pair is sized for and the read window's share of it (of 256),
// per mode, or RA_PHASE_GBPS / RA_PHASE_READ256 when set (measurements only).
static void phase_shape(int mode, int64_t* rate, int64_t* read256) {
  *rate = mode == kAllGather ? kPhaseRateAG : mode == kReduceScatter ? kPhaseRateRS : kPhaseRate;
  *read256 = mode == kAllGather      ? kPhaseReadShareAG
             : mode == kReduceScatter ? kPhaseReadShareRS
                                      : kPhaseReadShare;
  const char* v = std::getenv("RA_PHASE_GBPS");
  const double gbps = v ? std::atof(v) : 0.0;
  if (gbps > 100.0 && gbps < 100000.0) *rate = (int64_t)(gbps * 1e9);
  const char* w = std::getenv("RA_PHASE_READ256");
  const int share = w ? std::atoi(w) : 0;
  if (share > 0 && share < 256) *read256 = share;
}

// The pass as k_fused_phased when `phases` asks for it (kPhasesForce) or allows
// it (kPhasesAuto: an all-reduce or all-gather of 8 ranks of at least
// kPhasedMinRankBytes each) and the device holds the whole grid; *launched false
// leaves the call to the one-shot kernel.
template <int DT, int OP, bool WIDE, bool NT, int MODE>
static hipError_t phased_launch(const RankPtrs& P, const ChunkGeo& g, int p, int64_t n,
                                int64_t T, int64_t ntiles, int edges, int phases, hipStream_t s,
                                int* grid_used, bool* launched) {
  *launched = false;
  if (phases == kPhasesOff) return hipSuccess;
  if (phases == kPhasesAuto && (MODE == kReduceScatter || p != kPhasedRanks || !NT ||
                                n * (int64_t)sizeof(typename Elem<DT>::S) < kPhasedMinRankBytes))
    return hipSuccess;
  int cus = 0;
  int64_t tick_hz = 0;
  hipError_t e = phase_device(&cus, &tick_hz);
  if (e != hipSuccess) return e;
  const unsigned lds = edges ? (unsigned)sizeof(EdgeLds<DT>) : 0u;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, reinterpret_cast<const void*>(k_fused_phased<DT, OP, WIDE, NT, MODE>), kBlock, lds);
  if (e != hipSuccess) return e;
  if (per_cu < kPhasedPerCU) return hipSuccess;
  if (phases == kPhasesAuto) {
    // a variant that spills registers to memory to fit 8 waves per SIMD (float64
    // maximum) would stream its spills beside the data: left to the one-shot pass
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa,
                             reinterpret_cast<const void*>(k_fused_phased<DT, OP, WIDE, NT, MODE>));
    if (e != hipSuccess) return e;
    if (fa.localSizeBytes > 0) return hipSuccess;
  }
  const int64_t G = (int64_t)kPhasedPerCU * cus;
  // one window pair: G tiles, each moving per thread p vectors read and p written
  // (all-reduce), p read and 1 written (reduce-scatter), 1 read and p - 1 written
  // (all-gather)
  const int64_t per_tile = MODE == kAllReduce ? 2 * (int64_t)p : MODE == kReduceScatter
                                                                      ? (int64_t)p + 1
                                                                      : (int64_t)p;
  const int64_t bytes = G * kBlock * 16 * per_tile;
  int64_t rate = 0, read256 = 0;
  phase_shape(MODE, &rate, &read256);
  const int64_t period = std::max<int64_t>(64, (bytes * (tick_hz / 1000) + rate / 1000 - 1) /
                                                   (rate / 1000));
  if (period > 0x7FFFFFFFll) return hipSuccess;
  const uint32_t rwin = (uint32_t)(period * read256 / 256);
  const int grid = (int)std::max<int64_t>(std::max<int64_t>(std::min<int64_t>(G, ntiles), edges), 1);
  *grid_used = grid;
  hipLaunchKernelGGL((k_fused_phased<DT, OP, WIDE, NT, MODE>), dim3(grid), dim3(kBlock), lds, s, P,
                     g, p, T, ntiles, edges, (uint32_t)period, rwin);
  *launched = true;
  return hipGetLastError();
}


// One vector per thread.  Measured on MI355X at 8 x 16 GiB bf16: one vector per
// thread with the most workgroups in flight streams best (6.40 TB/s on 2pS
// against 6.35 with two and 6.30 with four).
template <int DT, int OP, bool WIDE, int MODE>
static hipError_t fused_launch(const RankPtrs& P, int p, int64_t n, int phases, hipStream_t s,
                               int* grid_used) {
  const int V = Elem<DT>::V;
  const ChunkGeo g = make_geo(0, n, p);
  int64_t widest = 0;
  int edges = 0;
  for (int c = 0; c < p; ++c) {
    const int64_t lo = host_chunk_lo(0, n, p, c), hi = host_chunk_lo(0, n, p, c + 1);
    widest = std::max<int64_t>(widest, tiled_vecs_in(lo, hi, V));
    if (hi > lo && (lo % V != 0 || hi % V != 0 || vecs_in(lo, hi, V) == 0))
      edges = (p + kWavesPerBlock - 1) / kWavesPerBlock;     // a wave per chunk
  }
  const int64_t T = std::max<int64_t>(1, (widest + kBlock - 1) / kBlock);
  const int64_t ntiles = (int64_t)p * T;
  // the chunks' last tiles are short, in a launch whose tiles are all resident
  const int tail_last = ntiles <= kResidentTiles && short_tail(widest, kBlock);
  if (ntiles + edges > 0xFFFFFFFFll) return hipErrorInvalidValue;   // tile_of decodes 32 bits
  {
    bool launched = false;
    const hipError_t e =
        streaming(p, n, DT)
            ? phased_launch<DT, OP, WIDE, true, MODE>(P, g, p, n, T, ntiles, edges, phases, s,
                                                      grid_used, &launched)
            : phased_launch<DT, OP, WIDE, false, MODE>(P, g, p, n, T, ntiles, edges, phases, s,
                                                       grid_used, &launched);
    if (e != hipSuccess || launched) return e;
  }
  const int grid = (int)std::min<int64_t>(ntiles + edges, kMaxGrid);
  const int64_t e0 = edge_start(ntiles, p, tail_last, edges, grid);
  const unsigned lds = edges ? (unsigned)sizeof(EdgeLds<DT>) : 0u;
  *grid_used = grid;
  if (streaming(p, n, DT))
    hipLaunchKernelGGL((k_fused<DT, OP, WIDE, true, MODE>), dim3(grid), dim3(kBlock), lds, s, P, g,
                       p, T, ntiles, edges, e0, tail_last);
  else
    hipLaunchKernelGGL((k_fused<DT, OP, WIDE, false, MODE>), dim3(grid), dim3(kBlock), lds, s, P, g,
                       p, T, ntiles, edges, e0, tail_last);
  return hipGetLastError();
}

// (dtype, op, wide) combinations that exist: avg needs a float type, wide needs
// bfloat16, float16 or float32 and a sum or an average (a maximum is exact).
template <int DT, int MODE>
static hipError_t fused_op(const RankPtrs& P, int p, int64_t n, int op, bool wide, int phases,
                           hipStream_t s, int* grid_used) {
  constexpr bool kFloat = DT == 1 || DT == 2 || DT == 3 || DT == 4;
  constexpr bool kWide = DT == 1 || DT == 2 || DT == 3;
  if (MODE == kAllGather) return fused_launch<DT, kSum, false, MODE>(P, p, n, phases, s, grid_used);
  if (op == kMax) return fused_launch<DT, kMax, false, MODE>(P, p, n, phases, s, grid_used);
  if constexpr (kWide) {
    if (wide) {
      if (op == kAvg) return fused_launch<DT, kAvg, true, MODE>(P, p, n, phases, s, grid_used);
      return fused_launch<DT, kSum, true, MODE>(P, p, n, phases, s, grid_used);
    }
  }
  if constexpr (kFloat) {
    if (op == kAvg) return fused_launch<DT, kAvg, false, MODE>(P, p, n, phases, s, grid_used);
  }
  return fused_launch<DT, kSum, false, MODE>(P, p, n, phases, s, grid_used);
}

template <int MODE>
static hipError_t fused_mode(const RankPtrs& P, int p, int64_t n, int dtype, int op, bool wide,
                             int phases, hipStream_t s, int* grid_used) {
  switch (dtype) {
    case 0: return fused_op<0, MODE>(P, p, n, op, wide, phases, s, grid_used);
    case 1: return fused_op<1, MODE>(P, p, n, op, wide, phases, s, grid_used);
    case 2: return fused_op<2, MODE>(P, p, n, op, wide, phases, s, grid_used);
    case 3: return fused_op<3, MODE>(P, p, n, op, wide, phases, s, grid_used);
    case 4: return fused_op<4, MODE>(P, p, n, op, wide, phases, s, grid_used);
    default: return fused_op<5, MODE>(P, p, n, op, wide, phases, s, grid_used);
  }
}

// ---------------------------------------------------------------- two-level order

// The hierarchical ring ("Ring All-Reduce, in depth", section "What real
// libraries add", hierarchy) in one pass.  With g ranks per node and m = p / g
// nodes, element i lies in chunk c of the g-way partition (the shard that local
// rank c - 1 owns after the in-node reduce-scatter) and in sub-chunk d of that
// shard cut m ways (the piece whose cross-node ring starts at node d).  Its
// result is
//   A_q = x[q*g + c] (op) x[q*g + c+1] (op) ... (op) x[q*g + c+g-1]   (local indices mod g)
//   out = A_d (op) A_{d+1} (op) ... (op) A_{d+m-1}                   (nodes mod m)
// with every hop rounded to the element type: the order in which the in-node
// reduce-scatter and the cross-node ring accumulate it.  Tile t = (segment
// (c, d), tile j), one 16-byte vector per thread.
// Segment (c, d) of the two-level partition: sub-chunk d of in-node chunk c.
__device__ __forceinline__ void hier_segment(const ChunkGeo& gi, int M, int seg, int* c, int* d,
                                             int64_t* lo, int64_t* hi) {
  *c = seg / M;
  *d = seg - *c * M;
  const int64_t clo = chunk_lo(gi, *c), chi = chunk_hi(gi, *c);
  const ChunkGeo sg = {clo, (chi - clo) / M, (chi - clo) % M};
  *lo = chunk_lo(sg, *d);
  *hi = chunk_hi(sg, *d);
}

// The segments' edge elements, one segment per wave (edge_wave): edge workgroup
// w carries segments 4w .. 4w + 3.  Lane k folds element k of segment (c, d) in
// the two-level order and stores the result to every rank.
template <int DT, int OP>
__device__ __forceinline__ void hier_edges(const RankPtrs& P, const ChunkGeo& gi, int p, int G,
                                           int M, int64_t w) {
  typedef Elem<DT> E;
  typedef Fold<DT, OP, false> F;
  EdgeLds<DT>& L = edge_lds<DT>();
  void** lp = L.lp;
  load_rank_table(lp, P, p);
  const int wave = (int)(threadIdx.x / kWave);
  const int64_t sw = w * kWavesPerBlock + wave;
  int c = 0, d = 0;
  int64_t lo = 0, hi = 0;
  if (sw < (int64_t)G * M) hier_segment(gi, M, (int)sw, &c, &d, &lo, &hi);
  edge_wave<DT>(lp, p, lo, hi, L.slab[wave], [&](EdgeSlab<DT>& sl, int k) {
    typename E::S total = 0;
    for (int k2 = 0; k2 < M; ++k2) {
      const int q = d + k2 < M ? d + k2 : d + k2 - M;
      typename E::S acc = F::start1(sl.x[k][q * G + c], p);
      for (int k1 = 1; k1 < G; ++k1) {
        const int l = c + k1 < G ? c + k1 : c + k1 - G;
        acc = F::step1(acc, sl.x[k][q * G + l], p);
      }
      total = k2 == 0 ? acc : comb1<DT, OP>(total, acc);
    }
    for (int r = 0; r < p; ++r) sl.x[k][r] = total;
    sl.mask[k] = all_ranks(p);
  });
}

// Tiles as in k_fused, over the G*M segments; the segments' edge elements, when
// there are any, go to edge workgroups e0 .. e0 + edges - 1, a segment per wave,
// as in k_fused.
template <int DT, int OP, bool NT>
__global__ __launch_bounds__(kBlock) void k_fused_hier(RankPtrs P, ChunkGeo gi, int p, int G,
                                                       int M, int64_t T, int64_t ntiles,
                                                       int edges, int64_t e0, int tail_last) {
  typedef Fold<DT, OP, false> F;
  constexpr int V = Elem<DT>::V;
  const int64_t b = blockIdx.x;
  if (b >= e0 && b < e0 + edges) hier_edges<DT, OP>(P, gi, p, G, M, b - e0);
  for (int64_t v = b; v < ntiles + edges; v += gridDim.x) {
    if (v >= e0 && v < e0 + edges) continue;
    int c, d;
    int64_t lo, hi;
    int seg;
    int64_t j;
    tile_of((uint32_t)(v < e0 ? v : v - edges), (uint32_t)T, (uint32_t)(G * M), tail_last, &seg,
            &j);
    hier_segment(gi, M, seg, &c, &d, &lo, &hi);
    const Span sp = split_span<V>(lo, hi);
    const int64_t vt = sp.vb + j * kBlock;          // the tile's first vector
    const unsigned lane = threadIdx.x;
    if (vt + lane >= sp.v0 && vt + lane < sp.v1) {
      u32x4 total;
      for (int k2 = 0; k2 < M; ++k2) {
        const int q = d + k2 < M ? d + k2 : d + k2 - M;
        const int base = q * G;
        typename F::A acc = F::start(ld16t<NT>(P.b[base + c], vt, lane), p);
        fold_run<NT, F>(acc, P, base, G, c + 1, G - 1, vt, lane, p);
        const u32x4 node = F::finish(acc);
        total = k2 == 0 ? node : vcomb<DT, OP>(total, node);
      }
      store_all<NT>(P, p, vt, lane, total, -1);
    }
  }
}

template <int DT, int OP>
static hipError_t fused_hier_launch(const RankPtrs& P, int p, int64_t n, int G, hipStream_t s,
                                    int* grid_used) {
  const int V = Elem<DT>::V;
  const int M = p / G;
  const ChunkGeo gi = make_geo(0, n, G);
  int64_t widest = 0;
  int edges = 0;
  for (int c = 0; c < G; ++c) {
    const int64_t clo = host_chunk_lo(0, n, G, c), len = host_chunk_lo(0, n, G, c + 1) - clo;
    for (int d = 0; d < M; ++d) {
      const int64_t lo = host_chunk_lo(clo, len, M, d), hi = host_chunk_lo(clo, len, M, d + 1);
      widest = std::max<int64_t>(widest, tiled_vecs_in(lo, hi, V));
      if (hi > lo && (lo % V != 0 || hi % V != 0 || vecs_in(lo, hi, V) == 0))
        edges = (G * M + kWavesPerBlock - 1) / kWavesPerBlock;   // a wave per segment
    }
  }
  const int64_t T = std::max<int64_t>(1, (widest + kBlock - 1) / kBlock);
  const int64_t ntiles = (int64_t)G * M * T;
  const int tail_last = ntiles <= kResidentTiles && short_tail(widest, kBlock);
  if (ntiles + edges > 0xFFFFFFFFll) return hipErrorInvalidValue;   // tile_of decodes 32 bits
  const int grid = (int)std::min<int64_t>(ntiles + edges, kMaxGrid);
  const int64_t e0 = edge_start(ntiles, (int64_t)G * M, tail_last, edges, grid);
  const unsigned lds = edges ? (unsigned)sizeof(EdgeLds<DT>) : 0u;
  *grid_used = grid;
  if (streaming(p, n, DT))
    hipLaunchKernelGGL((k_fused_hier<DT, OP, true>), dim3(grid), dim3(kBlock), lds, s, P, gi, p, G,
                       M, T, ntiles, edges, e0, tail_last);
  else
    hipLaunchKernelGGL((k_fused_hier<DT, OP, false>), dim3(grid), dim3(kBlock), lds, s, P, gi, p, G,
                       M, T, ntiles, edges, e0, tail_last);
  return hipGetLastError();
}

template <int DT>
static hipError_t fused_hier_op(const RankPtrs& P, int p, int64_t n, int op, int G, hipStream_t s,
                                int* grid_used) {
  constexpr bool kFloat = DT == 1 || DT == 2 || DT == 3 || DT == 4;
  if (op == kMax) return fused_hier_launch<DT, kMax>(P, p, n, G, s, grid_used);
  if constexpr (kFloat) {
    if (op == kAvg) return fused_hier_launch<DT, kAvg>(P, p, n, G, s, grid_used);
  }
  return fused_hier_launch<DT, kSum>(P, p, n, G, s, grid_used);
}

hipError_t launch_fused_hier(const RankPtrs& P, int p, int64_t n, int dtype, int op, int g,
                             hipStream_t s, int* grid_used) {
  switch (dtype) {
    case 0: return fused_hier_op<0>(P, p, n, op, g, s, grid_used);
    case 1: return fused_hier_op<1>(P, p, n, op, g, s, grid_used);
    case 2: return fused_hier_op<2>(P, p, n, op, g, s, grid_used);
    case 3: return fused_hier_op<3>(P, p, n, op, g, s, grid_used);
    case 4: return fused_hier_op<4>(P, p, n, op, g, s, grid_used);
    default: return fused_hier_op<5>(P, p, n, op, g, s, grid_used);
  }
}

hipError_t launch_fused(const RankPtrs& P, int p, int64_t n, int dtype, int op, bool wide,
                        int mode, int phases, hipStream_t s, int* grid_used) {
  switch (mode) {
    case kReduceScatter:
      return fused_mode<kReduceScatter>(P, p, n, dtype, op, wide, phases, s, grid_used);
    case kAllGather: return fused_mode<kAllGather>(P, p, n, dtype, op, wide, phases, s, grid_used);
    default: return fused_mode<kAllReduce>(P, p, n, dtype, op, wide, phases, s, grid_used);
  }
}


}  // namespace ra
