// ra_steps.hip -- the step-by-step and pipelined ring kernels (gfx950) and their
// launchers.
//
// p virtual ranks live in one GPU's HBM; a "send" of the ring is a read of the
// sender's chunk and a "receive" is an add into (or a copy over) the receiver's
// chunk.  Sources: "Ring All-Reduce, in depth" (aicassindra.com), sections "The
// schedule", "An implementation", "What real libraries add"; "Derive the cost of
// a ring all-reduce" (aiinfrainterviews.com), section "Where it stops scaling".
//
//   k_step       one step of the schedule as a launch of its own: reduce-scatter
//                and all-gather steps (forward ring, or both rings of the
//                bidirectional variant on the two halves), the binomial tree's
//                levels, or the hierarchy's in-node and cross-node steps; the
//                stream's ordering separates steps.  The default for steps that
//                move more than 256 vectors; large copy steps take two vectors
//                per thread, everything else one.
//   k_steps      the same schedules in one launch: on a single workgroup (its own
//                barrier between steps; the default for smaller steps), or on a
//                persistent grid (every workgroup resident at once) with a grid
//                barrier between steps, each XCD's workgroups taking a
//                contiguous range of a step's tiles in order from a counter
//                (a caller's grid, channels, step timestamps, test hooks).
//   k_pipelined  the forward ring with chunks cut into slices; workgroups are
//                assigned to ranks, and a rank forwards slice k as soon as its
//                left neighbour has finished slice k (per-slice ready counters
//                instead of step barriers).
#include "ra_elem.h"
#include "ra_sync.h"
#include "ra_internal.h"

#include <mutex>
#include <numeric>
#include <utility>
#include <unordered_map>

namespace ra {

// ================================================================ hop on one tile

// Tile j of the segment [lo, hi): dst[i] = dst[i] (op) src[i] (ADD) or
// dst[i] = src[i].  A tile covers BS*U consecutive vectors (BS threads, U
// vectors each); tile 0 also takes the scalar head and tail of the segment.
//
// Averages ([InDepth] "Failure modes": pre-divide) divide every rank's
// contribution by p exactly once, at the first hop that reads it: div_src and
// div_dst say whether the incoming or the receiving value is still an undivided
// input, and keep_src writes the divided first term back over its input, so
// that the reduce-scatter leaves the same states as dividing every buffer first.
struct HopFlags {
  bool div_src, div_dst, keep_src;
};

// The vectors of the tile that starts at vector t0, U per thread, that lie in
// [tl, t1).  GUARD = false: the tile is whole (tl = t0, t1 - t0 = BS * U),
// so no access needs a bounds test and all 2U loads issue back to back before
// the first wait; with per-access guards the compiler splits them into
// separately waited branches.
template <int DT, int OP, int U, bool ADD, bool NT, bool GUARD, int BS>
__device__ __forceinline__ void hop_vectors(void* __restrict__ src, void* __restrict__ dst,
                                            int64_t t0, int64_t tl, int64_t t1, int p, HopFlags f) {
  constexpr bool kDiv = OP == kAvg && ADD;
  int64_t v[U];
  bool in[U];
  u32x4 a[U], b[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    v[u] = t0 + u * BS + threadIdx.x;
    in[u] = !GUARD || (v[u] >= tl && v[u] < t1);
    if (in[u]) {
      a[u] = ld16<NT>(src, v[u]);
      if (ADD) b[u] = ld16<NT>(dst, v[u]);
    }
  }
  if (kDiv) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (f.div_src) a[u] = vdiv<DT>(a[u], p);
      if (f.div_dst) b[u] = vdiv<DT>(b[u], p);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (in[u]) st16<NT>(dst, v[u], ADD ? vcomb<DT, OP>(b[u], a[u]) : a[u]);
  if (kDiv && f.keep_src) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (in[u]) st16<NT>(src, v[u], a[u]);
  }
}

template <int DT, int OP, int U, bool ADD, bool NT, int BS = kBlock>
__device__ __forceinline__ void hop_tile(void* __restrict__ src, void* __restrict__ dst,
                                         int64_t lo, int64_t hi, int64_t j, int p, HopFlags f) {
  typedef Elem<DT> E;
  constexpr int V = E::V;
  constexpr bool kDiv = OP == kAvg && ADD;
  const Span sp = split_span<V>(lo, hi);
  const int64_t tv = (int64_t)BS * U;
  const int64_t t0 = sp.vb + j * tv;               // tiles start on lines (Span)
  const int64_t tl = t0 > sp.v0 ? t0 : sp.v0;
  const int64_t t1 = t0 + tv < sp.v1 ? t0 + tv : sp.v1;
  // Tile 0 also takes the segment's edge elements.  Their loads go out before
  // the vectors' (the two sets of addresses are disjoint), so that their round
  // trip overlaps the vectors' instead of following it.
  const int64_t nh = sp.head_hi - lo, nt = hi - sp.tail_lo;
  const int t = threadIdx.x;
  const bool edge = j == 0 && t < nh + nt;
  const int64_t i = t < nh ? lo + t : sp.tail_lo + (t - nh);
  typename E::S x = 0, y = 0;
  if (edge) {
    x = ld1<DT>(src, i);
    if (ADD) y = ld1<DT>(dst, i);
  }
  if (tl == t0 && t1 - t0 == tv)        // the same for the whole workgroup
    hop_vectors<DT, OP, U, ADD, NT, false, BS>(src, dst, t0, tl, t1, p, f);
  else if (tl < t1)
    hop_vectors<DT, OP, U, ADD, NT, true, BS>(src, dst, t0, tl, t1, p, f);
  if (edge) {
    if (ADD) {
      if (kDiv) {
        if (f.div_src) x = E::div1(x, p);
        if (f.div_dst) y = E::div1(y, p);
      }
      st1<DT>(dst, i, comb1<DT, OP>(y, x));
      if (kDiv && f.keep_src) st1<DT>(src, i, x);
    } else {
      st1<DT>(dst, i, x);
    }
  }
}


// ================================================================ slice through LDS

// Vectors per thread of one LDS stage, and the stage's size in vectors.
constexpr int kStageU = 2;
constexpr int kStageV = kBlock * kStageU;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; export and LDS counters left free).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// 16-byte LDS reads that return only once the data is in registers.  The LDS
// address is the low 32 bits of the generic address of a __shared__ object.
__device__ __forceinline__ u32x4 lds_read(const u32x4* p) {
  u32x4 v;
  const uint32_t a = (uint32_t)(uintptr_t)p;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return v;
}
__device__ __forceinline__ void lds_read2(const u32x4* p, const u32x4* q, u32x4& x, u32x4& y) {
  const uint32_t a = (uint32_t)(uintptr_t)p, b = (uint32_t)(uintptr_t)q;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x), "=&v"(y) : "v"(a), "v"(b) : "memory");
}

// Issue the asynchronous copies of the stage that starts at vector v0 into one
// LDS buffer (src and dst halves): the vectors of [vl, v1) among its kStageV.
template <bool ADD, bool NT>
__device__ __forceinline__ void stage_fill(const u32x4* gsrc, const u32x4* gdst, int64_t vl,
                                           int64_t v0, int64_t v1, u32x4* __restrict__ lsrc,
                                           u32x4* __restrict__ ldst) {
  const int wave = threadIdx.x / 64;
#pragma unroll
  for (int u = 0; u < kStageU; ++u) {
    const int64_t v = v0 + u * kBlock + threadIdx.x;
    const int base = u * kBlock + wave * 64;           // this wave's 64 slots
    if (v >= vl && v < v1) {
      __builtin_amdgcn_global_load_lds(gsrc + v, lsrc + base, 16, 0, NT ? kNtPolicy : 0);
      if (ADD) __builtin_amdgcn_global_load_lds(gdst + v, ldst + base, 16, 0, NT ? kNtPolicy : 0);
    }
  }
}

// One double-buffered step: start filling the next stage, wait for the current
// one, combine it out of LDS and store.  Only the explicit wait below gates the
// reads of the current stage: they are issued as inline ds_read_b128, which
// the compiler's wait-count pass does not track.  Left to that pass, a read of
// the first buffer of each pair of stages waited for every outstanding copy,
// the next stage's included (it cannot tell the two buffers apart across the
// loop's back edge), and the double buffering was lost there: measured 10-14%
// slower at 4-16 MiB per rank.  Each read waits for its own LDS result
// (lgkmcnt) before returning, so no later copy into the same buffer can
// overtake it.  Vectors below vl (the slice's first, when its stages start on
// the line before it) are skipped; only the first stage has any.
template <int DT, int OP, bool ADD, bool NT>
__device__ __forceinline__ void stage_step(void* src, void* dst, int64_t vl, int64_t v0,
                                           int64_t v1, int64_t n0, int64_t n1, int p, HopFlags f,
                                           u32x4* __restrict__ cur_src, u32x4* __restrict__ cur_dst,
                                           u32x4* __restrict__ nxt_src, u32x4* __restrict__ nxt_dst) {
  constexpr bool kDiv = OP == kAvg && ADD;
  constexpr int kLoads = ADD ? 2 * kStageU : kStageU;    // copies per thread per stage
  if (n0 < n1) {
    stage_fill<ADD, NT>(reinterpret_cast<const u32x4*>(src), reinterpret_cast<const u32x4*>(dst),
                        vl, n0, n1, nxt_src, nxt_dst);
    // The current stage has landed once no more than the next stage's copies are
    // outstanding -- but only if this wave issued all kLoads of them.  A short
    // next stage (the slice's last) leaves some waves with fewer or none, and
    // the counter also holds the previous stage's stores, which may complete
    // before the current stage's copies; there, wait for everything.
    if (n1 - n0 == kStageV)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
#pragma unroll
  for (int u = 0; u < kStageU; ++u) {
    const int64_t v = v0 + u * kBlock + threadIdx.x;
    if (v >= vl && v < v1) {
      const int i = u * kBlock + threadIdx.x;
      u32x4 a, y;
      if (ADD)
        lds_read2(cur_src + i, cur_dst + i, a, y);
      else
        a = lds_read(cur_src + i);
      if (ADD) {
        if (kDiv) {
          if (f.div_src) a = vdiv<DT>(a, p);
          if (f.div_dst) y = vdiv<DT>(y, p);
        }
        st16<NT>(dst, v, vcomb<DT, OP>(y, a));
        if (kDiv && f.keep_src) st16<NT>(src, v, a);
      } else {
        st16<NT>(dst, v, a);
      }
    }
  }
}

// One hop over the whole slice [lo, hi), staged through LDS and double-buffered
// ("Ring All-Reduce, in depth", section "What real libraries add", pipelining:
// the next piece is already arriving while this one is reduced and forwarded).
// Stage t holds kStageV vectors of the incoming (src) and the receiving (dst)
// chunk; while stage t is combined out of LDS and stored, stage t+1 is being
// copied into the other LDS buffer by global_load_lds_dwordx4, which lands each
// lane's 16 bytes at the wave's LDS base without passing through registers.
// Every wave reads back only the LDS its own lanes filled, so the stages need
// no workgroup barrier: a wave waits on its own memory counter.  Averages as in
// hop_tile; the slice's unaligned head and tail go element by element.
template <int DT, int OP, bool ADD, bool NT>
__device__ __forceinline__ void hop_slice_lds(void* __restrict__ src, void* __restrict__ dst,
                                              int64_t lo, int64_t hi, int p, HopFlags f,
                                              u32x4 (*stage)[2][kStageV]) {
  typedef Elem<DT> E;
  constexpr int V = E::V;
  constexpr bool kDiv = OP == kAvg && ADD;
  const Span sp = split_span<V>(lo, hi);
  // stages start on lines (Span): stage t is [vb + t*kStageV, ...) within [v0, v1)
  const int64_t nst = sp.v1 > sp.v0 ? (sp.v1 - sp.vb + kStageV - 1) / kStageV : 0;
  auto first = [&](int64_t t) { return sp.vb + t * kStageV; };
  auto last = [&](int64_t t) { return first(t) + kStageV < sp.v1 ? first(t) + kStageV : sp.v1; };
  const int64_t vl = sp.v0;
  if (nst > 0)
    stage_fill<ADD, NT>(reinterpret_cast<const u32x4*>(src), reinterpret_cast<const u32x4*>(dst),
                        vl, first(0), last(0), stage[0][0], stage[0][1]);
  // stages alternate between buffer 0 and 1: two steps per trip so that each
  // step names its current and next buffer explicitly
  for (int64_t t = 0; t < nst; t += 2) {
    stage_step<DT, OP, ADD, NT>(src, dst, vl, first(t), last(t), first(t + 1),
                                t + 1 < nst ? last(t + 1) : first(t + 1), p, f,
                                stage[0][0], stage[0][1], stage[1][0], stage[1][1]);
    if (t + 1 < nst)
      stage_step<DT, OP, ADD, NT>(src, dst, vl, first(t + 1), last(t + 1), first(t + 2),
                                  t + 2 < nst ? last(t + 2) : first(t + 2), p, f,
                                  stage[1][0], stage[1][1], stage[0][0], stage[0][1]);
  }
  const int64_t nh = sp.head_hi - lo, nt = hi - sp.tail_lo;
  const int t = threadIdx.x;
  if (t < nh + nt) {
    const int64_t i = t < nh ? lo + t : sp.tail_lo + (t - nh);
    typename E::S x = ld1<DT>(src, i);
    if (ADD) {
      typename E::S y = ld1<DT>(dst, i);
      if (kDiv) {
        if (f.div_src) x = E::div1(x, p);
        if (f.div_dst) y = E::div1(y, p);
      }
      st1<DT>(dst, i, comb1<DT, OP>(y, x));
      if (kDiv && f.keep_src) st1<DT>(src, i, x);
    } else {
      st1<DT>(dst, i, x);
    }
  }
}


// ================================================================ step by step

// Tiles per workgroup from which a persistent grid's step takes its tiles from
// tile counters (in order) rather than in a fixed stride.
constexpr int64_t kHandOutTiles = 8;

struct StepArgs {
  RankPtrs P;
  ChunkGeo half[2];     // ring: half[0] = whole buffer; bidir: forward, mirrored half
  int64_t T;            // tiles per segment
  int64_t W;            // single-workgroup mode: whole-vector slots per segment
  int64_t n;            // elements per rank (tree segments are whole buffers)
  WsHeader* ws;
  uint64_t* step_ts;
  uint64_t limit;
  int p, mode, step_begin, step_end, levels;
  int channels;         // C: workgroup b serves channel b mod C
  int g, m;             // hier: ranks per node, nodes (half[0] = the g-way intra partition)
  int sync;             // SyncScope of the barriers between steps
  int qn;               // persistent grid: tile counters (workgroup groups) per channel
  int handout;          // persistent grid: the parts fill whole tiles (tile counters may pay)
  int edges;            // one workgroup: some segment has elements outside whole vectors
  uint32_t expect_extra;
  uint32_t stress;      // test hook: delays before arrivals (stress_delay)
};

struct Seg {
  int64_t lo, hi;
  int src, dst;
  bool add;
  HopFlags f;           // averages: which operands are still undivided inputs
};

// Number of segments (independent chunk transfers) in a step.
__device__ __forceinline__ int step_segments(const StepArgs& a, int step) {
  if (a.mode == kModeHier) return a.p;
  if (a.mode == kModeTree) {
    const int k = step < a.levels ? step : 2 * a.levels - 1 - step;
    return (a.p - 1 - (1 << k)) / (2 << k) + 1;
  }
  return a.mode == kModeBidir ? 2 * a.p : a.p;
}

// Segment `seg` of `step`.
//   Ring, direction d (+1 forward, -1 mirrored), chunk c:
//     reduce-scatter step s: sender c + d*s, receiver c + d*(s+1), add
//       (forward: rank r sends chunk r - s to r + 1; mirrored: chunk r + s to r - 1)
//     all-gather step s:     sender c + d*(s-1), receiver c + d*s, copy
//       (forward: rank r sends chunk r + 1 - s; mirrored: chunk r - 1 + s)
//   Tree level k, pair q, r = q * 2^(k+1): reduce adds rank r + 2^k into rank r;
//     broadcast copies rank r over rank r + 2^k; whole buffers.
// Averages: in the ring, the receiver's chunk is always an undivided input and
// the sender's only at step 0 (it leaves its first sender then).  In the tree,
// level 0 reads two inputs; at a later level k the receiver was already a
// receiver at level 0, and the sender r + 2^k (even) was one exactly when it had
// a level-0 partner, r + 2^k + 1 < p.
//   Hier ("Ring All-Reduce, in depth", section "What real libraries add",
//     hierarchy), rank = node * g + local:
//     intra steps: segment = (node, chunk cc of the g-way partition); the node's
//       ring over local ranks, reduce-scatter then (after the inter steps)
//       all-gather, with the ring's rules on local indices;
//     inter steps: segment = (local l, sub-chunk dd of l's shard), the shard
//       being intra chunk (l + 1) mod g, which local rank l owns after the
//       intra reduce-scatter, cut m ways; the ring over nodes on ranks
//       node * g + l, reduce-scatter then all-gather.
//     Averages: every input is divided during the intra reduce-scatter, so
//     the inter steps move divided partials -- unless g = 1, when there is no
//     intra step and the inter ring is the first to read the inputs.
__device__ __forceinline__ Seg hier_segment(const StepArgs& a, int step, int seg) {
  Seg g;
  const int G = a.g, M = a.m;
  const int inter0 = G - 1, ag0 = G - 1 + 2 * (M - 1);
  g.f.div_dst = g.f.div_src = g.f.keep_src = false;
  if (step < inter0 || step >= ag0) {
    const bool rs = step < inter0;
    const int s = rs ? step : step - ag0;
    const int node = seg / G, cc = seg - node * G;
    g.lo = chunk_lo(a.half[0], cc);
    g.hi = chunk_hi(a.half[0], cc);
    const int from = rs ? cc + s : cc + s - 1;
    g.src = node * G + mod_p(from, G);
    g.dst = node * G + mod_p(from + 1, G);
    g.add = rs;
    if (rs) {
      g.f.div_dst = true;
      g.f.div_src = g.f.keep_src = s == 0;
    }
    return g;
  }
  const int s2 = step - inter0;
  const bool rs = s2 < M - 1;
  const int s = rs ? s2 : s2 - (M - 1);
  const int l = seg / M, dd = seg - l * M;
  const int c = l + 1 == G ? 0 : l + 1;
  const int64_t slo = chunk_lo(a.half[0], c), shi = chunk_hi(a.half[0], c);
  const ChunkGeo sg = {slo, (shi - slo) / M, (shi - slo) % M};
  g.lo = chunk_lo(sg, dd);
  g.hi = chunk_hi(sg, dd);
  const int from = rs ? dd + s : dd + s - 1;
  g.src = mod_p(from, M) * G + l;
  g.dst = mod_p(from + 1, M) * G + l;
  g.add = rs;
  if (rs && G == 1) {
    g.f.div_dst = true;
    g.f.div_src = g.f.keep_src = s == 0;
  }
  return g;
}

__device__ __forceinline__ Seg step_segment(const StepArgs& a, int step, int seg) {
  Seg g;
  const int p = a.p;
  if (a.mode == kModeHier) return hier_segment(a, step, seg);
  if (a.mode == kModeTree) {
    const bool reduce = step < a.levels;
    const int k = reduce ? step : 2 * a.levels - 1 - step;
    const int r = seg * (2 << k);
    g.lo = 0;
    g.hi = a.n;
    g.add = reduce;
    g.src = reduce ? r + (1 << k) : r;
    g.dst = reduce ? r : r + (1 << k);
    g.f.div_dst = k == 0;
    g.f.div_src = k == 0 || g.src + 1 >= p;
    g.f.keep_src = false;
    return g;
  }
  const int h = seg >= p ? 1 : 0;
  const int c = seg - h * p;
  const int d = h ? -1 : 1;
  g.lo = chunk_lo(a.half[h], c);
  g.hi = chunk_hi(a.half[h], c);
  if (step < p - 1) {
    const int s = step;
    g.src = mod_p(c + d * s, p);
    g.dst = mod_p(c + d * (s + 1), p);
    g.add = true;
    g.f.div_dst = true;
    g.f.div_src = g.f.keep_src = s == 0;
  } else {
    const int s = step - (p - 1);
    g.src = mod_p(c + d * (s - 1), p);
    g.dst = mod_p(c + d * s, p);
    g.add = false;
    g.f.div_dst = g.f.div_src = g.f.keep_src = false;
  }
  return g;
}

// One step carried out by a single workgroup (kSyncBlock).  Each (segment,
// vector) pair of the step is a work item, so small chunks of many segments are
// served in parallel rather than one tile per segment; a thread takes UB items
// per round and issues all their loads before any store (within a step no
// segment writes what another reads).  The unaligned chunk edges follow, one
// element per thread.  Rank indices differ from lane to lane here; the caller
// passes the pointer table as an LDS copy.
template <int DT, int OP, bool NT>
__device__ __forceinline__ void block_step(const StepArgs& a, const RankPtrs& P, int step) {
  typedef Elem<DT> E;
  constexpr int V = E::V;
  constexpr int UB = 4;
  constexpr int E2 = 2 * (V - 1);           // edge elements a segment can have
  const int p = a.p;
  const int W = (int)a.W;                   // small: every index fits 32 bits
  const int nseg = step_segments(a, step);
  const int total = nseg * W;
  for (int f0 = 0; f0 < total; f0 += kBlock * UB) {
    Seg g[UB];
    int64_t v[UB];
    bool on[UB];
    u32x4 x[UB], y[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int f = f0 + u * kBlock + (int)threadIdx.x;
      on[u] = false;
      if (f < total) {
        const int seg = f / W;
        g[u] = step_segment(a, step, seg);
        const Span sp = split_span<V>(g[u].lo, g[u].hi);
        v[u] = sp.v0 + (f - seg * W);
        if (v[u] < sp.v1) {
          on[u] = true;
          x[u] = ld16<NT>(P.b[g[u].src], v[u]);
          if (g[u].add) y[u] = ld16<NT>(P.b[g[u].dst], v[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (!on[u]) continue;
      u32x4 o = x[u];
      if (g[u].add) {
        u32x4 xs = x[u], yd = y[u];
        if (OP == kAvg) {
          if (g[u].f.div_src) xs = vdiv<DT>(xs, p);
          if (g[u].f.div_dst) yd = vdiv<DT>(yd, p);
          if (g[u].f.keep_src) st16<NT>(P.b[g[u].src], v[u], xs);
        }
        o = vcomb<DT, OP>(yd, xs);
      }
      st16<NT>(P.b[g[u].dst], v[u], o);
    }
  }
  // edge elements: only when some segment has them.  With every chunk on whole
  // vectors, working out the geometry of p*E2 empty items was most of a step's
  // time on one workgroup (one wave per SIMD, nothing to hide latency behind):
  // p = 64 with 1 KiB per rank took 2.6 us per step with it and 1.0 without.
  // (Copying all ranks into LDS and running the steps there gained nothing:
  // the plain pointer accesses reach LDS through the vector-memory path.)
  const int etotal = a.edges ? nseg * E2 : 0;
  for (int f = (int)threadIdx.x; f < etotal; f += kBlock) {
    const int seg = f / E2;
    const int e = f - seg * E2;
    const Seg g = step_segment(a, step, seg);
    const Span sp = split_span<V>(g.lo, g.hi);
    const int64_t nh = sp.head_hi - g.lo, nt = g.hi - sp.tail_lo;
    if (e >= nh + nt) continue;
    const int64_t i = e < nh ? g.lo + e : sp.tail_lo + (e - nh);
    typename E::S xv = ld1<DT>(P.b[g.src], i);
    if (g.add) {
      typename E::S yv = ld1<DT>(P.b[g.dst], i);
      if (OP == kAvg) {
        if (g.f.div_src) xv = E::div1(xv, p);
        if (g.f.div_dst) yv = E::div1(yv, p);
        if (g.f.keep_src) st1<DT>(P.b[g.src], i, xv);
      }
      st1<DT>(P.b[g.dst], i, comb1<DT, OP>(yv, xv));
    } else {
      st1<DT>(P.b[g.dst], i, xv);
    }
  }
}

// Channels ("Ring All-Reduce, in depth", section "What real libraries add":
// a collective split across channels, each its own ring): channel h takes part h
// of every segment -- part h of [lo, hi) split C ways starts at
// lo + h*floor(len/C) + min(h, len mod C) -- and its workgroups wait only for
// each other between steps.  Every element still takes the same hops in the same
// order, so the result does not depend on C; C = 1 is the plain step-by-step ring.
template <int DT, int OP, int U, bool NT, int BS>
__global__ __launch_bounds__(BS) void k_steps(StepArgs a) {
  if (ws_failed(a.ws)) return;
  if (a.step_ts && blockIdx.x == 0 && threadIdx.x == 0) a.step_ts[0] = now_ticks();
  if constexpr (BS == kBlock) if (a.sync == kSyncBlock) {
    // one workgroup: its own barrier (with workgroup-scope release and acquire,
    // enough for threads of one CU) separates the steps.  The rank pointers,
    // indexed per lane here, are read from a copy in LDS.
    __shared__ RankPtrs lp;
    if (threadIdx.x < (unsigned)a.p) lp.b[threadIdx.x] = a.P.b[threadIdx.x];
    __syncthreads();
    for (int step = a.step_begin; step < a.step_end; ++step) {
      block_step<DT, OP, NT>(a, lp, step);
      __syncthreads();
      if (a.step_ts && threadIdx.x == 0) a.step_ts[step - a.step_begin + 1] = now_ticks();
    }
    return;
  }
  const int C = a.channels;
  const int h = (int)(blockIdx.x % (uint32_t)C);
  const uint32_t nbh = (gridDim.x - (uint32_t)h + (uint32_t)C - 1u) / (uint32_t)C;
  const int64_t b = blockIdx.x / (uint32_t)C;       // index within the channel
  uint32_t* bar = a.ws->bar[h];
  const bool leader = b == 0;
  uint32_t extra = a.expect_extra;
  // Steps with at least kHandOutTiles tiles per workgroup, on parts that fill
  // whole tiles (a.handout), hand their tiles out in order from tile counters,
  // one tile per grab.  The channel's workgroups
  // form qn groups (group x = b mod qn; with one channel, group x is XCD x,
  // since workgroup b runs on XCD b mod 8), and group x takes a contiguous range
  // of the step's tiles, sized to its share of the channel's workgroups, from a
  // counter of its own.  Measured at p = 8 with 16 GB per rank: a resident grid
  // whose workgroups walk fixed strided tiles takes 95.6 ms, the same grid with
  // in-order ranges per XCD 88.8 (one launch per step: 88.3); tiles of one
  // counter interleaved over the XCDs gained nothing, and one counter for the
  // whole grid doubled the time (its atomics serialise).  The host zeroes the
  // counters before a launch that has such a step; the step advances counter x
  // by its range's length plus one failing grab per workgroup of the group, so
  // every workgroup knows the next step's base without reading it (the barrier
  // between steps orders the grabs).  Smaller steps keep fixed strided tiles
  // (workgroup b: tiles b, b + nbh, ...): there a grab's round trip costs more
  // than the imbalance it removes (p = 9, 4 MB per rank: 0.121 against 0.095 ms
  // with eight channels).  (Taking the next tile before moving the current one,
  // to overlap the atomic with the loads, measured 1% slower.)
  const int qn = a.qn;
  const int xq = (int)(b % qn);
  const int64_t per = nbh / qn, more = nbh % qn;
  const int64_t w0 = xq * per + (xq < more ? xq : more);       // workgroups of groups < x
  const int64_t wq = per + (xq < more ? 1 : 0);               // workgroups of group x
  uint32_t* ctr = a.ws->tiles[h * qn + xq];
  uint32_t base = 0;
  __shared__ uint32_t grab;
  for (int step = a.step_begin; step < a.step_end; ++step) {
    const int64_t ntiles = (int64_t)step_segments(a, step) * a.T;
    auto move = [&](int64_t t) {
      const int seg = (int)(t / a.T);
      const int64_t j = t - (int64_t)seg * a.T;
      const Seg g = step_segment(a, step, seg);
      const int64_t len = g.hi - g.lo, q = len / C, rem = len % C;
      const int64_t lo = g.lo + h * q + (h < rem ? h : rem);
      const int64_t hi = lo + q + (h < rem ? 1 : 0);
      if (g.add)
        hop_tile<DT, OP, U, true, NT, BS>(a.P.b[g.src], a.P.b[g.dst], lo, hi, j, a.p, g.f);
      else
        hop_tile<DT, OP, U, false, NT, BS>(a.P.b[g.src], a.P.b[g.dst], lo, hi, j, a.p, g.f);
    };
    if (!a.handout || ntiles < kHandOutTiles * (int64_t)nbh) {
      for (int64_t t = b; t < ntiles; t += nbh) move(t);
    } else {
      const int64_t t0 = ntiles * w0 / nbh, t1 = ntiles * (w0 + wq) / nbh;
      for (;;) {
        if (threadIdx.x == 0)
          grab = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base;
        __syncthreads();
        const int64_t t = t0 + grab;
        __syncthreads();              // every thread has read the grab
        if (t >= t1) break;
        move(t);
      }
      base += (uint32_t)(t1 - t0 + wq);
    }
    const bool last = step + 1 == a.step_end;
    if (!last || a.step_ts || extra) {
      stress_delay(a.stress, (uint32_t)step);
      bool ok;
      if (a.sync == kSyncXcdGroups)
        ok = xcd_barrier(a.ws, bar, extra, a.limit);
      else if (a.sync == kSyncOneXcd)
        ok = xcd_local_barrier(a.ws, bar, leader, nbh, extra, a.limit);
      else
        ok = grid_barrier(a.ws, bar, leader, nbh, extra, a.limit);
      if (!ok) return;
      extra = 0;
      if (a.step_ts && blockIdx.x == 0 && threadIdx.x == 0)
        a.step_ts[step - a.step_begin + 1] = now_ticks();
    }
  }
}


// One step as a launch of its own: tile t = (segment, tile j of the segment),
// U 16-byte vectors per thread, as many workgroups as tiles.  The stream orders
// consecutive launches, so the kernel boundary is the step's barrier.  On
// MI355X a grid that covers the data once streams about a fifth faster than a
// resident grid looping over it (16 GiB copy: 6.47 TB/s against 5.0-5.3 TB/s;
// in-place add: 6.44 against 4.8-5.4 TB/s), and back-to-back launches on one
// stream cost about 3 us each, less than the resident grid's device-wide barrier
// (4-5 us).  Tile indices stay below 2^32 (a tile holds at least 4 KiB, and
// the launcher checks), so the tile's segment is found by a 32-bit division,
// which is several times shorter than a 64-bit one.
template <int DT, int OP, bool NT, int U>
__global__ __launch_bounds__(kBlock) void k_step(StepArgs a, int step, uint32_t T, uint32_t ntiles) {
  for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int seg = (int)(t / T);
    const int64_t j = (int64_t)(t - (uint32_t)seg * T);
    const Seg g = step_segment(a, step, seg);
    if (g.add)
      hop_tile<DT, OP, U, true, NT>(a.P.b[g.src], a.P.b[g.dst], g.lo, g.hi, j, a.p, g.f);
    else
      hop_tile<DT, OP, U, false, NT>(a.P.b[g.src], a.P.b[g.dst], g.lo, g.hi, j, a.p, g.f);
    if (t > 0xFFFFFFFFu - gridDim.x) break;   // the next t would wrap
  }
}

// ================================================================ pipelined

struct PipeArgs {
  RankPtrs P;
  ChunkGeo g;
  int64_t slice;        // elements per slice (multiple of the vector width)
  int64_t kmax;         // flag entries per chunk
  uint32_t* flags;      // flags[c * kmax + k]: hops finished on slice k of chunk c, + base
  WsHeader* ws;
  uint64_t limit;
  int p, workers, hop_begin, hop_end;
  uint32_t base, expect_extra;
  uint32_t stress;      // test hook: delays before slice hops (stress_delay)
};

// Slices of chunk [lo, hi): slice 0 starts at lo, later slices start at
// A + k*slice with A = lo rounded up to a whole 128-byte line (kLineVecs
// vectors), the last ends at hi.  The slice length is a whole number of lines
// too, so every slice after the first -- and every LDS stage in it -- starts on
// a line.  A slice starting mid-line (measured with 3,906,256-byte slices, 80
// bytes past a line) makes every 1 KiB wave access touch 9 lines instead of 8,
// and the line two accesses share was fetched twice or written back in two
// partial pieces: 7.9% more reads and 2.3% more writes than the schedule needs.
__host__ __device__ __forceinline__ int64_t slice_origin(int64_t lo, int V) {
  const int64_t L = (int64_t)V * kLineVecs;
  return (lo + L - 1) / L * L;
}
template <int V>
__device__ __forceinline__ int64_t n_slices(int64_t lo, int64_t hi, int64_t slice) {
  const int64_t A = slice_origin(lo, V);
  if (A >= hi) return 1;
  const int64_t k = (hi - A + slice - 1) / slice;
  return k < 1 ? 1 : k;
}

// Workgroup (d, w) = block d * W + w plays rank d: for each hop h it receives chunk c from rank
// d-1 (reduce-scatter hop s: c = d-1-s, add; all-gather hop s: c = d-s, copy),
// slice by slice (slices k = w, w + W, ...).  Slice k of chunk c may take hop h
// once its counter says hops 0..h-1 are done, i.e. once rank d-1 has finished
// with it; afterwards the counter is advanced for rank d+1.  Every dependency
// points to an earlier hop of the same slice, handled by workgroup (d-1, w), and
// every workgroup takes its hops in increasing order, so with all workgroups
// resident the chain always progresses.  When W is a multiple of 8, workgroups
// (d, w) of every rank d sit on XCD w mod 8, so each slice lives in one XCD's L2
// and publishing a slice needs no L2 write-back (LOCAL).
template <int DT, int OP, int U, bool NT, bool LOCAL>
__global__ __launch_bounds__(kBlock) void k_pipelined(PipeArgs a) {
  typedef Elem<DT> E;
  constexpr int V = E::V;
  __shared__ u32x4 stage[2][2][kStageV];                   // 32 KiB: 2 stages x (src, dst)
  if (ws_failed(a.ws)) return;
  const int p = a.p;
  const int d = blockIdx.x / a.workers;
  const int w = blockIdx.x - d * a.workers;
  const int left = d == 0 ? p - 1 : d - 1;
  void* src = a.P.b[left];
  void* dst = a.P.b[d];
  uint32_t extra = a.expect_extra;
  for (int h = a.hop_begin; h < a.hop_end; ++h) {
    const bool rs = h < p - 1;
    const int s = rs ? h : h - (p - 1);
    const int c = mod_p(rs ? d - 1 - s : d - s, p);
    const int64_t lo = chunk_lo(a.g, c), hi = chunk_hi(a.g, c);
    const int64_t K = n_slices<V>(lo, hi, a.slice);
    const int64_t A = slice_origin(lo, V);
    const uint32_t done = a.base + (uint32_t)(h - a.hop_begin);
    for (int64_t k = w; k < K; k += a.workers) {
      uint32_t* f = a.flags + (int64_t)c * a.kmax + k;
      // the first hop reads untouched inputs and depends on nothing; counters
      // left by earlier calls are all below `base`, so it must not wait
      stress_delay(a.stress, (uint32_t)(h * 4096 + k));
      if (h > a.hop_begin || extra) {
        if (!wait_flag(a.ws, f, done + extra, a.limit)) return;
        extra = 0;
      }
      const int64_t slo = k == 0 ? lo : A + k * a.slice;
      const int64_t shi = k == K - 1 ? hi : A + (k + 1) * a.slice;
      // averages: the receiver's chunk is always an input, the sender's only
      // at the first hop (see step_segment)
      HopFlags hf;
      hf.div_dst = rs;
      hf.div_src = hf.keep_src = rs && s == 0;
      if (rs)
        hop_slice_lds<DT, OP, true, NT>(src, dst, slo, shi, p, hf, stage);
      else
        hop_slice_lds<DT, OP, false, NT>(src, dst, slo, shi, p, hf, stage);
      post_flag<LOCAL>(f, done + 1);
    }
  }
}


// ================================================================ launchers

static hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) { *cus = it->second; return hipSuccess; }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) cache[dev] = *cus;
  return e;
}

// ---------------------------------------------------------------- placement

// Reads the XCC_ID hardware register: the XCD this workgroup runs on.
__global__ void k_xcc_probe(uint32_t* out) {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  if (threadIdx.x == 0) out[blockIdx.x] = v & 0xfu;
}

// Whether the dispatcher puts workgroup b on XCD b mod 8 on the current device:
// checked once per device with 1024 one-wave workgroups (every b must share the
// XCD of b mod 8, and blocks 0..7 must cover 8 distinct XCDs).  The two-level
// and XCD-local synchronisation rely on it; without it everything stays on the
// device-wide barrier.
static hipError_t xcd_placement(bool* ok, bool may_probe) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::unordered_map<int, bool> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) { *ok = it->second; return hipSuccess; }
  if (!may_probe) {         // the probe needs a device buffer: without it, assume nothing
    *ok = false;
    return hipSuccess;
  }
  constexpr int kProbe = 1024;
  uint32_t* d = nullptr;
  e = hipMalloc(&d, kProbe * sizeof(uint32_t));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_xcc_probe, dim3(kProbe), dim3(64), 0, 0, d);
  e = hipGetLastError();
  uint32_t h[kProbe];
  if (e == hipSuccess) e = hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost);
  (void)hipFree(d);
  if (e != hipSuccess) return e;
  bool good = true;
  uint32_t seen = 0;
  for (int b = 0; b < kXcds; ++b) {
    if (h[b] >= 32 || (seen >> h[b] & 1u)) good = false;
    else seen |= 1u << h[b];
  }
  for (int b = kXcds; b < kProbe && good; ++b) good = h[b] == h[b % kXcds];
  cache[dev] = good;
  *ok = good;
  return hipSuccess;
}

// Persistent grids (the step kernels' device-wide barriers, the flag-driven
// pipelined ring) are ordinary launches: nothing in them uses the runtime's
// grid-wide synchronisation, so all they need is that every workgroup be
// resident at once, and every wait in them is bounded (a grid that cannot
// become resident -- another persistent grid holds the rest of the GPU -- ends
// with RA_ERR_TIMEOUT instead of hanging).  The grid is therefore sized here
// from what one CU can hold of the kernel:
//  * the occupancy query, which accounts for vector registers and LDS, but not
//    for the scalar-register file (measured: 2043 workgroups of a kernel the
//    query rated at 8 per CU stalled, 576 did not);
//  * the scalar-register bound: a gfx9 SIMD holds 800 SGPRs and a wave's
//    allocation is at most 112 (the 102 addressable, VCC and the trap and
//    flat-scratch registers, in granules of 16), so at least 7 waves per SIMD
//    always fit -- 7 workgroups of 256 threads (one wave per SIMD each) per CU,
//    3 of 512, 1 of 1024.
// The kernels' actual use is below that (compiler resource report: at most
// 106 SGPRs and 117 VGPRs per wave among the persistent kernels).
static constexpr int kSgprWavesPerSimd = 7;
// Of the resident maximum, the grid a persistent step kernel of 256-thread
// workgroups takes by default: 3 per CU (the shape of large buffers and of
// every caller-sized grid; smaller buffers take larger workgroups, see
// persistent_shape).  Fewer workgroups each take more tiles, and a barrier
// costs more the more workgroups wait at it.  Measured on MI355X with the
// tiles handed out in order, ms per all-reduce at 2 / 3 / 4 / 5 per CU (bf16
// unless noted): ring at 8 x 16 GB 93.4 / 86.9 / 87.6 / 87.6 (one launch per
// step: 87.2); 8 x 1 GiB 12.7 / 12.1 / 12.5 / 12.6; 8 x 64 MiB float32 1.70 /
// 1.63 / 1.68 / 1.68; 8 x 16 MiB 0.253 / 0.271 / 0.289 / 0.289; channels at
// 8 x 16 GB 93.6 / 88.2 / 89.5 / 89.6.  (Before the in-order hand-out, 5 per CU
// was best: 103.3 ms with 4, 97.3 with 5, 98.7 with 6.)  A caller's
// ra_options.grid may ask for up to the resident maximum.
static constexpr int kPersistentPerCU = 3;
// The flag-driven pipelined kernel's default budget of workgroups, and the
// worker count its default slice length is sized for: 5 per CU, of which its
// 32 KiB of LDS per workgroup lets 4 be resident.
static constexpr int kPipelinedPerCU = 5;

// Workgroups of `func` that can be resident at once on the current device.
// Workgroups of `func` (`threads` each) that can be resident at once on the
// current device.
static hipError_t resident_blocks(const void* func, int* out, int threads = kBlock) {
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, func, threads, 0);
  if (e != hipSuccess) return e;
  *out = std::max(1, std::min(per_cu, kSgprWavesPerSimd * kBlock / threads)) * cus;
  return hipSuccess;
}

// Shape of a persistent step grid that the library sizes itself (no
// ra_options.grid): threads per workgroup and workgroups per CU, by bytes per
// rank.  A barrier's cost grows with the workgroups that wait at it (each one
// invalidates its XCD's L2 on the way out), so where a step moves little, the
// same threads in fewer, larger workgroups win; where steps are large, 256
// threads x 3 per CU stream best.  Measured on MI355X, bf16, ms per all-reduce
// at 256 x 3 / 512 x 2 / 1024 x 1 (channels chosen automatically):
//   p = 8:  4 MiB per rank 0.069 / 0.063 / 0.076; 16 MiB 0.239 / 0.164 / 0.117;
//           256 MiB 1.587 / 1.597 / 1.560; 1 GiB 6.02 / 6.20 / 6.08;
//   p = 16: 8 MiB 0.232 / 0.160 / 0.161; 16 MiB 0.504 / 0.336 / 0.227;
//           256 MiB 3.37 / 3.39 / 3.30; 512 MiB 6.50 / 6.64 / 6.61;
//   p = 64: 8 MiB 1.27 / 0.94 / 1.02; 64 MiB 4.52 / 4.22 / 4.13;
//           128 MiB 7.70 / 7.52 / 8.45;
//   p = 4 to 64 at 2 MiB per rank: 256 x 3 best or within 1%.
struct GridShape {
  int threads, per_cu;
};
static GridShape persistent_shape(int64_t rank_bytes, int p) {
  constexpr int64_t kMiB = 1ll << 20;
  if (rank_bytes >= 4 * kMiB && rank_bytes < 16 * kMiB) return {512, 2};
  if (rank_bytes >= 16 * kMiB && rank_bytes <= (p > 16 ? 64 : 256) * kMiB) return {1024, 1};
  return {kBlock, kPersistentPerCU};
}

int default_persistent_workgroups() {
  int cus = 0;
  if (device_cus(&cus) != hipSuccess || cus <= 0) return 0;
  return kPersistentPerCU * cus;
}


// Step-by-step kernels run on a persistent grid of a few workgroups per CU (see
// kPersistentPerCU), so each thread keeps more bytes in flight: measured at
// 8 x 16 GB bf16, four vectors per thread ran 103.8 ms against 107.3 with two.
static constexpr int kStepU = 4;

// Channels chosen when the caller leaves the count open: one per XCD.
static constexpr int kAutoChannels = 8;

// Smallest grid that synchronises through the two-level barrier.
static constexpr int kTwoLevelMinGrid = 128;
// Steps with at most this many whole vectors (4 KiB) across all their segments
// run on a single workgroup; larger ones one launch per step.  Measured on
// MI355X, bf16 ring, GPU time per all-reduce: p = 8 at 1 KiB per rank 24.5 us
// on one workgroup against 40.1 with a launch per step, p = 64 331 against 375;
// with the bound at 1024 vectors, p = 8 at 16 KiB took 54 us against 41 and
// p = 64 600 against 335.
static constexpr int64_t kBlockModeVecs = 256;
static constexpr int kPipeU = 4;
// Copy steps (all-gather, tree broadcast) whose widest segment holds at least
// this many vectors launch with two vectors per thread, reductions with one.
// Measured on MI355X, one launch per step, 8 x 16 GB bf16: all-gather phase
// 34.9 ms with two vectors against 43.7 with one; reduce-scatter phase 55.5
// against 50.4.  At 8 x 256 MiB fp32: all-gather 0.58 against 0.76 ms.  With
// 1024 vectors per segment (p = 64, 1 MiB per rank) two were 13% slower.
static constexpr int64_t kCopyU2Vecs = 8192;

// Whether step st of a schedule copies (all-gather, broadcast) rather than
// reduces; the same rule step_segment applies on the device.
static bool step_copies(StepMode mode, int st, int p, int levels, int g, int m) {
  if (mode == kModeTree) return st >= levels;
  if (mode == kModeHier) {
    const int inter0 = g - 1, ag0 = g - 1 + 2 * (m - 1);
    if (st >= ag0) return true;
    return st >= inter0 && st - inter0 >= m - 1;
  }
  return st >= p - 1;
}

// The step kernel with `threads` threads per workgroup (256, 512 or 1024).
template <int DT, int OP>
static const void* steps_kernel(bool nt, int threads) {
  if (threads == 1024)
    return nt ? reinterpret_cast<const void*>(&k_steps<DT, OP, kStepU, true, 1024>)
              : reinterpret_cast<const void*>(&k_steps<DT, OP, kStepU, false, 1024>);
  if (threads == 512)
    return nt ? reinterpret_cast<const void*>(&k_steps<DT, OP, kStepU, true, 512>)
              : reinterpret_cast<const void*>(&k_steps<DT, OP, kStepU, false, 512>);
  return nt ? reinterpret_cast<const void*>(&k_steps<DT, OP, kStepU, true, kBlock>)
            : reinterpret_cast<const void*>(&k_steps<DT, OP, kStepU, false, kBlock>);
}

template <int DT, int OP>
static hipError_t steps_dt(const RankPtrs& P, int p, int64_t n, StepMode mode, int step_begin,
                           int step_end, const SyncCfg& sc, hipStream_t s, int* grid_used,
                           int* launches) {
  const int V = Elem<DT>::V;
  StepArgs a;
  a.P = P;
  a.n = n;
  a.ws = sc.ws;
  a.step_ts = sc.step_ts;
  a.limit = sc.limit_ticks;
  a.p = p;
  a.mode = mode;
  a.step_begin = step_begin;
  a.step_end = step_end;
  a.expect_extra = sc.expect_extra;
  a.stress = sc.stress;
  a.channels = 1;
  a.g = sc.group > 0 ? sc.group : p;
  a.m = p / a.g;
  a.levels = 0;
  while ((1 << a.levels) < p) ++a.levels;
  // segment geometry and the widest segment in vectors
  // every element range a step may work on (chunks of the ring's halves, whole
  // buffers for the tree, intra chunks and their inter pieces for the hierarchy)
  // (enumerated on demand, not stored: a call allocates no host memory either)
  int64_t hier_intra = 0, hier_inter = 0;   // hier: widest in-node chunk, widest cross-node piece
  const int64_t len0 = mode == kModeBidir ? (n + 1) / 2 : n;
  if (mode == kModeHier) {
    a.half[0] = a.half[1] = make_geo(0, n, a.g);
  } else if (mode == kModeTree) {
    a.half[0] = a.half[1] = make_geo(0, n, p);
  } else {
    a.half[0] = make_geo(0, len0, p);
    a.half[1] = make_geo(len0, n - len0, p);
  }
  auto for_each_range = [&](auto fn) {
    if (mode == kModeHier) {
      for (int c = 0; c < a.g; ++c) {
        const int64_t lo = host_chunk_lo(0, n, a.g, c), hi = host_chunk_lo(0, n, a.g, c + 1);
        fn(lo, hi);
        for (int d = 0; d < a.m; ++d)
          fn(host_chunk_lo(lo, hi - lo, a.m, d), host_chunk_lo(lo, hi - lo, a.m, d + 1));
      }
    } else if (mode == kModeTree) {
      fn((int64_t)0, n);
    } else {
      const int nh = mode == kModeBidir ? 2 : 1;
      for (int h = 0; h < nh; ++h) {
        const int64_t off = h ? len0 : 0, len = h ? n - len0 : len0;
        for (int c = 0; c < p; ++c) fn(host_chunk_lo(off, len, p, c), host_chunk_lo(off, len, p, c + 1));
      }
    }
  };
  if (mode == kModeHier) {
    for (int c = 0; c < a.g; ++c) {
      const int64_t lo = host_chunk_lo(0, n, a.g, c), hi = host_chunk_lo(0, n, a.g, c + 1);
      hier_intra = std::max(hier_intra, tiled_vecs_in(lo, hi, V));
      for (int d = 0; d < a.m; ++d)
        hier_inter = std::max(hier_inter, tiled_vecs_in(host_chunk_lo(lo, hi - lo, a.m, d),
                                                        host_chunk_lo(lo, hi - lo, a.m, d + 1), V));
    }
  }
  // whole vectors of the widest part of any range cut C ways (the kernel's rule:
  // part h of [lo, hi) starts at lo + h*floor(len/C) + min(h, len mod C)); tiled:
  // counted from the line its first tile starts on, what the tile count needs
  auto widest = [&](int C, bool tiled) {
    int64_t w = 0;
    for_each_range([&](int64_t first, int64_t last) {
      const int64_t len = last - first, q = len / C, rem = len % C;
      for (int h = 0; h < C; ++h) {
        const int64_t lo = first + h * q + std::min<int64_t>(h, rem), hi = lo + q + (h < rem ? 1 : 0);
        w = std::max(w, tiled ? tiled_vecs_in(lo, hi, V) : vecs_in(lo, hi, V));
      }
    });
    return w;
  };
  const int64_t maxvec = widest(1, false), maxtiled = widest(1, true);
  a.handout = 0;
  a.edges = 0;
  for_each_range([&](int64_t lo, int64_t hi) {
    if (hi > lo && (lo % V != 0 || hi % V != 0 || vecs_in(lo, hi, V) == 0)) a.edges = 1;
  });
  // segments (independent chunk transfers) of step st, as step_segments counts them
  auto nseg_of = [&](int st) {
    if (mode == kModeHier) return p;
    if (mode == kModeTree) {
      const int k = st < a.levels ? st : 2 * a.levels - 1 - st;
      return (p - 1 - (1 << k)) / (2 << k) + 1;
    }
    return mode == kModeBidir ? 2 * p : p;
  };
  int most_seg = 0;
  for (int st = step_begin; st < step_end; ++st) most_seg = std::max(most_seg, nseg_of(st));
  // How the steps are separated.  Test hooks that need device waits (forced
  // timeout, stress delays) always get the persistent grid and its barriers.
  //  * block: steps that move at most kBlockModeVecs vectors run on a single
  //    workgroup of k_steps, its own barrier between steps;
  //  * launch: otherwise one launch per step (k_step), unless the caller asks
  //    for a grid, for channels (RING_CHANNELS) or for step timestamps.
  //    Measured against the persistent grid on MI355X (bf16, GPU time per
  //    all-reduce): ring p = 8 at 16 MiB per rank 0.149 ms against 0.227, at
  //    2 GiB 13.0 against 13.4; p = 64 at 1 MiB 0.40 against 0.62; tree p = 8
  //    at 2 GiB 11.7 against 13.9 ms;
  //  * the persistent grid with device-wide barriers in every other case.
  const bool hooks_free = sc.expect_extra == 0 && sc.stress == 0;
  const int64_t step_vecs = (int64_t)most_seg * maxvec;
  const bool block_ok = step_vecs <= kBlockModeVecs && (sc.grid == 0 || sc.grid == 1) &&
                        sc.channels <= 1 && hooks_free;
  const bool launch_ok = !block_ok && sc.grid == 0 && sc.channels == 1 && hooks_free &&
                         sc.step_ts == nullptr;
  if (launch_ok) {
    a.channels = 1;
    a.T = 0;
    a.sync = kSyncDevice;
    a.W = 0;
    int widest_grid = 0;
    const bool nt = streaming(p, n, DT);
    for (int st = step_begin; st < step_end; ++st) {
      // tiles per segment for this step's widest segment (the hierarchy's
      // cross-node steps move pieces m times smaller than its in-node steps)
      int64_t w = maxtiled;
      if (mode == kModeHier)
        w = st < a.g - 1 || st >= a.g - 1 + 2 * (a.m - 1) ? hier_intra : hier_inter;
      const bool two = w >= kCopyU2Vecs && step_copies(mode, st, p, a.levels, a.g, a.m);
      const int64_t tv = two ? 2 * kBlock : kBlock;
      const int64_t T = std::max<int64_t>(1, (w + tv - 1) / tv);
      const int64_t ntiles = (int64_t)nseg_of(st) * T;
      if (ntiles > 0xFFFFFFFFll) return hipErrorInvalidValue;
      const int g = (int)std::min<int64_t>(ntiles, kMaxGrid);
      widest_grid = std::max(widest_grid, g);
      const uint32_t T32 = (uint32_t)T, n32 = (uint32_t)ntiles;
      if (nt && two)
        hipLaunchKernelGGL((k_step<DT, OP, true, 2>), dim3(g), dim3(kBlock), 0, s, a, st, T32, n32);
      else if (nt)
        hipLaunchKernelGGL((k_step<DT, OP, true, 1>), dim3(g), dim3(kBlock), 0, s, a, st, T32, n32);
      else if (two)
        hipLaunchKernelGGL((k_step<DT, OP, false, 2>), dim3(g), dim3(kBlock), 0, s, a, st, T32, n32);
      else
        hipLaunchKernelGGL((k_step<DT, OP, false, 1>), dim3(g), dim3(kBlock), 0, s, a, st, T32, n32);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    *grid_used = widest_grid;
    *launches = step_end - step_begin;
    return hipSuccess;
  }
  const bool nt = streaming(p, n, DT);
  void* args[] = {&a};
  // Small steps run on one workgroup with its own barrier between steps: a
  // device-wide barrier costs microseconds (L2 write-back, atomics across XCDs,
  // L2 invalidate), a workgroup barrier well under one.  One workgroup is
  // resident by itself.
  if (block_ok) {
    a.sync = kSyncBlock;
    a.channels = 1;
    a.T = 1;
    a.W = std::max<int64_t>(1, maxvec);
    *grid_used = 1;
    *launches = 1;
    return hipLaunchKernel(steps_kernel<DT, OP>(nt, kBlock), dim3(1), dim3(kBlock), args, 0, s);
  }
  // the persistent grid's barriers live in the stream's workspace
  if (sc.ws == nullptr) return hipErrorInvalidValue;
  // a caller's grid counts workgroups of 256 threads
  const GridShape shape = sc.grid > 0 ? GridShape{kBlock, kPersistentPerCU}
                                      : persistent_shape(n * elem_bytes(DT), p);
  const void* func = steps_kernel<DT, OP>(nt, shape.threads);
  int resident = 0, cus = 0;
  hipError_t e = resident_blocks(func, &resident, shape.threads);
  if (e != hipSuccess) return e;
  e = device_cus(&cus);
  if (e != hipSuccess) return e;
  int grid = std::min(resident, sc.grid > 0 ? sc.grid : shape.per_cu * cus);
  const int64_t tv = (int64_t)shape.threads * kStepU;
  // no more workgroups than whole-segment tiles: on small buffers every extra
  // workgroup only adds to each barrier's cost
  const int64_t most = (int64_t)most_seg * std::max<int64_t>(1, (maxtiled + tv - 1) / tv);
  grid = (int)std::max<int64_t>(1, std::min<int64_t>(grid, most));
  // channels share that grid, the same number of workgroups each, at least one.
  // Unspecified (0): 8, one per XCD (each channel then lives in one XCD's L2 and
  // its barrier needs no write-back), when that still gives every segment of a
  // channel a workgroup of its own; otherwise 1 -- on small buffers a channel's
  // workgroups would walk segments one after another
  int want = sc.channels;
  if (want == 0) want = grid / std::max(1, most_seg) >= kAutoChannels ? kAutoChannels : 1;
  a.channels = std::max(1, std::min(std::min(want, kMaxChannels), grid));
  grid = grid / a.channels * a.channels;
  bool placed = false;
  e = xcd_placement(&placed, sc.may_probe);
  if (e != hipSuccess) return e;
  // the two-level barrier pays from about 128 workgroups (measured: 4.2 against
  // 10 us at 256, 2.8 against 2.5 us at 64)
  a.sync = !placed ? kSyncDevice
           : a.channels == 1 ? (grid >= kTwoLevelMinGrid ? kSyncXcdGroups : kSyncDevice)
           : a.channels % kXcds == 0 ? kSyncOneXcd : kSyncDevice;
  a.T = std::max<int64_t>(1, (widest(a.channels, true) + tv - 1) / tv);
  a.W = std::max<int64_t>(1, maxvec);
  // tile counters per channel: one per XCD that the channel's workgroups run on
  // (workgroup b*C + h on XCD (b*C + h) mod 8: 8 / gcd(C, 8) of them, taken in
  // turn, so group b mod qn is one XCD), fewer when a channel has fewer
  // workgroups (each group needs one) or the header's 64 counters would not hold
  // them.  More groups than XCDs only split an XCD's tiles into more streams:
  // eight channels with eight counters each took 92.5 ms at p = 8, 16 GB per
  // rank, against 89.7 with one each.
  const int spans = kXcds / std::gcd(a.channels, kXcds);
  a.qn = std::max(1, std::min(std::min(spans, grid / a.channels), kMaxChannels / a.channels));
  // counters only where the channel's parts fill whole tiles: with a part of a
  // few hundred bytes the tiles are nearly empty, and a grab costs more than
  // the part (p = 64 with 1 KiB per rank, 8 channels: 11.9 us per step with
  // the counters, 8 without)
  a.handout = widest(a.channels, true) >= tv ? 1 : 0;
  bool hand_out = false;
  for (int st = step_begin; st < step_end; ++st)
    hand_out = hand_out || (int64_t)nseg_of(st) * a.T >= kHandOutTiles * (grid / a.channels);
  hand_out = hand_out && a.handout;
  if (hand_out) {
    e = launch_fill_u32(&sc.ws->tiles[0][0], 0u, (int64_t)a.channels * a.qn * 32, s);
    if (e != hipSuccess) return e;
  }
  *grid_used = grid;
  *launches = 1;
  return hipLaunchKernel(func, dim3(grid), dim3(shape.threads), args, 0, s);
}

// (dtype, op) pairs that exist: avg needs a float type.
template <int DT>
static hipError_t steps_op(const RankPtrs& P, int p, int64_t n, int op, StepMode mode,
                           int step_begin, int step_end, const SyncCfg& sc, hipStream_t s,
                           int* grid_used, int* launches) {
  constexpr bool kFloat = DT == 1 || DT == 2 || DT == 3 || DT == 4;
  if (op == kMax)
    return steps_dt<DT, kMax>(P, p, n, mode, step_begin, step_end, sc, s, grid_used, launches);
  if constexpr (kFloat) {
    if (op == kAvg)
      return steps_dt<DT, kAvg>(P, p, n, mode, step_begin, step_end, sc, s, grid_used, launches);
  }
  return steps_dt<DT, kSum>(P, p, n, mode, step_begin, step_end, sc, s, grid_used, launches);
}

hipError_t launch_steps(const RankPtrs& P, int p, int64_t n, int dtype, int op, StepMode mode,
                        int step_begin, int step_end, const SyncCfg& sc, hipStream_t s,
                        int* grid_used, int* launches) {
  switch (dtype) {
    case 0: return steps_op<0>(P, p, n, op, mode, step_begin, step_end, sc, s, grid_used, launches);
    case 1: return steps_op<1>(P, p, n, op, mode, step_begin, step_end, sc, s, grid_used, launches);
    case 2: return steps_op<2>(P, p, n, op, mode, step_begin, step_end, sc, s, grid_used, launches);
    case 3: return steps_op<3>(P, p, n, op, mode, step_begin, step_end, sc, s, grid_used, launches);
    case 4: return steps_op<4>(P, p, n, op, mode, step_begin, step_end, sc, s, grid_used, launches);
    default: return steps_op<5>(P, p, n, op, mode, step_begin, step_end, sc, s, grid_used, launches);
  }
}

// Default slice: about four slices per worker per hop, at least 64 KiB.  Every
// slice hop pays one acquire and one release (an L2 invalidate and an L2
// write-back); measured at 8 x 16 GB bf16, 64 KiB slices ran 719 ms and 4 MiB
// slices 105 ms, so slices must be large enough to amortise that cost while
// leaving every worker several slices to pipeline.

int64_t pipelined_default_slice(int p, int64_t n, int dtype, int grid_override) {
  const int V = elems_per_vec(dtype);
  int cus = 0;
  int64_t workers = 64;
  if (device_cus(&cus) == hipSuccess && cus > 0) {
    const int64_t budget = grid_override > 0 ? grid_override : (int64_t)cus * kPipelinedPerCU;
    workers = std::max<int64_t>(1, budget / p);
  }
  const int64_t chunk = n / p + 1;
  int64_t slice = (chunk + 4 * workers - 1) / (4 * workers);
  // Slices of at least 64 KiB, except that a chunk with room for eight 16 KiB
  // slices is cut into eight or more, so that eight workers per rank, one per
  // XCD, can take them and publish through their own XCD's L2 (measured on
  // MI355X, bf16: p = 8 at 1 MiB per rank 0.049 ms against 0.091, p = 64 at
  // 16 MiB 1.04 against 2.66).
  const int64_t small = (16 << 10) / elem_bytes(dtype), large = (64 << 10) / elem_bytes(dtype);
  int64_t least = large;
  if ((chunk + small - 1) / small >= 8) least = std::max(small, std::min(large, chunk / 8));
  slice = std::max<int64_t>(slice, least);
  const int64_t L = (int64_t)V * kLineVecs;
  return (slice + L - 1) / L * L;
}

int64_t pipelined_slices_per_chunk(int p, int64_t n, int dtype, int64_t slice) {
  const int V = elems_per_vec(dtype);
  int64_t kmax = 1;
  for (int c = 0; c < p; ++c) {
    const int64_t lo = host_chunk_lo(0, n, p, c), hi = host_chunk_lo(0, n, p, c + 1);
    const int64_t A = slice_origin(lo, V);
    int64_t k = 1;
    if (A < hi) k = std::max<int64_t>(1, (hi - A + slice - 1) / slice);
    kmax = std::max(kmax, k);
  }
  return kmax;
}

template <int DT, int OP>
static hipError_t pipelined_dt(const RankPtrs& P, int p, int64_t n, int hop_begin, int hop_end,
                               int64_t slice, int64_t kmax, uint32_t* flags, uint32_t base,
                               const SyncCfg& sc, hipStream_t s, int* grid_used) {
  PipeArgs a;
  a.P = P;
  a.g = make_geo(0, n, p);
  a.slice = slice;
  a.kmax = kmax;
  a.flags = flags;
  a.ws = sc.ws;
  a.limit = sc.limit_ticks;
  a.p = p;
  a.hop_begin = hop_begin;
  a.hop_end = hop_end;
  a.base = base;
  a.expect_extra = sc.expect_extra;
  a.stress = sc.stress;
  const bool nt = streaming(p, n, DT);
  const void* func = nt ? reinterpret_cast<const void*>(&k_pipelined<DT, OP, kPipeU, true, false>)
                        : reinterpret_cast<const void*>(&k_pipelined<DT, OP, kPipeU, false, false>);
  int resident = 0;
  hipError_t e = resident_blocks(func, &resident);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = device_cus(&cus);
  if (e != hipSuccess) return e;
  int budget = sc.grid > 0 ? std::min(sc.grid, resident) : std::min(resident, kPipelinedPerCU * cus);
  int workers = (int)std::max<int64_t>(1, std::min<int64_t>(budget / p, kmax));
  if (workers * p > resident) return hipErrorInvalidConfiguration;   // p > resident
  bool placed = false;
  e = xcd_placement(&placed, sc.may_probe);
  if (e != hipSuccess) return e;
  // a multiple of 8 workers keeps every slice on one XCD: measured on MI355X
  // (bf16, p = 9) 0.61 ms at 64 MiB per rank with 112 workers against 1.60 with
  // 113, which must publish every slice through an L2 write-back
  if (placed && workers >= kXcds) workers = workers / kXcds * kXcds;
  if (placed && workers % kXcds == 0)
    func = nt ? reinterpret_cast<const void*>(&k_pipelined<DT, OP, kPipeU, true, true>)
              : reinterpret_cast<const void*>(&k_pipelined<DT, OP, kPipeU, false, true>);
  a.workers = workers;
  *grid_used = workers * p;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(func), dim3(workers * p), dim3(kBlock), args,
                         0, s);
}

template <int DT>
static hipError_t pipelined_op(const RankPtrs& P, int p, int64_t n, int op, int hop_begin,
                               int hop_end, int64_t slice, int64_t kmax, uint32_t* flags,
                               uint32_t base, const SyncCfg& sc, hipStream_t s, int* grid_used) {
  constexpr bool kFloat = DT == 1 || DT == 2 || DT == 3 || DT == 4;
  if (op == kMax)
    return pipelined_dt<DT, kMax>(P, p, n, hop_begin, hop_end, slice, kmax, flags, base, sc, s,
                                  grid_used);
  if constexpr (kFloat) {
    if (op == kAvg)
      return pipelined_dt<DT, kAvg>(P, p, n, hop_begin, hop_end, slice, kmax, flags, base, sc, s,
                                    grid_used);
  }
  return pipelined_dt<DT, kSum>(P, p, n, hop_begin, hop_end, slice, kmax, flags, base, sc, s,
                                grid_used);
}

hipError_t launch_pipelined(const RankPtrs& P, int p, int64_t n, int dtype, int op, int hop_begin,
                            int hop_end, int64_t slice, int64_t kmax, uint32_t* flags,
                            uint32_t base, const SyncCfg& sc, hipStream_t s, int* grid_used) {
#define RA_PIPE(D) \
  pipelined_op<D>(P, p, n, op, hop_begin, hop_end, slice, kmax, flags, base, sc, s, grid_used)
  switch (dtype) {
    case 0: return RA_PIPE(0);
    case 1: return RA_PIPE(1);
    case 2: return RA_PIPE(2);
    case 3: return RA_PIPE(3);
    case 4: return RA_PIPE(4);
    default: return RA_PIPE(5);
  }
#undef RA_PIPE
}


}  // namespace ra
