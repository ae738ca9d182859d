// ra_rider.hip -- the pipelined ring in its byte-lean form (gfx950): chunks cut
// into slices, and every slice carried round the ring by one workgroup.
//
// "Ring All-Reduce, in depth", section "What real libraries add", pipelining:
// chunks are cut into pieces, and a piece goes on to the next rank as soon as it
// is done instead of waiting for its whole chunk, so per-step waiting overlaps
// with moving data.  On one GPU the finest form of that is a workgroup per slice
// that takes its slice through every hop itself: hop h of slice k runs as soon
// as hop h-1 of the same slice is done (program order inside the workgroup),
// and the slices of all chunks are in flight at once with no barrier and no
// flag between workgroups.  The running partial stays in registers from hop
// to hop, so a hop reads only the receiver's copy, combines it and writes the
// receiver's new partial -- the state the step-by-step schedule leaves there
// ("The schedule": reduce-scatter step s adds rank r's chunk r - s into rank
// r + 1).  After p - 1 hops the partial is the full sum, sitting at the owner
// (rank c - 1 owns chunk c); the all-gather then writes it over the p - 1 other
// copies.  HBM bytes per all-reduce: p reads and 2(p - 1) writes per element
// position, (3p - 2)S, against 5(p - 1)S for the step-by-step schedule, which
// re-reads each partial from the rank it was just written to.
//
// Every element is folded in exactly the ring's order and rounding, so the
// result (and, for a reduce-scatter, every partial) has the same bits as the
// step-by-step ring.
//
// Accesses are cached, at every size: a receiver's partial and, soon after, the
// finished value land on the same lines, and in the L2 and the Infinity Cache
// some of those pairs merge into one write to HBM.  Measured at p = 8 with 16 GB
// per rank: 45.3 ms and 0.81 x 2(p-1)S of writes counted, against 57.1 ms and
// 0.99 x with the streaming hint the other kernels use at that size (0.81 against
// 1.14 ms at 256 MiB of float32 per rank; a tie at p = 2, whose hops write no
// partial that a final value overwrites).
#include "ra_elem.h"
#include "ra_sync.h"
#include "ra_internal.h"

namespace ra {

// What a launch carries out: hops 0..p-2 (reduce-scatter), then the all-gather
// (all-reduce), or either phase alone.
enum RiderMode { kRideAllReduce = 0, kRideReduceScatter = 1, kRideAllGather = 2 };

// Hops first .. first + N - 1 of a slice's reduce-scatter at vector vt + lane:
// the N receivers' copies are loaded together (no receiver of one hop is read by
// another, so the loads may all be in flight), then each is combined with the
// running partial, rounded, and written back as that receiver's partial.
// Averages divide every receiver's input by p as it joins (the sender's was
// divided at the first hop).  Ring positions are taken mod p: rank
// (c + first + i) mod p, with c + first + N - 1 < 2p.
template <int N, int DT, int OP>
__device__ __forceinline__ void ride_batch(u32x4& acc, const RankPtrs& P, int p, int c, int first,
                                           int64_t vt, unsigned lane) {
  void* q[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int r = c + first + i;
    q[i] = P.b[r >= p ? r - p : r];
  }
  u32x4 x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = ld16t(q[i], vt, lane);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    acc = vcomb<DT, OP>(acc, OP == kAvg ? vdiv<DT>(x[i], p) : x[i]);
    st16t(q[i], vt, lane, acc);
  }
}

template <int DT, int OP>
__device__ __forceinline__ void ride_hops(u32x4& acc, const RankPtrs& P, int p, int c,
                                          int64_t vt, unsigned lane) {
  int first = 1;
  for (; p - first >= kRankBatch; first += kRankBatch)
    ride_batch<kRankBatch, DT, OP>(acc, P, p, c, first, vt, lane);
  switch (p - first) {
    case 7: ride_batch<7, DT, OP>(acc, P, p, c, first, vt, lane); break;
    case 6: ride_batch<6, DT, OP>(acc, P, p, c, first, vt, lane); break;
    case 5: ride_batch<5, DT, OP>(acc, P, p, c, first, vt, lane); break;
    case 4: ride_batch<4, DT, OP>(acc, P, p, c, first, vt, lane); break;
    case 3: ride_batch<3, DT, OP>(acc, P, p, c, first, vt, lane); break;
    case 2: ride_batch<2, DT, OP>(acc, P, p, c, first, vt, lane); break;
    case 1: ride_batch<1, DT, OP>(acc, P, p, c, first, vt, lane); break;
    default: break;
  }
}

// Element i of chunk c carried through its hops on its own (the chunks'
// unaligned edges), as ride_hops does for a vector: the receivers of a batch of
// hops are loaded together (load_positions), then each is combined with the
// running partial and written back.  lp is the LDS copy of the rank pointers.
template <int DT, int OP, int MODE>
__device__ __forceinline__ void ride_element(void* const* lp, int p, int c, int64_t i) {
  typedef Elem<DT> E;
  constexpr bool kDiv = OP == kAvg && MODE != kRideAllGather;
  const int owner = c == 0 ? p - 1 : c - 1;
  if (MODE == kRideAllGather) {
    const typename E::S out = ld1<DT>(lp[owner], i);
    for (int r = 0; r < p; ++r)
      if (r != owner) st1<DT>(lp[r], i, out);
    return;
  }
  typename E::S acc = ld1<DT>(lp[c], i);
  if (kDiv) {
    acc = E::div1(acc, p);
    if (MODE == kRideReduceScatter) st1<DT>(lp[c], i, acc);
  }
  for (int h0 = 1; h0 < p; h0 += kRankBatch) {
    typename E::S x[kRankBatch];
    load_positions<DT>(x, lp, 0, p, c, h0, p, i);
#pragma unroll
    for (int u = 0; u < kRankBatch; ++u) {
      if (h0 + u >= p) break;
      const int r = c + h0 + u < p ? c + h0 + u : c + h0 + u - p;
      acc = comb1<DT, OP>(acc, kDiv ? E::div1(x[u], p) : x[u]);
      st1<DT>(lp[r], i, acc);
    }
  }
  if (MODE == kRideAllReduce) {
    asm volatile("" ::: "memory");
    for (int r = 0; r < p; ++r)
      if (r != owner) st1<DT>(lp[r], i, acc);
  }
}

// Slice q = (chunk c, slice k of that chunk): tiles k*tps .. (k+1)*tps - 1 of
// the chunk, one 16-byte vector per thread per tile, carried through its hops
// tile by tile.  The partials of the reduce-scatter are written before the
// all-gather overwrites them (a compiler barrier keeps those stores: they are
// the step states, not dead stores).  When the chunks have unaligned edge
// elements (edges = 1), workgroup 0 carries them all, element by element, while
// the slices run (in each chunk's first slice they were a second chain of
// round trips after its vectors).
template <int DT, int OP, int MODE>
__global__ __launch_bounds__(kBlock) void k_rider(RankPtrs P, ChunkGeo g, int p, int64_t T,
                                                  int64_t tps, int64_t K, int64_t nslices,
                                                  int edges, uint32_t stress) {
  typedef Elem<DT> E;
  constexpr int V = E::V;
  constexpr bool kDiv = OP == kAvg && MODE != kRideAllGather;
  for (int64_t q = blockIdx.x; q < nslices; q += gridDim.x) {
    if (q < edges) {
      constexpr int kPer = 2 * V - 2;
      __shared__ void* lp[kMaxRanks];
      load_rank_table(lp, P, p);
      for (int e = threadIdx.x; e < p * kPer; e += kBlock) {
        const int c = e / kPer, k = e - c * kPer;
        const int64_t lo = chunk_lo(g, c), hi = chunk_hi(g, c);
        const Span sp = split_span<V>(lo, hi);
        const int64_t nh = sp.head_hi - lo, nt = hi - sp.tail_lo;
        if (k < nh + nt) ride_element<DT, OP, MODE>(lp, p, c, k < nh ? lo + k : sp.tail_lo + (k - nh));
      }
      continue;
    }
    const int64_t qq = q - edges;
    const int c = (int)(qq / K);
    const int64_t k = qq - (int64_t)c * K;
    const int owner = c == 0 ? p - 1 : c - 1;
    const int64_t lo = chunk_lo(g, c), hi = chunk_hi(g, c);
    const Span sp = split_span<V>(lo, hi);
    const int64_t j1 = (k + 1) * tps < T ? (k + 1) * tps : T;
    const unsigned lane = threadIdx.x;
    stress_delay(stress, (uint32_t)q);
    for (int64_t j = k * tps; j < j1; ++j) {
      const int64_t vt = sp.vb + j * kBlock;        // the tile's first vector
      if (vt + lane < sp.v0 || vt + lane >= sp.v1) continue;
      if (MODE == kRideAllGather) {
        const u32x4 out = ld16t(P.b[owner], vt, lane);
        store_all<false>(P, p, vt, lane, out, owner);
        continue;
      }
      u32x4 acc = ld16t(P.b[c], vt, lane);
      if (kDiv) {
        acc = vdiv<DT>(acc, p);
        // a reduce-scatter leaves the sender's divided term, as the step kernels do
        if (MODE == kRideReduceScatter) st16t(P.b[c], vt, lane, acc);
      }
      ride_hops<DT, OP>(acc, P, p, c, vt, lane);
      if (MODE == kRideAllReduce) {
        asm volatile("" ::: "memory");
        store_all<false>(P, p, vt, lane, acc, owner);
      }
    }
  }
}

// Default slice: one tile (kBlock vectors, 4 KiB of every rank's chunk) per
// workgroup, the most workgroups in flight -- the shape the one-pass kernel
// streams best with.
template <int DT, int OP, int MODE>
static hipError_t rider_launch(const RankPtrs& P, int p, int64_t n, int64_t slice_elems,
                               uint32_t stress, hipStream_t s, int* grid_used) {
  const int V = Elem<DT>::V;
  const ChunkGeo g = make_geo(0, n, p);
  int64_t T = 1;
  int edges = 0;
  for (int c = 0; c < p; ++c) {
    const int64_t lo = host_chunk_lo(0, n, p, c), hi = host_chunk_lo(0, n, p, c + 1);
    T = std::max<int64_t>(T, (tiled_vecs_in(lo, hi, V) + kBlock - 1) / kBlock);
    if (hi > lo && (lo % V != 0 || hi % V != 0 || vecs_in(lo, hi, V) == 0)) edges = 1;
  }
  const int64_t tile_elems = (int64_t)kBlock * V;
  const int64_t tps = slice_elems > 0 ? std::max<int64_t>(1, (slice_elems + tile_elems - 1) / tile_elems)
                                      : 1;
  const int64_t K = (T + tps - 1) / tps;
  const int64_t nslices = edges + (int64_t)p * K;
  const int grid = (int)std::min<int64_t>(nslices, kMaxGrid);
  *grid_used = grid;
  hipLaunchKernelGGL((k_rider<DT, OP, MODE>), dim3(grid), dim3(kBlock), 0, s, P, g, p, T, tps, K,
                     nslices, edges, stress);
  return hipGetLastError();
}

template <int DT, int MODE>
static hipError_t rider_op(const RankPtrs& P, int p, int64_t n, int op, int64_t slice_elems,
                           uint32_t stress, hipStream_t s, int* grid_used) {
  constexpr bool kFloat = DT == 1 || DT == 2 || DT == 3 || DT == 4;
  if (MODE == kRideAllGather) return rider_launch<DT, kSum, MODE>(P, p, n, slice_elems, stress, s, grid_used);
  if (op == kMax) return rider_launch<DT, kMax, MODE>(P, p, n, slice_elems, stress, s, grid_used);
  if constexpr (kFloat) {
    if (op == kAvg) return rider_launch<DT, kAvg, MODE>(P, p, n, slice_elems, stress, s, grid_used);
  }
  return rider_launch<DT, kSum, MODE>(P, p, n, slice_elems, stress, s, grid_used);
}

template <int MODE>
static hipError_t rider_mode(const RankPtrs& P, int p, int64_t n, int dtype, int op,
                             int64_t slice_elems, uint32_t stress, hipStream_t s, int* grid_used) {
  switch (dtype) {
    case 0: return rider_op<0, MODE>(P, p, n, op, slice_elems, stress, s, grid_used);
    case 1: return rider_op<1, MODE>(P, p, n, op, slice_elems, stress, s, grid_used);
    case 2: return rider_op<2, MODE>(P, p, n, op, slice_elems, stress, s, grid_used);
    case 3: return rider_op<3, MODE>(P, p, n, op, slice_elems, stress, s, grid_used);
    case 4: return rider_op<4, MODE>(P, p, n, op, slice_elems, stress, s, grid_used);
    default: return rider_op<5, MODE>(P, p, n, op, slice_elems, stress, s, grid_used);
  }
}

hipError_t launch_rider(const RankPtrs& P, int p, int64_t n, int dtype, int op, int mode,
                        int64_t slice_elems, uint32_t stress, hipStream_t s, int* grid_used) {
  switch (mode) {
    case kRideReduceScatter:
      return rider_mode<kRideReduceScatter>(P, p, n, dtype, op, slice_elems, stress, s, grid_used);
    case kRideAllGather:
      return rider_mode<kRideAllGather>(P, p, n, dtype, op, slice_elems, stress, s, grid_used);
    default:
      return rider_mode<kRideAllReduce>(P, p, n, dtype, op, slice_elems, stress, s, grid_used);
  }
}

}  // namespace ra
