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

// The chunks' edge elements carried through their hops, one chunk per wave
// (edge_wave): edge workgroup w carries chunks 4w .. 4w + 3.  Lane k runs
// element k of chunk c through the hops as ride_hops does for a vector and
// leaves what each rank ends with: a reduce-scatter's partials (each receiver's
// after its hop, and the sender's divided term for an average), the finished
// sum everywhere for an all-reduce (its partials are overwritten by the
// all-gather), the owner's copy for an all-gather.
template <int DT, int OP, int MODE>
__device__ __forceinline__ void ride_edges(const RankPtrs& P, const ChunkGeo& g, int p,
                                           int64_t w) {
  typedef Elem<DT> E;
  constexpr bool kDiv = OP == kAvg && MODE != kRideAllGather;
  EdgeLds<DT>& L = edge_lds<DT>();
  void** lp = L.lp;
  load_rank_table(lp, P, p);
  const int wave = (int)(threadIdx.x / kWave);
  const int64_t cw = w * kWavesPerBlock + wave;
  const int c = cw < p ? (int)cw : 0;
  const int64_t lo = cw < p ? chunk_lo(g, c) : 0, hi = cw < p ? chunk_hi(g, c) : 0;
  const int owner = c == 0 ? p - 1 : c - 1;
  edge_wave<DT>(lp, p, lo, hi, L.slab[wave], [&](EdgeSlab<DT>& sl, int k) {
    if (MODE == kRideAllGather) {
      const typename E::S out = sl.x[k][owner];
      for (int r = 0; r < p; ++r) sl.x[k][r] = out;
      sl.mask[k] = all_ranks(p) & ~(1ull << owner);
      return;
    }
    typename E::S acc = sl.x[k][c];
    uint64_t m = 0;
    if (kDiv) {
      acc = E::div1(acc, p);
      if (MODE == kRideReduceScatter) {
        sl.x[k][c] = acc;
        m |= 1ull << c;
      }
    }
    for (int h = 1; h < p; ++h) {
      const int r = c + h < p ? c + h : c + h - p;
      const typename E::S x = sl.x[k][r];
      acc = comb1<DT, OP>(acc, kDiv ? E::div1(x, p) : x);
      sl.x[k][r] = acc;
      m |= 1ull << r;
    }
    if (MODE == kRideAllReduce) {
      for (int r = 0; r < p; ++r) sl.x[k][r] = acc;
      m = all_ranks(p);
    }
    sl.mask[k] = m;
  });
}

// Slice q = (chunk c, slice k of that chunk), numbered by tile_of: tiles
// k*tps .. (k+1)*tps - 1 of the chunk, one 16-byte vector per thread per tile,
// carried through its hops tile by tile.  The partials of the reduce-scatter
// are written before the all-gather overwrites them (a compiler barrier keeps
// those stores: they are the step states, not dead stores).  When the chunks
// have unaligned edge elements, edge workgroups (placed by edge_start) carry
// them, a chunk per wave, while the slices run (in each chunk's first slice
// they were a second chain of round trips after its vectors).
template <int DT, int OP, int MODE>
__global__ __launch_bounds__(kBlock) void k_rider(RankPtrs P, ChunkGeo g, int p, int64_t T,
                                                  int64_t tps, int64_t K, int64_t nslices,
                                                  int edges, int64_t e0, int tail_last,
                                                  uint32_t stress) {
  typedef Elem<DT> E;
  constexpr int V = E::V;
  constexpr bool kDiv = OP == kAvg && MODE != kRideAllGather;
  // edge workgroups e0 .. e0 + edges - 1 carry the edge elements, outside the
  // slice loop (as in k_fused); the other workgroups take the slices in order
  const int64_t b = blockIdx.x;
  if (b >= e0 && b < e0 + edges) ride_edges<DT, OP, MODE>(P, g, p, b - e0);
  for (int64_t q = b; q < nslices + edges; q += gridDim.x) {
    if (q >= e0 && q < e0 + edges) continue;
    int c;
    int64_t k;
    tile_of((uint32_t)(q < e0 ? q : q - edges), (uint32_t)K, (uint32_t)p, tail_last, &c, &k);
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
  int64_t widest = 0;
  int edges = 0;
  for (int c = 0; c < p; ++c) {
    const int64_t lo = host_chunk_lo(0, n, p, c), hi = host_chunk_lo(0, n, p, c + 1);
    widest = std::max<int64_t>(widest, tiled_vecs_in(lo, hi, V));
    if (hi > lo && (lo % V != 0 || hi % V != 0 || vecs_in(lo, hi, V) == 0))
      edges = (p + kWavesPerBlock - 1) / kWavesPerBlock;     // a wave per chunk
  }
  const int64_t T = std::max<int64_t>(1, (widest + kBlock - 1) / kBlock);
  const int64_t tile_elems = (int64_t)kBlock * V;
  const int64_t tps = slice_elems > 0 ? std::max<int64_t>(1, (slice_elems + tile_elems - 1) / tile_elems)
                                      : 1;
  const int64_t K = (T + tps - 1) / tps;
  const int64_t nslices = (int64_t)p * K;
  // the chunks' last slices are short, in a launch whose slices are all resident
  const int tail_last = nslices <= kResidentTiles && short_tail(widest, kBlock * tps);
  if (nslices + edges > 0xFFFFFFFFll) return hipErrorInvalidValue;  // tile_of decodes 32 bits
  const int grid = (int)std::min<int64_t>(nslices + edges, kMaxGrid);
  const int64_t e0 = edge_start(nslices, p, tail_last, edges, grid);
  *grid_used = grid;
  const unsigned lds = edges ? (unsigned)sizeof(EdgeLds<DT>) : 0u;
  hipLaunchKernelGGL((k_rider<DT, OP, MODE>), dim3(grid), dim3(kBlock), lds, s, P, g, p, T, tps, K,
                     nslices, edges, e0, tail_last, stress);
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
