// ra_elem.h -- element types, vector memory access and chunk geometry of the
// ring all-reduce kernels (gfx950).
//
// * element types: one hop of the ring is "receiver's chunk += incoming chunk",
//   rounded to the buffer type ("Ring All-Reduce, in depth", section "An
//   implementation": the torch ring adds in the tensor's dtype).  Values move in
//   16-byte vectors (global_load/store_dwordx4): 4 int32, 4 float32 or 8 bfloat16.
// * chunk geometry: chunk c of an n-element buffer split p ways starts at
//   c*floor(n/p) + min(c, n mod p) (same page, "An implementation").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ra {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxRanks = 64;
constexpr int kBlock = 256;               // threads per workgroup (4 wave64s)
constexpr int kLineVecs = 8;              // 16-byte vectors per 128-byte cache line

// Device pointers of the p rank buffers, passed by value in the kernel
// arguments; a wave-uniform index into it compiles to a scalar load from the
// argument segment.
struct RankPtrs {
  void* b[kMaxRanks];
};

// Partition of a segment [off, off + len) into p chunks.
struct ChunkGeo {
  int64_t off;    // first element of the segment
  int64_t base;   // floor(len / p)
  int64_t extra;  // len mod p
};

__device__ __forceinline__ int64_t chunk_lo(const ChunkGeo& g, int c) {
  return g.off + (int64_t)c * g.base + (c < g.extra ? c : g.extra);
}
__device__ __forceinline__ int64_t chunk_hi(const ChunkGeo& g, int c) {
  return chunk_lo(g, c + 1);
}

__device__ __forceinline__ int mod_p(int x, int p) {
  x %= p;
  return x < 0 ? x + p : x;
}

// ---------------------------------------------------------------- element types
// dtype codes match ra_dtype: 0 int32, 1 float32, 2 bfloat16, 3 float16,
// 4 float64, 5 int64.  op codes match ra_op: 0 sum, 1 max, 2 avg.

enum Op { kSum = 0, kMax = 1, kAvg = 2 };

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// IEEE 754-2019 maximum of two floats given as values and bit patterns: a NaN
// operand gives the canonical quiet NaN, +0 counts as larger than -0, so the
// result does not depend on the operand order.
template <typename B, typename F>
__device__ __forceinline__ B max_bits(B a, B b, F va, F vb, B qnan, B sign) {
  if (va != va || vb != vb) return qnan;
  if (vb > va) return b;
  if (va > vb) return a;
  return (a & sign) ? b : a;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  f32x2 v = {f, 0.0f};
  return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2)) & 0xffffu);
}
__device__ __forceinline__ float f16_to_f32(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Per element type: V elements per 16-byte vector, storage S, and
//   add1(a, b)   one hop of the sum, rounded to the type
//   max1(a, b)   exact maximum
//   div1(a, p)   a / p rounded to the type (floats: a contribution to an average)
//   add(a, b)    add1 on every element of a 16-byte vector
// Floats with a wide accumulation type W also have to_w (exact), from_w (one
// rounding to nearest even) and divw (a / p rounded to W).
template <int DT> struct Elem;

template <> struct Elem<0> {                 // int32: wraps modulo 2^32
  static constexpr int V = 4;
  typedef uint32_t S;
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) { return a + b; }
  __device__ static __forceinline__ S add1(S a, S b) { return a + b; }
  __device__ static __forceinline__ S max1(S a, S b) { return (int32_t)a >= (int32_t)b ? a : b; }
  __device__ static __forceinline__ S div1(S a, int) { return a; }
};

template <> struct Elem<5> {                 // int64: wraps modulo 2^64
  static constexpr int V = 2;
  typedef uint64_t S;
  __device__ static __forceinline__ S add1(S a, S b) { return a + b; }
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) {
    return __builtin_bit_cast(u32x4, __builtin_bit_cast(u64x2, a) + __builtin_bit_cast(u64x2, b));
  }
  __device__ static __forceinline__ S max1(S a, S b) { return (int64_t)a >= (int64_t)b ? a : b; }
  __device__ static __forceinline__ S div1(S a, int) { return a; }
};

template <> struct Elem<1> {                 // float32: IEEE add, nearest even
  static constexpr int V = 4;
  typedef uint32_t S;
  typedef double W;
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) {
    f32x4 s = __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b);
    return __builtin_bit_cast(u32x4, s);
  }
  __device__ static __forceinline__ S add1(S a, S b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }
  __device__ static __forceinline__ S max1(S a, S b) {
    return max_bits<S, float>(a, b, __uint_as_float(a), __uint_as_float(b), 0x7fc00000u, 0x80000000u);
  }
  __device__ static __forceinline__ S div1(S a, int p) { return __float_as_uint(__uint_as_float(a) / (float)p); }
  __device__ static __forceinline__ W to_w(S a) { return (double)__uint_as_float(a); }
  __device__ static __forceinline__ S from_w(W w) { return __float_as_uint((float)w); }
  __device__ static __forceinline__ W divw(W w, int p) { return w / (double)p; }
};

template <> struct Elem<4> {                 // float64: IEEE add, nearest even
  static constexpr int V = 2;
  typedef uint64_t S;
  __device__ static __forceinline__ double val(S a) { return __builtin_bit_cast(double, a); }
  __device__ static __forceinline__ S bits(double d) { return __builtin_bit_cast(S, d); }
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) {
    return __builtin_bit_cast(u32x4, __builtin_bit_cast(f64x2, a) + __builtin_bit_cast(f64x2, b));
  }
  __device__ static __forceinline__ S add1(S a, S b) { return bits(val(a) + val(b)); }
  __device__ static __forceinline__ S max1(S a, S b) {
    return max_bits<S, double>(a, b, val(a), val(b), 0x7ff8000000000000ull, 0x8000000000000000ull);
  }
  __device__ static __forceinline__ S div1(S a, int p) { return bits(val(a) / (double)p); }
};

// bfloat16: both operands widened exactly to float32 (a bf16 is the top half of
// a float32), added in float32 (nearest even), narrowed back to bf16 (nearest
// even) with the gfx950 packed convert.  Rounding through float32 first gives
// the same result as rounding the exact sum once, because float32 carries more
// than twice bf16's precision plus two bits.  The same holds for a quotient by
// p <= 64 (both operands bf16 values), so div1 divides in float32.
__device__ __forceinline__ uint32_t bf16_pair_add(uint32_t a, uint32_t b) {
  f32x2 s;
  s.x = __uint_as_float(a << 16) + __uint_as_float(b << 16);
  s.y = __uint_as_float(a & 0xffff0000u) + __uint_as_float(b & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(s, bf16x2));
}

template <> struct Elem<2> {
  static constexpr int V = 8;
  typedef uint16_t S;
  typedef float W;
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) {
    u32x4 r;
    r.x = bf16_pair_add(a.x, b.x);
    r.y = bf16_pair_add(a.y, b.y);
    r.z = bf16_pair_add(a.z, b.z);
    r.w = bf16_pair_add(a.w, b.w);
    return r;
  }
  __device__ static __forceinline__ S add1(S a, S b) {
    return (S)(bf16_pair_add((uint32_t)a, (uint32_t)b) & 0xffffu);
  }
  __device__ static __forceinline__ S max1(S a, S b) {
    return max_bits<S, float>(a, b, bf16_to_f32(a), bf16_to_f32(b), (S)0x7fc0, (S)0x8000);
  }
  __device__ static __forceinline__ S div1(S a, int p) { return f32_to_bf16(bf16_to_f32(a) / (float)p); }
  __device__ static __forceinline__ W to_w(S a) { return bf16_to_f32(a); }
  __device__ static __forceinline__ S from_w(W w) { return f32_to_bf16(w); }
  __device__ static __forceinline__ W divw(W w, int p) { return w / (float)p; }
};

// float16: the hardware half add rounds the exact sum once (nearest even); the
// quotient goes through float32 as for bf16 (24 >= 2 * 11 + 2).
template <> struct Elem<3> {
  static constexpr int V = 8;
  typedef uint16_t S;
  typedef float W;
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) {
    return __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, a) + __builtin_bit_cast(f16x8, b));
  }
  __device__ static __forceinline__ S add1(S a, S b) {
    return __builtin_bit_cast(S, (_Float16)(__builtin_bit_cast(_Float16, a) + __builtin_bit_cast(_Float16, b)));
  }
  __device__ static __forceinline__ S max1(S a, S b) {
    return max_bits<S, float>(a, b, f16_to_f32(a), f16_to_f32(b), (S)0x7e00, (S)0x8000);
  }
  __device__ static __forceinline__ S div1(S a, int p) { return f32_to_f16(f16_to_f32(a) / (float)p); }
  __device__ static __forceinline__ W to_w(S a) { return f16_to_f32(a); }
  __device__ static __forceinline__ S from_w(W w) { return f32_to_f16(w); }
  __device__ static __forceinline__ W divw(W w, int p) { return w / (float)p; }
};

// Maximum of 16-bit floats (bfloat16: infinity 0x7f80, quiet NaN 0x7fc0;
// float16: 0x7c00, 0x7e00), two lanes per 32-bit word, through integer keys.
// For a value that is not NaN, x ^ (x's sign ? 0x7fff : 0), read as a signed
// 16-bit integer, orders like the value itself, with -0 (key -1) below +0
// (key 0), so one packed signed maximum takes the larger of two lanes.  NaN
// lanes are tracked apart: adding 0x7fff - infinity to a lane's magnitude sets
// its bit 15 exactly when the magnitude exceeds infinity's.  The result lane is
// the canonical quiet NaN wherever any operand lane was NaN.
typedef short s16x2 __attribute__((ext_vector_type(2)));

template <uint32_t kInf, uint32_t kQNaN>
struct Max16 {
  __device__ static __forceinline__ uint32_t key(uint32_t w) {   // an involution
    return w ^ (((w >> 15) & 0x00010001u) * 0x7fffu);
  }
  __device__ static __forceinline__ uint32_t nan_bits(uint32_t w) {
    return ((w & 0x7fff7fffu) + (0x7fffu - kInf) * 0x00010001u) & 0x80008000u;
  }
  __device__ static __forceinline__ uint32_t kmax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                 __builtin_bit_cast(s16x2, b)));
  }
  // keys and NaN bits back to values
  __device__ static __forceinline__ uint32_t finish(uint32_t k, uint32_t nan) {
    const uint32_t m = ((nan >> 15) & 0x00010001u) * 0xffffu;
    return (key(k) & ~m) | (kQNaN * 0x00010001u & m);
  }
};
typedef Max16<0x7f80u, 0x7fc0u> MaxBf16;
typedef Max16<0x7c00u, 0x7e00u> MaxF16;

// Elements of a 16-byte vector as an array of storage words.
template <int DT> struct Lanes {
  typename Elem<DT>::S e[Elem<DT>::V];
};
template <int DT>
__device__ __forceinline__ Lanes<DT> unpack(u32x4 v) { return __builtin_bit_cast(Lanes<DT>, v); }
template <int DT>
__device__ __forceinline__ u32x4 pack(const Lanes<DT>& l) { return __builtin_bit_cast(u32x4, l); }

// One hop of reduction OP on a whole vector (sum and avg add; max takes the larger).
template <int DT, int OP>
__device__ __forceinline__ u32x4 vcomb(u32x4 a, u32x4 b) {
  typedef Elem<DT> E;
  if constexpr (OP == kMax && (DT == 2 || DT == 3)) {
    typedef typename std::conditional<DT == 2, MaxBf16, MaxF16>::type M;
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = M::finish(M::kmax(M::key(a[i]), M::key(b[i])), M::nan_bits(a[i]) | M::nan_bits(b[i]));
    return r;
  } else if constexpr (OP == kMax) {
    Lanes<DT> x = unpack<DT>(a), y = unpack<DT>(b);
#pragma unroll
    for (int i = 0; i < E::V; ++i) x.e[i] = E::max1(x.e[i], y.e[i]);
    return pack<DT>(x);
  } else {
    return E::add(a, b);
  }
}
template <int DT, int OP>
__device__ __forceinline__ typename Elem<DT>::S comb1(typename Elem<DT>::S a, typename Elem<DT>::S b) {
  if constexpr (OP == kMax) return Elem<DT>::max1(a, b);
  else return Elem<DT>::add1(a, b);
}

// A contribution to an average: every element divided by p, rounded to the type.
template <int DT>
__device__ __forceinline__ u32x4 vdiv(u32x4 a, int p) {
  Lanes<DT> x = unpack<DT>(a);
#pragma unroll
  for (int i = 0; i < Elem<DT>::V; ++i) x.e[i] = Elem<DT>::div1(x.e[i], p);
  return pack<DT>(x);
}

// Folding p terms, in the order given, into one result:
//   WIDE = false: every hop rounds to the element type (avg divides each term first)
//   WIDE = true:  terms widened exactly to W (avg divides them there), every hop
//                 rounds to W, the result is rounded once to the element type
template <int DT, int OP, bool WIDE> struct Fold;

// Maximum of 16-bit floats: keys and NaN bits accumulate, values come back once.
template <int DT> struct Fold16Max {
  typedef typename std::conditional<DT == 2, MaxBf16, MaxF16>::type M;
  typedef typename Elem<DT>::S S;
  struct A {
    u32x4 k, nan;
  };
  typedef S A1;
  __device__ static __forceinline__ A start(u32x4 x, int) {
    A a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a.k[i] = M::key(x[i]);
      a.nan[i] = M::nan_bits(x[i]);
    }
    return a;
  }
  __device__ static __forceinline__ A step(A a, u32x4 x, int) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a.k[i] = M::kmax(a.k[i], M::key(x[i]));
      a.nan[i] |= M::nan_bits(x[i]);
    }
    return a;
  }
  __device__ static __forceinline__ u32x4 finish(const A& a) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = M::finish(a.k[i], a.nan[i]);
    return r;
  }
  __device__ static __forceinline__ A1 start1(S x, int) { return x; }
  __device__ static __forceinline__ A1 step1(A1 acc, S x, int) { return Elem<DT>::max1(acc, x); }
  __device__ static __forceinline__ S finish1(A1 acc) { return acc; }
};
template <> struct Fold<2, kMax, false> : Fold16Max<2> {};
template <> struct Fold<3, kMax, false> : Fold16Max<3> {};

template <int DT, int OP> struct Fold<DT, OP, false> {
  typedef Elem<DT> E;
  typedef u32x4 A;
  typedef typename E::S A1;
  __device__ static __forceinline__ A start(u32x4 x, int p) { return OP == kAvg ? vdiv<DT>(x, p) : x; }
  __device__ static __forceinline__ A step(A acc, u32x4 x, int p) {
    return vcomb<DT, OP>(acc, OP == kAvg ? vdiv<DT>(x, p) : x);
  }
  __device__ static __forceinline__ u32x4 finish(A acc) { return acc; }
  __device__ static __forceinline__ A1 start1(typename E::S x, int p) { return OP == kAvg ? E::div1(x, p) : x; }
  __device__ static __forceinline__ A1 step1(A1 acc, typename E::S x, int p) {
    return comb1<DT, OP>(acc, OP == kAvg ? E::div1(x, p) : x);
  }
  __device__ static __forceinline__ typename E::S finish1(A1 acc) { return acc; }
};

template <int DT, int OP> struct Fold<DT, OP, true> {
  typedef Elem<DT> E;
  typedef typename E::W W;
  struct A { W w[E::V]; };
  typedef W A1;
  __device__ static __forceinline__ W term(typename E::S x, int p) {
    const W w = E::to_w(x);
    return OP == kAvg ? E::divw(w, p) : w;
  }
  __device__ static __forceinline__ A start(u32x4 x, int p) {
    const Lanes<DT> l = unpack<DT>(x);
    A a;
#pragma unroll
    for (int i = 0; i < E::V; ++i) a.w[i] = term(l.e[i], p);
    return a;
  }
  __device__ static __forceinline__ A step(A acc, u32x4 x, int p) {
    const Lanes<DT> l = unpack<DT>(x);
#pragma unroll
    for (int i = 0; i < E::V; ++i) acc.w[i] = acc.w[i] + term(l.e[i], p);
    return acc;
  }
  __device__ static __forceinline__ u32x4 finish(const A& acc) {
    Lanes<DT> l;
#pragma unroll
    for (int i = 0; i < E::V; ++i) l.e[i] = E::from_w(acc.w[i]);
    return pack<DT>(l);
  }
  __device__ static __forceinline__ A1 start1(typename E::S x, int p) { return term(x, p); }
  __device__ static __forceinline__ A1 step1(A1 acc, typename E::S x, int p) { return acc + term(x, p); }
  __device__ static __forceinline__ typename E::S finish1(A1 acc) { return E::from_w(acc); }
};

// ---------------------------------------------------------------- memory access

// NT = true marks the access non-temporal (streaming): used when the buffers are
// far larger than the 256 MB Infinity Cache, so nothing would be re-read from it.
// kNtPolicy is the same hint as an instruction cache-policy operand.
constexpr int kNtPolicy = 2;
template <bool NT = false>
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t vec) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base) + vec;
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT = false>
__device__ __forceinline__ void st16(void* base, int64_t vec, u32x4 v) {
  u32x4* p = reinterpret_cast<u32x4*>(base) + vec;
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}
// The same accesses addressed as (tile start, lane): vector vt + lane of a
// buffer, with vt wave-uniform.  Cached accesses take the tile's start address
// as a scalar and the lane's offset as a 32-bit vector register, which the
// global instructions accept as scalar base plus vector offset: one offset
// register serves every rank, instead of a 64-bit address pair per access in
// flight.  Streaming accesses keep the per-lane 64-bit address, the form the
// 16 GB-per-rank measurements favour (see the issue patterns below).
template <bool NT = false>
__device__ __forceinline__ u32x4 ld16t(const void* base, int64_t vt, unsigned lane) {
  if (NT) return ld16<true>(base, vt + (int64_t)lane);
  return (reinterpret_cast<const u32x4*>(base) + vt)[lane];
}
template <bool NT = false>
__device__ __forceinline__ void st16t(void* base, int64_t vt, unsigned lane, u32x4 v) {
  if (NT) st16<true>(base, vt + (int64_t)lane, v);
  else (reinterpret_cast<u32x4*>(base) + vt)[lane] = v;
}

template <int DT>
__device__ __forceinline__ typename Elem<DT>::S ld1(const void* base, int64_t i) {
  return reinterpret_cast<const typename Elem<DT>::S*>(base)[i];
}
template <int DT>
__device__ __forceinline__ void st1(void* base, int64_t i, typename Elem<DT>::S v) {
  reinterpret_cast<typename Elem<DT>::S*>(base)[i] = v;
}

// Vector vt + lane of every rank (vt wave-uniform), folded or stored.
//
// The rank index is wave-uniform, so each rank's pointer is a scalar load from
// the kernel arguments.  Two ways of issuing the accesses, chosen by the
// streaming flag because each measured best in its own regime:
//  * Cache-resident calls (NT = false) issue in batches of eight ring positions
//    of straight-line code: the batch's pointer fetches go back to back behind
//    one wait, then its vector accesses, all in flight together, addressed as a
//    scalar tile base plus one 32-bit lane offset.  Guarding each rank on its
//    own lets the compiler sink every fetch into its guard, which costs one
//    scalar round trip per rank before its access can issue; at p = 64 and
//    4 KiB per rank that was 16.6 us per call against 12.7 batched.  A run of
//    any length is whole batches and one shorter batch, picked by a wave-uniform
//    switch.
//  * Streaming calls (NT = true) take one rank at a time, each access behind its
//    own pointer fetch.  At 8 x 16 GB the batched issue measured 0.2% (loads)
//    and 0.6% (stores) slower: there the round trips hide behind HBM time and
//    the spaced issue streams slightly better.
constexpr int kRankBatch = 8;

// acc <- acc (op) x[first] (op) ... (op) x[first + N - 1], positions taken mod m
// and offset by base: rank base + (first + i) mod m.  first + N - 1 < 2m.
template <int N, bool NT, class F>
__device__ __forceinline__ void fold_batch(typename F::A& acc, const RankPtrs& P, int base, int m,
                                           int first, int64_t vt, unsigned lane, int p) {
  void* q[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int r = first + i;
    q[i] = P.b[base + (r >= m ? r - m : r)];
  }
  u32x4 x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = ld16t<NT>(q[i], vt, lane);
#pragma unroll
  for (int i = 0; i < N; ++i) acc = F::step(acc, x[i], p);
}

// Fold `count` ring positions starting at `first` (count >= 0, first + count - 1
// < 2m) in ring order, at vector vt + lane.
template <bool NT, class F>
__device__ __forceinline__ void fold_run(typename F::A& acc, const RankPtrs& P, int base, int m,
                                         int first, int count, int64_t vt, unsigned lane, int p) {
  if constexpr (NT) {
    const int64_t v = vt + lane;
    for (int k0 = 0; k0 < count; k0 += kRankBatch) {
      u32x4 x[kRankBatch];
#pragma unroll
      for (int i = 0; i < kRankBatch; ++i) {
        if (k0 + i < count) {
          const int r = first + k0 + i;
          x[i] = ld16<NT>(P.b[base + (r >= m ? r - m : r)], v);
        }
      }
#pragma unroll
      for (int i = 0; i < kRankBatch; ++i)
        if (k0 + i < count) acc = F::step(acc, x[i], p);
    }
  } else {
    for (; count >= kRankBatch; count -= kRankBatch, first += kRankBatch)
      fold_batch<kRankBatch, NT, F>(acc, P, base, m, first, vt, lane, p);
    switch (count) {
      case 7: fold_batch<7, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      case 6: fold_batch<6, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      case 5: fold_batch<5, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      case 4: fold_batch<4, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      case 3: fold_batch<3, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      case 2: fold_batch<2, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      case 1: fold_batch<1, NT, F>(acc, P, base, m, first, vt, lane, p); break;
      default: break;
    }
  }
}

// Store val as vector vt + lane of ranks r0 .. r0 + N - 1, except rank `skip`
// (-1: none).
template <int N, bool NT>
__device__ __forceinline__ void store_batch(const RankPtrs& P, int r0, int64_t vt, unsigned lane,
                                            u32x4 val, int skip) {
  void* q[N];
#pragma unroll
  for (int i = 0; i < N; ++i) q[i] = P.b[r0 + i];
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (r0 + i != skip) st16t<NT>(q[i], vt, lane, val);
}

// Store val as vector vt + lane of every rank except `skip` (-1: none).
template <bool NT>
__device__ __forceinline__ void store_all(const RankPtrs& P, int p, int64_t vt, unsigned lane,
                                          u32x4 val, int skip) {
  if constexpr (NT) {
    const int64_t v = vt + lane;
    for (int r = 0; r < p; ++r)
      if (r != skip) st16<NT>(P.b[r], v, val);
  } else {
    int r0 = 0;
    for (; p - r0 >= kRankBatch; r0 += kRankBatch)
      store_batch<kRankBatch, NT>(P, r0, vt, lane, val, skip);
    switch (p - r0) {
      case 7: store_batch<7, NT>(P, r0, vt, lane, val, skip); break;
      case 6: store_batch<6, NT>(P, r0, vt, lane, val, skip); break;
      case 5: store_batch<5, NT>(P, r0, vt, lane, val, skip); break;
      case 4: store_batch<4, NT>(P, r0, vt, lane, val, skip); break;
      case 3: store_batch<3, NT>(P, r0, vt, lane, val, skip); break;
      case 2: store_batch<2, NT>(P, r0, vt, lane, val, skip); break;
      case 1: store_batch<1, NT>(P, r0, vt, lane, val, skip); break;
      default: break;
    }
  }
}

// Split [lo, hi) into a scalar head, whole 16-byte vectors, and a scalar tail.
// All rank buffers start 16-byte aligned, so element i has the same alignment
// in every buffer.
// Tiles of a span count from vb, v0 rounded down to a 128-byte line (from the
// buffer's start), so that every wave's 1 KiB access covers whole lines; the
// vectors of the first tile below v0 belong to the span before and are left
// alone.  Tiles counted from v0 instead start mid-line whenever the span does
// (a chunk start that is not a multiple of 64 bfloat16), every access then
// touches one line more and the line two tiles share is fetched twice or
// written back in pieces: measured at p = 8 with 256 MiB of bfloat16 per rank,
// the one-pass all-reduce took 826 us with chunk starts 6 bytes past a line
// against 736 us with line-aligned ones.
struct Span {
  int64_t v0, v1;       // vector indices [v0, v1)
  int64_t vb;           // first vector of tile 0: v0 rounded down to a line
  int64_t head_hi;      // head = [lo, head_hi)
  int64_t tail_lo;      // tail = [tail_lo, hi)
};

template <int V>
__device__ __forceinline__ Span split_span(int64_t lo, int64_t hi) {
  Span s;
  int64_t a0 = (lo + V - 1) / V * V;
  int64_t a1 = hi / V * V;
  if (a0 >= a1) {                 // no whole vector: all scalar
    s.v0 = s.v1 = s.vb = 0;
    s.head_hi = hi;
    s.tail_lo = hi;
  } else {
    s.v0 = a0 / V;
    s.v1 = a1 / V;
    s.vb = s.v0 / kLineVecs * kLineVecs;
    s.head_hi = a0;
    s.tail_lo = a1;
  }
  return s;
}

// Tile tt of a launch over nseg segments of T tiles each: (segment tt / T, tile
// tt mod T), or, when the segments' last tiles are at most half full
// (tail_last, short_tail on the host), numbered so that every segment's last
// tile comes after all the others: tiles 0 .. nseg*(T-1) - 1 are (segment
// tt / (T-1), tile tt mod (T-1)), the last nseg are (segment tt - nseg*(T-1),
// tile T-1).  The dispatcher hands out workgroups in order, one per compute
// unit first, so the workgroups past the first round double up on compute units
// that already hold a tile; numbered segment by segment, those were whole
// tiles, and a compute unit moving two of them took twice as long: p = 64 with
// 8,256 bfloat16 per chunk (5 tiles of 256 vectors, the fifth 8 vectors) ran
// the one-pass all-reduce in 30.6 us, 26.9 with the short tiles last, against
// 24.8 for 8,192 per chunk (4 whole tiles); the slice-carrying ring 43.4 and
// 35.2 against 33.1.  With whole last tiles the plain order is kept (it
// measured 0.5 us faster there).  Tile counts stay below 2^32 (a tile holds at
// least 4 KiB of every rank; the launchers check), so the arithmetic is 32-bit:
// a 64-bit division is several times longer, and at one or two tiles per
// workgroup the decode is a visible part of a small call (p = 64 with 8,192
// bfloat16 per chunk: 25.8 us with 64-bit decoding, against 25.0 before the
// short-tile numbering).
__device__ __forceinline__ void tile_of(uint32_t tt, uint32_t T, uint32_t nseg, int tail_last,
                                        int* seg, int64_t* j) {
  const uint32_t full = tail_last ? nseg * (T - 1) : 0u;
  uint32_t s, k;
  if (tt < full) {
    s = tt / (T - 1);
    k = tt - s * (T - 1);
  } else if (tail_last) {
    s = tt - full;
    k = T - 1;
  } else {
    s = tt / T;
    k = tt - s * T;
  }
  *seg = (int)s;
  *j = (int64_t)k;
}

// ---------------------------------------------------------------- edge elements
// A segment's edge elements -- at most V - 1 before its first whole vector and
// V - 1 after its last (2V - 2 when it holds no whole vector) -- share a 16-byte
// vector with the neighbouring segment, whose fold order differs, so they are
// folded one by one.  One wave carries all of a segment's edge elements:
//  1. lane r loads rank r's copy of every edge element, all loads in flight at
//     once, into LDS: x[k][r];
//  2. lane k folds element k in the segment's order from LDS, leaves in x[k][r]
//     the value rank r is to store and in mask[k] the ranks that store;
//  3. lane r stores its rank's values.
// The loads take one memory round trip.  One element per thread, each lane
// fetching its ranks one after another, an element waited for p round trips in
// a row (2p while the pointers came from the kernel arguments), longer than the
// tiles of a small call take: p = 64 with 524,365 bfloat16 per rank, 172 us per
// one-pass all-reduce with 2p, 55 with batches of eight ranks, against 25 us
// for 524,288 elements (no edges).
constexpr int kWave = 64;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kEdgePass = 4;

template <int DT>
struct EdgeSlab {
  typedef typename Elem<DT>::S S;
  static constexpr int K = 2 * Elem<DT>::V - 2;
  // rows padded by one 32-bit word (or one element): lanes 0..K-1 reading the
  // same column of different rows then meet different LDS banks
  static constexpr int kRow = kMaxRanks + (sizeof(S) < 4 ? 4 / (int)sizeof(S) : 1);
  S x[K][kRow];
  uint64_t mask[K];
};

// LDS of an edge workgroup: the rank-pointer table and one slab per wave.  It
// is the kernel's dynamic LDS, sized at launch (sizeof, or 0 when no chunk has
// edge elements), so launches without edge elements allocate none.
template <int DT>
struct EdgeLds {
  void* lp[kMaxRanks];
  EdgeSlab<DT> slab[kWavesPerBlock];
};

template <int DT>
__device__ __forceinline__ EdgeLds<DT>& edge_lds() {
  extern __shared__ __align__(16) unsigned char ra_dynamic_lds[];
  return *reinterpret_cast<EdgeLds<DT>*>(ra_dynamic_lds);
}

// Bit r set for every rank r < p.
__device__ __forceinline__ uint64_t all_ranks(int p) {
  return p >= 64 ? ~0ull : (1ull << p) - 1;
}

// Copy the p rank pointers to LDS (every thread of the workgroup calls this).
__device__ __forceinline__ void load_rank_table(void** lp, const RankPtrs& P, int p) {
  if (threadIdx.x < (unsigned)p) lp[threadIdx.x] = P.b[threadIdx.x];
  __syncthreads();
}

// The edge elements of [lo, hi) (lo == hi: none), carried by the calling wave
// with its own slab; lp is the LDS copy of the p rank pointers.  Every thread of
// the workgroup calls this, since it holds workgroup barriers.  fold(slab, k)
// runs on lane k for each edge element k.
template <int DT, class FoldLane>
__device__ __forceinline__ void edge_wave(void* const* lp, int p, int64_t lo, int64_t hi,
                                          EdgeSlab<DT>& sl, FoldLane fold) {
  constexpr int V = Elem<DT>::V, K = EdgeSlab<DT>::K;
  const Span sp = split_span<V>(lo, hi);
  const int64_t nh = sp.head_hi - lo;
  const int ne = (int)(nh + (hi - sp.tail_lo));
  const int lane = (int)(threadIdx.x % kWave);
  auto index = [&](int k) { return k < nh ? lo + k : sp.tail_lo + (k - nh); };
  if (ne > 0 && lane < p) {
    // kEdgePass elements' loads at a time, which keeps the callers at their tile
    // code's register counts (all K at once took up to 61 registers and ran no
    // faster: p = 64 with 524,365 bfloat16 per rank, 31.0 us either way).
    // Elements past the last repeat it (loaded, not used), so the loads need no
    // guard.
    for (int k0 = 0; k0 < ne; k0 += kEdgePass) {
      typename Elem<DT>::S v[kEdgePass];
#pragma unroll
      for (int u = 0; u < kEdgePass; ++u)
        v[u] = ld1<DT>(lp[lane], index(k0 + u < ne ? k0 + u : ne - 1));
#pragma unroll
      for (int u = 0; u < kEdgePass; ++u)
        if (k0 + u < ne) sl.x[k0 + u][lane] = v[u];
    }
  }
  __syncthreads();
  if (lane < ne) fold(sl, lane);
  __syncthreads();
  if (ne > 0 && lane < p) {
    for (int k = 0; k < ne; ++k)
      if ((sl.mask[k] >> lane) & 1) st1<DT>(lp[lane], index(k), sl.x[k][lane]);
  }
}

}  // namespace ra
