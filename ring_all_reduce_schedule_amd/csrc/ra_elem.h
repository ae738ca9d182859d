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

namespace ra {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxRanks = 64;
constexpr int kBlock = 256;               // threads per workgroup (4 wave64s)

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
// dtype codes match ra_dtype: 0 int32, 1 float32, 2 bfloat16.

template <int DT> struct Elem;

template <> struct Elem<0> {                 // int32: wraps modulo 2^32
  static constexpr int V = 4;                // elements per 16-byte vector
  typedef uint32_t S;                        // storage of one element
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) { return a + b; }
  __device__ static __forceinline__ S add1(S a, S b) { return a + b; }
};

template <> struct Elem<1> {                 // float32: IEEE add, nearest even
  static constexpr int V = 4;
  typedef uint32_t S;
  __device__ static __forceinline__ u32x4 add(u32x4 a, u32x4 b) {
    f32x4 s = __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b);
    return __builtin_bit_cast(u32x4, s);
  }
  __device__ static __forceinline__ S add1(S a, S b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }
};

// bfloat16: both operands widened exactly to float32 (a bf16 is the top half of
// a float32), added in float32 (nearest even), narrowed back to bf16 (nearest
// even) with the gfx950 packed convert.  Rounding through float32 first gives
// the same result as rounding the exact sum once, because float32 carries more
// than twice bf16's precision plus two bits.
__device__ __forceinline__ uint32_t bf16_pair_add(uint32_t a, uint32_t b) {
  f32x2 s;
  s.x = __uint_as_float(a << 16) + __uint_as_float(b << 16);
  s.y = __uint_as_float(a & 0xffff0000u) + __uint_as_float(b & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(s, bf16x2));
}

template <> struct Elem<2> {
  static constexpr int V = 8;
  typedef uint16_t S;
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
};

// ---------------------------------------------------------------- memory access

// NT = true marks the access non-temporal (streaming): used when the buffers are
// far larger than the 256 MB Infinity Cache, so nothing would be re-read from it.
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
template <int DT>
__device__ __forceinline__ typename Elem<DT>::S ld1(const void* base, int64_t i) {
  return reinterpret_cast<const typename Elem<DT>::S*>(base)[i];
}
template <int DT>
__device__ __forceinline__ void st1(void* base, int64_t i, typename Elem<DT>::S v) {
  reinterpret_cast<typename Elem<DT>::S*>(base)[i] = v;
}

// Split [lo, hi) into a scalar head, whole 16-byte vectors, and a scalar tail.
// All rank buffers start 16-byte aligned, so element i has the same alignment
// in every buffer.
struct Span {
  int64_t v0, v1;       // vector indices [v0, v1)
  int64_t head_hi;      // head = [lo, head_hi)
  int64_t tail_lo;      // tail = [tail_lo, hi)
};

template <int V>
__device__ __forceinline__ Span split_span(int64_t lo, int64_t hi) {
  Span s;
  int64_t a0 = (lo + V - 1) / V * V;
  int64_t a1 = hi / V * V;
  if (a0 >= a1) {                 // no whole vector: all scalar
    s.v0 = s.v1 = 0;
    s.head_hi = hi;
    s.tail_lo = hi;
  } else {
    s.v0 = a0 / V;
    s.v1 = a1 / V;
    s.head_hi = a0;
    s.tail_lo = a1;
  }
  return s;
}

}  // namespace ra
