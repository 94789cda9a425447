// gdn2_device.hpp -- device building blocks shared by the libgdn2 kernels
// (gfx950 / CDNA4, wave64).
//
// Fragment convention used by every matrix-core product in this library.
// A 16x16 tile X is spread over one wave; lane l has row/column index
// r = l % 16 and k-group g = l / 16, and holds four consecutive k values:
//   RowFrag(X): lane (r, g) holds X[r][4g .. 4g+3]   (A operand)
//   ColFrag(X): lane (c, g) holds X[4g .. 4g+3][c]   (B operand, accumulator)
// so RowFrag(X) == ColFrag(X^T).  mma16 adds RowFrag(A) * ColFrag(B) (a
// 16x16x16 product) into a ColFrag accumulator; for bf16 operands it is one
// v_mfma_f32_16x16x16_bf16, for float32 four v_mfma_f32_16x16x4_f32.  Because
// the accumulator has the B-operand layout, a product's result feeds the next
// product's B operand without any data movement, and
//   transpose(F) = mma16(F, ColFrag(I))
// turns a RowFrag into the ColFrag of the same matrix (and back), exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

// ---------------------------------------------------------------- scalars --
__device__ __forceinline__ float bf2f(bf16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}
// float -> bfloat16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ bf16_t f2bf(float x) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}

// Element type of the I/O tensors.
template <typename T> struct io;
template <> struct io<float> {
  typedef float elem;
  __device__ static __forceinline__ float to_f(float x) { return x; }
  __device__ static __forceinline__ float from_f(float x) { return x; }
  // 4 consecutive elements
  __device__ static __forceinline__ f32x4 load4(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
  }
  __device__ static __forceinline__ void store4(float *p, f32x4 x) {
    *reinterpret_cast<f32x4 *>(p) = x;
  }
};
template <> struct io<bf16_t> {
  typedef bf16_t elem;
  __device__ static __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
  __device__ static __forceinline__ bf16_t from_f(float x) { return f2bf(x); }
  __device__ static __forceinline__ f32x4 load4(const bf16_t *p) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    f32x4 r;
    r[0] = __builtin_bit_cast(float, u.x << 16);
    r[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
    r[2] = __builtin_bit_cast(float, u.y << 16);
    r[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
    return r;
  }
  __device__ static __forceinline__ void store4(bf16_t *p, f32x4 x) {
    uint2 u;
    u.x = static_cast<uint32_t>(f2bf(x[0])) | (static_cast<uint32_t>(f2bf(x[1])) << 16);
    u.y = static_cast<uint32_t>(f2bf(x[2])) | (static_cast<uint32_t>(f2bf(x[3])) << 16);
    *reinterpret_cast<uint2 *>(p) = u;
  }
};

// Four consecutive elements to global memory through an address-space(1)
// pointer (the compiler may then reorder LDS accesses around the store).
typedef __attribute__((address_space(1))) float gfloat_t;
typedef __attribute__((address_space(1))) bf16_t gbf16_t;
__device__ __forceinline__ void store4_global(gfloat_t *p, f32x4 x) {
  *reinterpret_cast<__attribute__((address_space(1))) f32x4 *>(p) = x;
}
__device__ __forceinline__ void store4_global(gbf16_t *p, f32x4 x) {
  typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
  u32x2 u;
  u.x = static_cast<uint32_t>(f2bf(x[0])) | (static_cast<uint32_t>(f2bf(x[1])) << 16);
  u.y = static_cast<uint32_t>(f2bf(x[2])) | (static_cast<uint32_t>(f2bf(x[3])) << 16);
  *reinterpret_cast<__attribute__((address_space(1))) u32x2 *>(p) = u;
}

// -------------------------------------------------------------- fragments --
// Operand fragment in the matrix-core input type.
template <typename T> struct frag;
template <> struct frag<bf16_t> {
  s16x4 v;
  __device__ static __forceinline__ frag from(f32x4 x) {
    frag f;  // two v_cvt_pk_bf16_f32 (round to nearest even)
    f.v = __builtin_bit_cast(s16x4, __builtin_convertvector(x, bf16x4));
    return f;
  }
  __device__ static __forceinline__ frag zero() {
    frag f;
    f.v = s16x4{0, 0, 0, 0};
    return f;
  }
  __device__ __forceinline__ f32x4 to_f32() const {
    return __builtin_convertvector(__builtin_bit_cast(bf16x4, v), f32x4);
  }
  __device__ __forceinline__ frag neg() const {
    frag f;  // flip the sign bits of the four halves
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
    f.v = __builtin_bit_cast(s16x4, __builtin_bit_cast(u32x2, v) ^ u32x2{0x80008000u, 0x80008000u});
    return f;
  }
  // fragment-ordered memory (LDS or global): 8 bytes per lane
  __device__ static __forceinline__ frag ld(const void *tile, int lane) {
    frag f;
    f.v = reinterpret_cast<const s16x4 *>(tile)[lane];
    return f;
  }
  __device__ __forceinline__ void st(void *tile, int lane) const {
    reinterpret_cast<s16x4 *>(tile)[lane] = v;
  }
  // this lane's 8 bytes at an address computed by the caller
  __device__ static __forceinline__ frag ld_at(const void *p) {
    frag f;
    f.v = *reinterpret_cast<const s16x4 *>(p);
    return f;
  }
  __device__ __forceinline__ void st_at(void *p) const { *reinterpret_cast<s16x4 *>(p) = v; }
  static constexpr int TILE_BYTES = 64 * 8;
};
template <> struct frag<float> {
  f32x4 v;
  __device__ static __forceinline__ frag from(f32x4 x) {
    frag f;
    f.v = x;
    return f;
  }
  __device__ static __forceinline__ frag zero() {
    frag f;
    f.v = f32x4{0.f, 0.f, 0.f, 0.f};
    return f;
  }
  __device__ __forceinline__ f32x4 to_f32() const { return v; }
  __device__ __forceinline__ frag neg() const {
    frag f;
    f.v = -v;
    return f;
  }
  __device__ static __forceinline__ frag ld(const void *tile, int lane) {
    frag f;
    f.v = reinterpret_cast<const f32x4 *>(tile)[lane];
    return f;
  }
  __device__ __forceinline__ void st(void *tile, int lane) const {
    reinterpret_cast<f32x4 *>(tile)[lane] = v;
  }
  __device__ static __forceinline__ frag ld_at(const void *p) {
    frag f;
    f.v = *reinterpret_cast<const f32x4 *>(p);
    return f;
  }
  __device__ __forceinline__ void st_at(void *p) const { *reinterpret_cast<f32x4 *>(p) = v; }
  static constexpr int TILE_BYTES = 64 * 16;
};

// acc (ColFrag) += A (RowFrag) * B (ColFrag), one 16x16x16 product
__device__ __forceinline__ void mma16(f32x4 &acc, const frag<bf16_t> &a, const frag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
// The float32 product is four 16x16x4 instructions, each from a zero
// accumulator, summed on the vector ALU: no product reads another's result
// as its accumulator (chained float32 accumulators whose destination
// differs from their source were measured to read stale values here).
__device__ __forceinline__ void mma16(f32x4 &acc, const frag<float> &a, const frag<float> &b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], z, 0, 0, 0);
  const f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], z, 0, 0, 0);
  const f32x4 p2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], z, 0, 0, 0);
  const f32x4 p3 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], z, 0, 0, 0);
  acc += (p0 + p1) + (p2 + p3);
}

// Product shapes and accumulators.  On gfx950 an accumulator written by a
// 16x16x16 bf16 product and read as the accumulator (srcC) of a 16x16x32 bf16
// product, or the other way round, needs at least 5 wait states in between
// (measured: with fewer, two of the four result registers are stale), and the
// compiler does not insert them.  Every accumulator chain in this library
// therefore uses a single product shape, or passes through a vector-ALU op
// (whose hazards the compiler does handle) when the shape changes.
//
// Two fragments of adjacent 16-wide k tiles, stored interleaved per lane
// (lane's tile-0 values, then its tile-1 values) so one vector load fetches
// both.  mma32 adds A * B over the 32 k values of the pair: for bf16 it is a
// single v_mfma_f32_16x16x32_bf16 whose k slot (g, i) is taken to mean k tile
// i / 4, index 4g + i % 4 in both operands -- any assignment of k values to
// slots gives the same sum as long as A and B agree, and this one makes a
// pair of ColFrag accumulators a valid B operand with no data movement.
template <typename T> struct frag2 {
  frag<T> lo, hi;
  __device__ static __forceinline__ frag2 ld(const void *base, int lane);
  __device__ __forceinline__ void st(void *base, int lane) const;
  __device__ static __forceinline__ frag2 make(const frag<T> &a, const frag<T> &b) {
    frag2 f;
    f.lo = a;
    f.hi = b;
    return f;
  }
};

typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

template <> __device__ __forceinline__ frag2<bf16_t> frag2<bf16_t>::ld(const void *base, int lane) {
  const s16x8 x = reinterpret_cast<const s16x8 *>(base)[lane];  // one 16-byte load
  frag2 f;
  f.lo.v = __builtin_shufflevector(x, x, 0, 1, 2, 3);
  f.hi.v = __builtin_shufflevector(x, x, 4, 5, 6, 7);
  return f;
}
template <> __device__ __forceinline__ frag2<float> frag2<float>::ld(const void *base, int lane) {
  const f32x4 *p = reinterpret_cast<const f32x4 *>(base) + 2 * lane;
  frag2 f;
  f.lo.v = p[0];
  f.hi.v = p[1];
  return f;
}

template <> __device__ __forceinline__ void frag2<bf16_t>::st(void *base, int lane) const {
  reinterpret_cast<s16x8 *>(base)[lane] = __builtin_shufflevector(lo.v, hi.v, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <> __device__ __forceinline__ void frag2<float>::st(void *base, int lane) const {
  f32x4 *p = reinterpret_cast<f32x4 *>(base) + 2 * lane;
  p[0] = lo.v;
  p[1] = hi.v;
}

__device__ __forceinline__ void mma32(f32x4 &acc, const frag2<bf16_t> &a, const frag2<bf16_t> &b) {
  const s16x8 av = __builtin_shufflevector(a.lo.v, a.hi.v, 0, 1, 2, 3, 4, 5, 6, 7);
  const s16x8 bv = __builtin_shufflevector(b.lo.v, b.hi.v, 0, 1, 2, 3, 4, 5, 6, 7);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x4 &acc, const frag2<float> &a, const frag2<float> &b) {
  mma16(acc, a.lo, b.lo);
  mma16(acc, a.hi, b.hi);
}

// Byte offset of the fragment of tile (r, kk) for `lane` in a tile array with
// NKK k tiles per row r: k tiles are paired (frag2 order) when NKK is even.
template <typename T, int NKK>
__host__ __device__ constexpr size_t tile_off(int r, int kk, int lane) {
  return (NKK % 2 == 0)
             ? ((static_cast<size_t>(r * (NKK / 2) + kk / 2) * 64 + lane) * 2 + (kk & 1)) * sizeof(frag<T>)
             : (static_cast<size_t>(r * NKK + kk) * 64 + lane) * sizeof(frag<T>);
}

// ColFrag of the 16x16 identity for this lane
template <typename T> __device__ __forceinline__ frag<T> identity_colfrag(int lane) {
  const int c = lane & 15, g = lane >> 4;
  f32x4 x;
  for (int i = 0; i < 4; ++i)
    x[i] = (4 * g + i == c) ? 1.f : 0.f;
  return frag<T>::from(x);
}

// Exact re-layout RowFrag <-> ColFrag of the same matrix (values already
// representable in T).
template <typename T>
__device__ __forceinline__ f32x4 transpose_frag(const frag<T> &x, const frag<T> &eye) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mma16(acc, x, eye);
  return acc;
}

// acc (ColFrag) += a (RowFrag) * b (ColFrag), operands rounded to CT: one
// 16x16x16 bfloat16 instruction accumulating in place, or the float32 form
// of mma16 above.
template <typename CT> __device__ __forceinline__ void mm(f32x4 &acc, f32x4 a, f32x4 b) {
  if constexpr (sizeof(CT) == 2) {
    mma16(acc, frag<CT>::from(a), frag<CT>::from(b));
  } else {
    mma16(acc, frag<float>::from(a), frag<float>::from(b));
  }
}

// RowFrag <-> ColFrag of one tile, exactly (a float32 identity product)
__device__ __forceinline__ f32x4 transpose_f32(f32x4 x, int lane);

// acc += a * b for fragments of the I/O type (the float32 form of mm)
template <typename T> __device__ __forceinline__ void mm_io(f32x4 &acc, const frag<T> &a, const frag<T> &b) {
  if constexpr (sizeof(T) == 2)
    mma16(acc, a, b);
  else
    mm<float>(acc, a.v, b.v);
}

// The same for a fragment of the I/O type (one bfloat16 product, or the
// float32 form above)
template <typename T> __device__ __forceinline__ f32x4 transpose_io(const frag<T> &x, const frag<T> &eye, int lane) {
  if constexpr (sizeof(T) == 2)
    return transpose_frag(x, eye);
  else
    return transpose_f32(x.v, lane);
}

__device__ __forceinline__ f32x4 transpose_f32(f32x4 x, int lane) {
  const int c = lane & 15, g = lane >> 4;
  f32x4 e;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    e[i] = (4 * g + i == c) ? 1.f : 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mm<float>(acc, x, e);
  return acc;
}

// A dk x dv float32 state handed between the backward's kernels as fragment
// tiles of the I/O type: the NK x NK tiles (kk, n) (rows 16kk.., columns
// 16n..) as ColFrag, then (float32 only: HAS_ROW) the same tiles as RowFrag.
// A bfloat16 reader forms the RowFrag of a tile from its ColFrag with one
// identity product (transpose_frag, exact), which costs less than moving a
// second copy through HBM.  BYTES per chunk-head.
template <typename IO, int D> struct state_tiles {
  static constexpr int NK = D / 16;
  static constexpr size_t TB = frag<IO>::TILE_BYTES;
  static constexpr bool HAS_ROW = sizeof(IO) != 2;
  static constexpr size_t COL = 0, ROW = static_cast<size_t>(NK) * NK * TB, BYTES = (HAS_ROW ? 2 : 1) * ROW;
  __host__ __device__ static constexpr size_t off(int kk, int n) { return static_cast<size_t>(kk * NK + n) * TB; }
};

// ------------------------------------------------------------- barriers --
// Workgroup barrier that orders LDS accesses only: LDS writes issued before it
// are complete and visible after it, but outstanding global loads and stores
// are not waited for (unlike __syncthreads()).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------ wave scans --
// Inclusive prefix sum over the 16 lanes of a DPP row (lanes 16g .. 16g+15).
__device__ __forceinline__ float row16_inclusive_scan(float x) {
  int xi;
  xi = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, false);
  x += __builtin_bit_cast(float, xi);
  xi = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xF, 0xF, false);
  x += __builtin_bit_cast(float, xi);
  xi = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xF, 0xF, false);
  x += __builtin_bit_cast(float, xi);
  xi = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xF, 0xF, false);
  x += __builtin_bit_cast(float, xi);
  return x;
}

// Value held by lane 15 of this lane's DPP row.
__device__ __forceinline__ float row16_last(float x, int lane) {
  return __shfl(x, (lane & ~15) | 15, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace gdn2
