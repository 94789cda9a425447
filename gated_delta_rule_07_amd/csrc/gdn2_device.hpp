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

// -------------------------------------------------------------- fragments --
// Operand fragment in the matrix-core input type.
template <typename T> struct frag;
template <> struct frag<bf16_t> {
  s16x4 v;
  __device__ static __forceinline__ frag from(f32x4 x) {
    frag f;
    f.v[0] = static_cast<short>(f2bf(x[0]));
    f.v[1] = static_cast<short>(f2bf(x[1]));
    f.v[2] = static_cast<short>(f2bf(x[2]));
    f.v[3] = static_cast<short>(f2bf(x[3]));
    return f;
  }
  __device__ static __forceinline__ frag zero() {
    frag f;
    f.v = s16x4{0, 0, 0, 0};
    return f;
  }
  __device__ __forceinline__ f32x4 to_f32() const {
    f32x4 r;
    for (int i = 0; i < 4; ++i)
      r[i] = bf2f(static_cast<bf16_t>(v[i]));
    return r;
  }
  __device__ __forceinline__ frag neg() const {
    frag f;
    for (int i = 0; i < 4; ++i)
      f.v[i] = static_cast<short>(v[i] ^ static_cast<short>(0x8000));
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
  static constexpr int TILE_BYTES = 64 * 16;
};

// acc (ColFrag) += A (RowFrag) * B (ColFrag), one 16x16x16 product
__device__ __forceinline__ void mma16(f32x4 &acc, const frag<bf16_t> &a, const frag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4 &acc, const frag<float> &a, const frag<float> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc, 0, 0, 0);
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
