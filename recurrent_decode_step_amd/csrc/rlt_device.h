// Device-side numerics shared by the decoder and encoder kernels: 16-byte
// fragment types, bf16 rounding, the per-type fragment helpers, one MFMA
// k-step, exact GELU and wavefront reductions.
#pragma once
#include "rlt_internal.h"

#include <math.h>

namespace rlt {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN), by the hardware
// conversion (v_cvt_pk_bf16_f32, two values per instruction)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}
// two values, lo in bits 0..15 and hi in bits 16..31
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Num;
template <> struct Num<float> {
  static constexpr int EPL = 4;          // elements per 16-byte fragment
  __device__ static void unpack(const u32x4 &v, float *f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static u32x4 pack(const float *f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
  __device__ static float round(float v) { return v; }
  __device__ static void store4(float *p, const float *y) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{y[0], y[1], y[2], y[3]};
  }
  __device__ static void store1(float *p, float y) { *p = y; }
};
template <> struct Num<bf16_t> {
  static constexpr int EPL = 8;
  __device__ static void unpack(const u32x4 &v, float *f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static u32x4 pack(const float *f) {
    return u32x4{f2bf2(f[0], f[1]), f2bf2(f[2], f[3]), f2bf2(f[4], f[5]), f2bf2(f[6], f[7])};
  }
  __device__ static float round(float v) { return bf2f(f2bf(v)); }
  __device__ static void store4(bf16_t *p, const float *y) {
    *reinterpret_cast<u32x2 *>(p) = u32x2{f2bf2(y[0], y[1]), f2bf2(y[2], y[3])};
  }
  __device__ static void store1(bf16_t *p, float y) { *p = (bf16_t)f2bf(y); }
};

// One MFMA k-step: 16 weight rows x 16 batch columns x (32 bf16 | 16 fp32) k.
// Lane l holds weight row (l & 15) and batch column (l & 15); its 16-byte
// fragment covers k = (l >> 4) * EPL .. +EPL-1 of the step in both operands,
// so the products of A and B pair the same k.
__device__ __forceinline__ f32x4 mma_step(const u32x4 &a, const u32x4 &b, f32x4 c, bf16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_step(const u32x4 &a, const u32x4 &b, f32x4 c, float) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float gelu_erf(float y) {
  return 0.5f * y * (1.0f + erff(y * 0.70710678118654752440f));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

}  // namespace rlt
