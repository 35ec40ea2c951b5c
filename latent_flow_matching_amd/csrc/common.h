// Shared device helpers of the gfx950 kernels: bf16 storage, wave reductions, vector types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// fp32 -> bf16 with round-to-nearest-even (gfx950 converts in hardware with RNE).
__device__ __forceinline__ bf16 to_bf16(float f) { return static_cast<bf16>(f); }
// fp32 -> fp16, round-to-nearest-even, saturating at the largest finite fp16 so that an
// out-of-range activation stays finite.
__device__ __forceinline__ f16 to_f16(float f) {
  return static_cast<f16>(fminf(fmaxf(f, -65504.f), 65504.f));
}
__device__ __forceinline__ float to_f32(bf16 h) { return static_cast<float>(h); }
__device__ __forceinline__ float to_f32(f16 h) { return static_cast<float>(h); }
__device__ __forceinline__ float to_f32(float f) { return f; }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { return to_bf16(f); }
template <> __device__ __forceinline__ f16 from_f32<f16>(float f) { return to_f16(f); }

// Conversion of values known to lie inside the fp16 range (no saturation step).
template <typename T> __device__ __forceinline__ T from_f32_inrange(float f) {
  return static_cast<T>(f);
}

// MFMA operand traits: 16-bit operand type -> 8-element vector, the 32x32x16 and the 16x16x32
// MFMAs.
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<f16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// store 4 consecutive values (8 bytes for 16-bit types, 16 bytes for fp32)
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
  bf16x4 v = {to_bf16(a), to_bf16(b), to_bf16(c), to_bf16(d)};
  *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(f16 *p, float a, float b, float c, float d) {
  f16x4 v = {to_f16(a), to_f16(b), to_f16(c), to_f16(d)};
  *reinterpret_cast<f16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4 *>(p) = v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// SiLU with the hardware reciprocal (1 ulp) instead of an IEEE division: z * 1 / (1 + e^-z),
// which still gives -0 for z -> -inf (e^-z = inf) and z for large z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// OCP E4M3 codes of four values, packed low byte first: each is clamped to +-448 and rounded
// to the nearest E4M3 value, ties to even mantissa (v_cvt_pk_fp8_f32 rounds that way on
// gfx950 but does not saturate: past 464 it gives the NaN code, hence the clamp).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

// Segment (0 text, 1 image, 2 reference) of token row m given the two boundaries.
__device__ __forceinline__ int segment_of(int m, int b1, int b2) {
  return (m >= b1) + (m >= b2);
}
// The same for row m of one of two sequences of per rows each (m < 2 * per).
__device__ __forceinline__ int segment_of(int m, int b1, int b2, int per) {
  return segment_of(m >= per ? m - per : m, b1, b2);
}

}  // namespace dit
