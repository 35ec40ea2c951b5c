// Sustained matrix-core rate of this device, for the benchmark's roofline denominators.
//
// Every wave runs chains of independent v_mfma_f32_16x16x32_{f16,bf16} (the form the GEMMs and
// the attention use) on register operands, two waves per SIMD on every compute unit.  The host
// divides the executed flops by the event-timed duration (sustained TFLOP/s).
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int kChains = 8;  // independent accumulators per wave

// One in-place MFMA: accumulator registers are both source C and destination (written as
// inline assembly so that the register allocator cannot route the chains through copies).
template <typename T> struct MfmaInPlace;
template <> struct MfmaInPlace<f16> {
  static __device__ __forceinline__ void run(f32x4 &c, const f16x8 &a, const f16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
};
template <> struct MfmaInPlace<bf16> {
  static __device__ __forceinline__ void run(f32x4 &c, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
};

template <typename T>
__global__ __launch_bounds__(256) void k_mfma_rate(float *sink, int iters) {
  typedef typename Mfma<T>::v8 V8;
  V8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<T>(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = static_cast<T>(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x4 c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) MfmaInPlace<T>::run(c[j], a, b);
  }
  // the last MFMAs complete before their results are read (16 passes of wait)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  // the result is kept only so that the chains are not removed; it is never a real value
  if (s == 123456.f) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t mfma_rate(int op, int blocks, int iters, float *sink, hipStream_t s) {
  if (blocks < 1 || iters < 1) return hipErrorInvalidValue;
  if (op == OP_F16)
    k_mfma_rate<f16><<<blocks, 256, 0, s>>>(sink, iters);
  else if (op == OP_BF16)
    k_mfma_rate<bf16><<<blocks, 256, 0, s>>>(sink, iters);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// flops of one launch: every wave runs iters * kChains MFMAs of 16 x 16 x 32
double mfma_rate_flops(int blocks, int iters) {
  return (double)blocks * 4 * iters * kChains * (2.0 * 16 * 16 * 32);
}

}  // namespace dit
