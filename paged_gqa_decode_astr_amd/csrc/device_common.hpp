// Device helpers for the gfx950 kernels: bf16 rounding and wavefront
// (64-lane) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace astr {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// fp32 -> bf16 with round-to-nearest-even; NaN maps to a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Butterfly sum / max over lanes whose ids differ only in the bits of
// [FROM, TO) (powers of two); every participating lane gets the result.
template <int FROM, int TO>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int m = FROM; m < TO; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int FROM, int TO>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
  for (int m = FROM; m < TO; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

}  // namespace astr
