// Device helpers shared by the kernels: fp16 conversion, wave-level exchange,
// the fixed constants of the rotations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_layout.h"

namespace kvq {

typedef _Float16 half_t;

// 1/sqrt(128) correctly rounded to binary64.
constexpr double kInvSqrt128 = 0x1.6a09e667f3bcdp-4;

__device__ __forceinline__ float h2f(uint16_t b) {
  half_t h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}
__device__ __forceinline__ uint16_t f2h_bits(float x) {  // round to nearest even
  half_t h = (half_t)x;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}
// fp16 of x with saturation at +-65504 instead of overflow to infinity.
__device__ __forceinline__ uint16_t f2h_sat_bits(float x) {
  return f2h_bits(fminf(fmaxf(x, -65504.0f), 65504.0f));
}
__device__ __forceinline__ double shfl_xor_d(double x, int m) {
  return __shfl_xor(x, m, 64);
}
__device__ __forceinline__ float shfl_xor_f(float x, int m) {
  return __shfl_xor(x, m, 64);
}
__device__ __forceinline__ bool sign_neg(const uint32_t* signs, int i) {
  return (signs[i >> 5] >> (i & 31)) & 1u;
}

}  // namespace kvq
