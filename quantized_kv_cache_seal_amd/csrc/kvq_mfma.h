// Helpers shared by the matrix-core decode kernels (v_mfma_f32_16x16x32_f16).
//
// Operand layouts of the 16x16x32 product D = A B + C, lane l of a wave:
//   A (16 x 32): row l & 15, columns 8 (l >> 4) .. 8 (l >> 4) + 7   (8 halves)
//   B (32 x 16): rows 8 (l >> 4) .. + 7, column l & 15                 (8 halves)
//   C, D (16 x 16, fp32): rows 4 (l >> 4) .. + 3, column l & 15        (4 floats)
#pragma once
#include "kvq_device.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ half8 mfma_a(const uint4& u) {
  half8 h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return (uint32_t)f2h_bits(lo) | ((uint32_t)f2h_bits(hi) << 16);
}

// x = hi + lo with hi = fp16(x) and lo = fp16(x - hi): 22 significant bits of
// x survive the fp16 operands of the matrix cores.
__device__ __forceinline__ void split_h2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_h2(x0, x1);
  lo = pack_h2(x0 - h2f((uint16_t)hi), x1 - h2f((uint16_t)(hi >> 16)));
}

__device__ __forceinline__ half2v as_h2(uint32_t u) {
  half2v h;
  __builtin_memcpy(&h, &u, 4);
  return h;
}
__device__ __forceinline__ uint32_t as_u32(half2v h) {
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

__device__ __forceinline__ float xsum4(float x) {  // sum over the four lane groups of a wave
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
__device__ __forceinline__ float xmax4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

}  // namespace kvq
