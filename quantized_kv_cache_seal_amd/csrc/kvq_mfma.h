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

// The same split with the remainder stored times 2^11 (kLoScale): x = hi +
// lo 2^-11.  The remainder is at most 2^-11 |hi|, so unscaled it falls into
// the fp16 subnormals (absolute precision 2^-24) whenever |x| < 2^-3, and a
// query operand near 0.1 keeps ~17 of its 22 bits; scaled, lo stays normal
// down to |x| ~ 2^-14.  The products of lo operands take the 2^-11 back
// (exact: a power of two).
constexpr float kLoScale = 2048.0f, kLoUnscale = 1.0f / 2048.0f;
__device__ __forceinline__ void split_h2s(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_h2(x0, x1);
  lo = pack_h2((x0 - h2f((uint16_t)hi)) * kLoScale, (x1 - h2f((uint16_t)(hi >> 16))) * kLoScale);
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

// Over the four lane groups of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48), with
// the 32- and 16-lane swaps of this target (each returns the lane's own value
// and its partner's, in some order): no trip through LDS.
__device__ __forceinline__ float xsum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}
__device__ __forceinline__ float xmax4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
// x + the value of lane l ^ 8 (within the 16-lane row: DPP row_ror:8)
__device__ __forceinline__ float add_x8(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
// The same for a packed hi/lo product whose columns 8..15 (lanes with bit 3
// set) carry scaled lo operands: those lanes take the 2^-11 back first, so
// lanes c and c + 8 add the same two values and get the same sum, bit for bit.
__device__ __forceinline__ float add_x8_lo(float x, int lane) {
  return add_x8((lane & 8) ? x * kLoUnscale : x);
}

// Eight 6-bit codes held as 48 bits (lo, low 16 bits of hi), as fp16 u - 32.
__device__ __forceinline__ half8 codes6_reg(uint32_t lo, uint32_t hi) {
  uint4 u;
  u.x = (lo & 63u) | ((lo << 10) & 0x3F0000u) | 0x64006400u;
  u.y = ((lo >> 12) & 63u) | ((lo >> 2) & 0x3F0000u) | 0x64006400u;
  u.z = ((lo >> 24) & 63u) | ((((lo >> 30) | (hi << 2)) & 63u) << 16) | 0x64006400u;
  u.w = ((hi >> 4) & 63u) | ((hi << 6) & 0x3F0000u) | 0x64006400u;
  const half8 off1056 = {(_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f,
                         (_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f};
  return mfma_a(u) - off1056;
}

// Transpose 4 tokens x 8 channels (one half8 per token) into 8 channel rows of
// 4 tokens: row e of the destination gets halves e of t0..t3.
__device__ __forceinline__ void store_t4x8(uint16_t* vt, int pitch, int row0, int col, const uint4 (&t)[4]) {
  const uint32_t* w0 = (const uint32_t*)&t[0];
  const uint32_t* w1 = (const uint32_t*)&t[1];
  const uint32_t* w2 = (const uint32_t*)&t[2];
  const uint32_t* w3 = (const uint32_t*)&t[3];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint2 r;
    r.x = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
    r.y = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
    *(uint2*)(vt + (row0 + e) * pitch + col) = r;
  }
}

}  // namespace kvq
