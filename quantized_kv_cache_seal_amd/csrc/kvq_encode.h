// tq6_0 staging encoder of one vector, shared by the append kernel and the
// fused decode step (the same bytes either way).
//
// SJ-KVaRN 2.1 items 1-2 and 2.2: every token past the sink is rotated and
// written to the staging ring as tq6_0 (98 bytes per 128 values).  128-wide
// heads use the randomized Walsh-Hadamard transform of the KV cache math page
// (sign flip, transform, sign flip).
//
// Exactness: a signed sum of at most 256 fp16 values is exact in binary64, so
// the butterflies run in double across the wave and the result is rounded once
// to fp32 (256-point: the /16 is exact; 128-point: one double multiply by
// 1/sqrt(128), then the second sign flip).  The quantiser is plain IEEE fp32:
// d = fp16(amax / 31), q = clamp(rne(x * fp32(1/d)), -31, 31), u = q + 32, and
// the 128 codes form an LSB-first 6-bit stream.
#pragma once
#include "kvq_device.h"

namespace kvq {

// VPL values per lane: 4 for a 256-point chunk (two tq6 blocks, 32 lanes
// each), 2 for a 128-point chunk (one block over the whole wave).  deq
// returns the lane's decoded values (rotated domain), element VPL lane + j.
template <int VPL>
__device__ __forceinline__ void encode_chunk(const uint16_t* __restrict__ src, uint8_t* __restrict__ codes,
                                             uint16_t* __restrict__ scales, int lane, const uint32_t* signs,
                                             bool rwht, float (&deq)[VPL]) {
  double x[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int i = VPL * lane + j;
    double v = (double)h2f(src[i]);
    if (rwht && sign_neg(signs, i)) v = -v;
    x[j] = v;
  }
  // butterflies inside the lane (strides 1 .. VPL/2)
#pragma unroll
  for (int st = 1; st < VPL; st <<= 1) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (!(j & st)) {
        const double p = x[j], q = x[j + st];
        x[j] = p + q;
        x[j + st] = p - q;
      }
    }
  }
  // butterflies across lanes (strides VPL .. 32*VPL): partner = lane ^ m
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const double o = shfl_xor_d(x[j], m);
      x[j] = (lane & m) ? (o - x[j]) : (x[j] + o);
    }
  }
  float yv[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    double r;
    if (rwht) {
      r = x[j] * kInvSqrt128;
      if (sign_neg(signs, 128 + VPL * lane + j)) r = -r;
    } else {
      r = x[j] * 0.0625;
    }
    yv[j] = (float)r;
  }

  constexpr int kLanesPerBlock = kQBlock / VPL;  // 32 or 64
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) am = fmaxf(am, fabsf(yv[j]));
#pragma unroll
  for (int m = 1; m < kLanesPerBlock; m <<= 1) am = fmaxf(am, shfl_xor_f(am, m));
  const uint16_t dbits = f2h_bits(am / 31.0f);
  const float d = h2f(dbits);
  const float inv = d > 0.0f ? 1.0f / d : 0.0f;
  int u[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    float q = rintf(yv[j] * inv);
    q = fminf(fmaxf(q, -31.0f), 31.0f);
    u[j] = (int)q + 32;
    deq[j] = d * q;  // the decoded value d (u - 32), exact in fp32
  }
  const int blk = lane / kLanesPerBlock;
  const int lb = lane % kLanesPerBlock;
  if (lb == 0) scales[blk] = dbits;
  uint32_t word;
  int byte_off;
  bool writer = true;
  if constexpr (VPL == 4) {
    word = (uint32_t)u[0] | ((uint32_t)u[1] << 6) | ((uint32_t)u[2] << 12) | ((uint32_t)u[3] << 18);
    byte_off = blk * kQBytes + 3 * lb;
  } else {
    const int p0 = __shfl_xor(u[0], 1, 64);
    const int p1 = __shfl_xor(u[1], 1, 64);
    word = (uint32_t)u[0] | ((uint32_t)u[1] << 6) | ((uint32_t)p0 << 12) | ((uint32_t)p1 << 18);
    byte_off = 3 * (lane >> 1);
    writer = !(lane & 1);
  }
  if (writer) {
    codes[byte_off + 0] = (uint8_t)(word & 0xFF);
    codes[byte_off + 1] = (uint8_t)((word >> 8) & 0xFF);
    codes[byte_off + 2] = (uint8_t)(word >> 16);
  }
}

}  // namespace kvq
