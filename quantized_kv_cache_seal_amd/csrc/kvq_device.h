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
// Profiling stamps of a kernel by the device wall clock: the start of
// workgroup 0, which the dispatcher launches first (one plain store: an atomic
// from every workgroup at launch would contend on one address and hold up each
// workgroup's first wait for memory), and the latest workgroup end (atomic
// max from one lane, after the workgroup's work).
__device__ __forceinline__ void prof_start(unsigned long long* ts) {
  if (ts && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    ts[0] = (unsigned long long)wall_clock64();
}
__device__ __forceinline__ void prof_end(unsigned long long* ts) {
  if (ts) {
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(&ts[1], (unsigned long long)wall_clock64());
  }
}
__device__ __forceinline__ bool sign_neg(const uint32_t* signs, int i) {
  return (signs[i >> 5] >> (i & 31)) & 1u;
}

// In-register Walsh-Hadamard transform of size N over one wave: lane l holds
// the VPL consecutive elements VPL l .. VPL l + VPL - 1 (N / VPL lanes per
// transform, so a wave holds 64 VPL / N independent transforms).  Butterflies
// of stride < VPL stay in the lane; larger strides pair lane l with l ^ (st / VPL).
template <int VPL, int N>
__device__ __forceinline__ void wave_fwht(float (&v)[VPL], int lane) {
#pragma unroll
  for (int st = 1; st < N; st <<= 1) {
    if (st < VPL) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (!(i & st)) {
          const float x = v[i], y = v[i + st];
          v[i] = x + y;
          v[i + st] = x - y;
        }
    } else {
      const bool upper = (lane & (st / VPL)) != 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const float o = __shfl_xor(v[i], st / VPL, 64);
        v[i] = upper ? o - v[i] : v[i] + o;
      }
    }
  }
}

// R^T of one D-vector held D / 64 values per lane (lane l: elements
// (D / 64) l ..): head_dim 128: s1 . H . s2 / sqrt(128); 256 and 512: H_256 / 16
// on each 256-point half.
template <int D>
__device__ __forceinline__ void rotate_back(float (&v)[D / 64], int lane, const uint32_t* signs) {
  constexpr int VPL = D / 64;
  if (D == 128) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (sign_neg(signs, 128 + VPL * lane + i)) v[i] = -v[i];
    wave_fwht<VPL, 128>(v, lane);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      v[i] *= (float)kInvSqrt128;
      if (sign_neg(signs, VPL * lane + i)) v[i] = -v[i];
    }
  } else {
    wave_fwht<VPL, 256>(v, lane);
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] *= 0.0625f;
  }
}

}  // namespace kvq
