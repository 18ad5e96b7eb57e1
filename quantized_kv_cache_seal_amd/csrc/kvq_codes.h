// Code unpacking and operand helpers shared by the matrix-core attention
// kernels (decode and block attention): body key and value codes into exact
// centred fp16 operands, the q~ = q' C products, the staging of a
// sub-record's scales into LDS.
#pragma once
#include "kvq_mfma.h"

namespace kvq {

// ---------------------------------------------------------------------------
// Loads of the sealed records, which a scan reads once: non-temporal, so that
// the caches do not keep them (a streaming read of HBM with these loads ran
// 10-15 % faster than with ordinary ones, at every grid size measured).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
  const u32x4v v = __builtin_nontemporal_load((const u32x4v*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const uint8_t* p) {
  const u32x2v v = __builtin_nontemporal_load((const u32x2v*)p);
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------------------
// Code unpacking

// (a & m) | b in one v_and_or_b32.  The masks and the exponent pattern are
// passed in registers: a VOP3 instruction on this target cannot carry two
// literal constants, and the compiler otherwise splits it into an AND and an OR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t b) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(m), "v"(b));
  return d;
}

// Eight 4-bit value codes of one dword as exact, centred fp16 values.  One
// AND-OR per pair puts a nibble n into the mantissa of 1024 (the high nibble
// of a byte stays in place, i.e. 1024 + 16 n; its 1/16 is folded into the
// other operand) and one packed subtract leaves n - 8 (or 16 (n - 8)).
// Slots: [n0, n4, 16 n1, 16 n5, n2, n6, 16 n3, 16 n7] - centre.
// The value product needs the centre in the codes.  Uncentred, its sums run
// with one sign to ~8 sum(p S) per record, and the matrix cores' accumulation
// loses bits in proportion to them: 1e-3 to 3e-3 of the output at head width
// 256 and 512 (measured twice: with the centre taken from the exact weights,
// and from the rounded hi + lo weights by a product with a constant operand),
// against ~5e-5 centred.  The centre moves into the zero point instead:
// x = C (S (n - 8) + (Z + 8 S)).
__device__ __forceinline__ half8 nib8_centred(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const uint32_t lo_m = 0x000F000Fu, hi_m = 0x00F000F0u, e = 0x64006400u;
  uint4 u;
  u.x = and_or(w, lo_m, e);
  u.y = and_or(w, hi_m, e);
  u.z = and_or(w8, lo_m, e);
  u.w = and_or(w8, hi_m, e);
  const half8 off = {(_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1152.0f, (_Float16)1152.0f,
                     (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1152.0f, (_Float16)1152.0f};
  return mfma_a(u) - off;
}

// Key codes enter the score product as exact fp16 subnormals n 2^-24 (one AND
// per pair, no subtract: nib8_sub, byte8_sub), and the centre leaves the fp32
// product instead: q'.k_i = S_i 2^24 (q~ . n_i 2^-24 - mid sigma 2^-24) +
// (Z_i + mid S_i) sigma, mid = 2^(b-1).  The zero point Z_i is the row
// minimum, so the plain form S_i (q~ . n_i) + Z_i sigma runs both terms to the
// size of the row's range times |q~|, which then cancel to the score: with keys
// near the fp16 maximum (channels at +-60,000) they reach ~1e5 in fp32 for a
// score of ~1e3.  With the centre taken off the dot product before the scale
// multiplies, both terms stay at the size of the score; the dot product itself
// runs to at most twice its centred size (codes 0..2^b - 1 against -mid..mid).
// (Value codes stay centred in the operand: nib8_centred.)

// Eight 4-bit key codes of one dword as fp16 subnormals, in the slot order of
// nib8_centred: [n0, n4, 16 n1, 16 n5, n2, n6, 16 n3, 16 n7] 2^-24.
__device__ __forceinline__ half8 nib8_sub(uint32_t w) {
  const uint32_t w8 = w >> 8;
  uint4 u;
  u.x = w & 0x000F000Fu;
  u.y = w & 0x00F000F0u;
  u.z = w8 & 0x000F000Fu;
  u.w = w8 & 0x00F000F0u;
  return mfma_a(u);
}

// Eight 8-bit key codes of two dwords as fp16 subnormals n 2^-24 in channel
// order: one byte permute per pair (selector 4 takes a zero byte).
__device__ __forceinline__ half8 byte8_sub(uint32_t w0, uint32_t w1) {
  uint4 u;
  u.x = __builtin_amdgcn_perm(0u, w0, 0x04010400u);
  u.y = __builtin_amdgcn_perm(0u, w0, 0x04030402u);
  u.z = __builtin_amdgcn_perm(0u, w1, 0x04010400u);
  u.w = __builtin_amdgcn_perm(0u, w1, 0x04030402u);
  return mfma_a(u);
}
constexpr float kSub = 5.9604644775390625e-08f;  // 2^-24: the fp16 subnormal unit
constexpr float kUnSub = 16777216.0f;            // 2^24

__device__ __forceinline__ uint32_t pick(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// q~ = q' * C for one operand slot pair, split into hi + lo fp16 so that the
// score keeps fp32-level precision: q' = qh + ql 2^-11 (both fp16, ql scaled
// as split_h2s makes it), hi = fp16(qh C), lo = fp16((qh C - hi) 2^11 + ql C),
// with qh C - hi exact in fp32; q~ = hi + lo 2^-11.
__device__ __forceinline__ void qtilde_pair(uint32_t qh2, uint32_t ql2, uint32_t c2, uint32_t& hi2, uint32_t& lo2) {
  const half2v qh = as_h2(qh2), ql = as_h2(ql2), c = as_h2(c2);
  const half2v hi = qh * c;
  float r0 = fmaf((float)qh[0], (float)c[0], -(float)hi[0]);
  float r1 = fmaf((float)qh[1], (float)c[1], -(float)hi[1]);
  r0 = fmaf((float)ql[0], (float)c[0], r0 * kLoScale);
  r1 = fmaf((float)ql[1], (float)c[1], r1 * kLoScale);
  hi2 = as_u32(hi);
  lo2 = pack_h2(r0, r1);
}

__device__ __forceinline__ int slot_token(int p) {  // token at position p (0..7) of an 8-token group
  return (p >> 1) + 4 * (p & 1);
}

// Eight 8-bit key codes of two dwords as exact centred fp16 values n - 128 in
// channel order: one byte permute per pair puts n under the exponent byte of
// 1024 (selector 4 takes a byte of the 0x64 pattern), one packed subtract per
// pair removes 1024 + 128.
__device__ __forceinline__ half8 byte8_centred(uint32_t w0, uint32_t w1) {
  uint4 u;
  u.x = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
  u.y = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
  u.z = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
  u.w = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
  const half8 off = {(_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f,
                     (_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f};
  return mfma_a(u) - off;
}

// Thread tid's 8 bytes of a sub-record's scales (bytes 8 tid.. of the record's
// scale block) into the LDS layout of a record shape Sh (offsets L_KS .. L_VZ
// past the key C): key C copied, the rest as fp32 at twice the offset past it.
template <class Sh>
__device__ __forceinline__ void stage_scales(uint8_t* dst, uint2 m, int tid) {
  const int o = 8 * tid;
  if (o < 2 * Sh::SUBW) {
    *(uint2*)(dst + o) = m;
    return;
  }
  const half2v a = as_h2(m.x), b = as_h2(m.y);
  *(float4*)(dst + 2 * o - 2 * Sh::SUBW) = make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
}

// Eight consecutive B-bit codes (B = 2 or 3) at bits 0 .. 8 B - 1 of x as exact
// centred fp16 values c - 2^(B-1), in order.  The low half of u keeps x, the
// high half x >> B, so that one AND-OR per pair takes codes 2i and 2i + 1
// (after a shift of u by 2 B i) into the mantissas of 1024 + c; at 3 bits the
// last pair comes from x >> 18 the same way.
template <int B>
__device__ __forceinline__ half8 codes_lb(uint32_t x) {
  const uint32_t mm = ((1u << B) - 1) * 0x10001u, e = 0x64006400u;
  const uint32_t u0 = (x & 0xFFFFu) | ((x << (16 - B)) & 0xFFFF0000u);
  uint4 u;
  u.x = and_or(u0, mm, e);
  u.y = and_or(u0 >> (2 * B), mm, e);
  u.z = and_or(u0 >> (4 * B), mm, e);
  if (B == 2) {
    u.w = and_or(u0 >> (6 * B), mm, e);
  } else {
    const uint32_t x3 = x >> 18;
    u.w = and_or((x3 & 0xFFFFu) | ((x3 << 13) & 0xFFFF0000u), mm, e);
  }
  const _Float16 c = (_Float16)(1024.0f + (float)(1 << (B - 1)));
  const half8 off = {c, c, c, c, c, c, c, c};
  return mfma_a(u) - off;
}

// The same eight codes as fp16 subnormals c 2^-24, uncentred (keys: the
// centre leaves the fp32 product, as for nib8_sub).
template <int B>
__device__ __forceinline__ half8 codes_lb_sub(uint32_t x) {
  const uint32_t mm = ((1u << B) - 1) * 0x10001u;
  const uint32_t u0 = (x & 0xFFFFu) | ((x << (16 - B)) & 0xFFFF0000u);
  uint4 u;
  u.x = u0 & mm;
  u.y = (u0 >> (2 * B)) & mm;
  u.z = (u0 >> (4 * B)) & mm;
  if (B == 2) {
    u.w = (u0 >> (6 * B)) & mm;
  } else {
    const uint32_t x3 = x >> 18;
    u.w = ((x3 & 0xFFFFu) | ((x3 << 13) & 0xFFFF0000u)) & mm;
  }
  return mfma_a(u);
}

// Bits 8 B s .. 8 B s + 8 B - 1 of a lane's dwords d (the codes of its k-step s)
// in the low bits of the result (higher bits are ignored by codes_lb).
template <int B>
__device__ __forceinline__ uint32_t step_bits(const uint32_t* d, int s) {
  const int bit = 8 * B * s, w = bit >> 5, o = bit & 31;
  return o == 0 ? d[w] : o + 8 * B <= 32 ? d[w] >> o : __builtin_amdgcn_alignbit(d[w + 1], d[w], o);
}

}  // namespace kvq
