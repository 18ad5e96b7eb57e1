// Seal: one workgroup (4 waves) turns one 128-token x SUB-channel tile of the
// staging ring into one half of a body sub-record (K or V).
//
// SJ-KVaRN 2.1 item 4: full 128-token groups older than the newest tail are
// compressed into body records in one batch.  2.2: the tile is balanced by
// alternating row and column passes in the log domain (rows first), keeping the
// final column scales C (row factors are absorbed by the per-row scale and
// zero point), then each row is rounded to the target width with its own fp16
// scale S and zero point Z.
//
// Balancing on the matrix cores.  The tile is x_ij = d_ib q_ij with q = u - 32
// an integer in [-31, 31] (exact in fp16) and d_ib the tq6_0 scale of row i's
// 128-value block b.  A pass needs two sums per row (or column) of the tile
// scaled by the other side's factors:
//   rows:    s_i = sum_b d_ib sum_{j in b} q_ij c_j,   s2_i = sum_b d_ib^2 sum_j q_ij^2 c_j^2
//   columns: t_j = sum_i q_ij (d_ib r_i),              t2_j = sum_i q_ij^2 (d_ib r_i)^2
// i.e. matrix-vector products, done as v_mfma_f32_16x16x32_f16 with the tile
// (or its square, exact up to 961) as the A operand and the factor vector in B
// (fp16 hi in the even columns, fp16 lo, the remainder, in the odd ones), so
// each factor keeps 22 significant bits and every product is exact; a column
// pair of the result is added.  Row passes take the tile from registers (8
// consecutive columns of one row per lane, their squares kept beside them);
// column passes read 8 consecutive rows of one column per lane from a
// row-major copy in LDS by transpose loads, two k-steps ahead of the products.
// The updated side's factor is 1/spread (equal to exp(-l) of the
// log-domain update l += ln spread, spread the population standard deviation);
// a row or column of zeros (zero sum of squares: every product is exact, so
// that sum is zero only then) keeps its factor and log scale; the factors pass
// between waves through LDS, one barrier per pass.
//
// Tiles the fp32 passes cannot resolve go through binary64 instead.  The
// one-pass variance E[y^2] - mean^2 loses bits in proportion to mean^2 /
// variance, and the fp16 hi + lo operands hold a factor to 22 bits only within
// a range of magnitudes.  So the tile is flagged, and balanced again from the
// start in binary64 on the vector ALU (balance_f64: the passes exactly as
// defined, the spread taken about the first element, so that equal values give
// exactly zero, and a spread at or below 2^-40 of the RMS counting as zero),
// when in any pass a nonzero row or column has a spread at or below 1/8 of its
// RMS (kIllCond: the cancellation then costs at most 6 of fp32's 24 bits), or
// a factor leaves the range in which its hi + lo operands and those of its
// square keep ~2^-18 relative precision and stay finite.  Real caches are
// rotated first, which spreads every channel's energy over the tile, so their
// tiles stay on the fast path; repeated tokens, constant channels far above
// their spread, and channels orders of magnitude below the rest take the
// exact one.
//
// The balancing factors (1/spread, ln spread) use the hardware reciprocal
// square root and log2 of the variance (about 1 ulp): only the column scales C leave the
// balancing, and they are rounded to fp16.  Rounding is IEEE fp32 with no
// fused multiply-add (built with -ffp-contract=off): y = x * fp32(1/C),
// S = fp16((max - min) / (2^b - 1)) (1.0 if zero), Z = fp16(min),
// code = clamp(rne((y - Z) * fp32(1/S)), 0, 2^b - 1) (the clamp as one median
// of three, the same value for every finite input); x = d q as one mixed
// fp16 x fp32 multiply (mul_e), the codes packed as bytes (store_codes8).
#include "kvq_mfma.h"

namespace kvq {

// The fast passes flag a tile for the binary64 passes when a nonzero row or
// column has variance <= kIllCond * mean square (spread <= RMS / 8).
constexpr float kIllCond = 0.015625f;  // 2^-6
// Factors enter the matrix cores pre-scaled by a power of two (column factors
// c by kCScale, row factors d r by kRScale, so that typical balanced tiles sit
// near 1 to 4) and must then lie in [kFMin, kFMax]: f^2 below 65504 in fp16,
// and f, f^2 at or above 2^-3, 2^-6, where the fp16 hi + lo pair still
// carries ~2^-18 of the value.  A factor outside flags the tile.
constexpr float kCScale = 4.0f, kRScale = 16.0f;
constexpr float kFMin = 0.125f, kFMax = 255.0f;
// binary64 passes: a spread at or below 2^-40 of the RMS counts as zero
constexpr double kZeroSpread64 = 9.094947017729282e-13;  // 2^-40

template <int SUBW>
struct SealShape {
  static constexpr int NB = SUBW / kQBlock;  // tq6_0 blocks per row
  static constexpr int KR = SUBW / 32;       // row-pass k-steps (32 columns each)
  static constexpr int CT = SUBW / 64;       // column tiles (16 columns) per wave
  // LDS: the tile q, row-major fp16 (tile_half), from the load to the last
  // rounding; the binary64 passes of a flagged tile take the area for their
  // own state
  static constexpr int BYTES = 128 * SUBW * 2;
};

// Half index of tile element (r, c) in LDS: rows of SUBW halves, the row's
// 16-byte chunks permuted by an XOR with 2 ((r & 3) | ((r >> 3) & 1) << 2), so
// that a transpose load (load_col8) of 4 + 4 rows x 2 chunks per half-wave
// meets 16 distinct chunk positions modulo 16: no bank conflicts.
template <int SUBW>
__device__ __forceinline__ int tile_half(int r, int c) {
  return r * SUBW + 8 * ((c >> 3) ^ (2 * ((r & 3) | (((r >> 3) & 1) << 2)))) + (c & 7);
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// The column layout of the tile (the A operand of a column pass, 8 rows of one
// column per lane) by two LDS transpose loads (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, element k of lane j's result is element j & 3 of the
// four halves that lane 4 k + (j >> 2) of the group addresses.  So lane L of
// group g addresses row r0 + 8 g + (L >> 2) (4 more for the second load) at
// columns c0 + 4 (L & 3) .. + 3, and lane (j, g) receives column c0 + j, rows
// r0 + 8 g .. + 7.  c0 a multiple of 16, r0 of 8.
template <int SUBW>
__device__ __forceinline__ half8 load_col8(const uint16_t* tile, int r0, int c0, int l) {
  const int L = l & 15, r = r0 + 8 * (l >> 4) + (L >> 2), c = c0 + 4 * (L & 3);
  const __attribute__((address_space(3))) uint16_t* t = (const __attribute__((address_space(3))) uint16_t*)tile;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(t + tile_half<SUBW>(r, c)));
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(t + tile_half<SUBW>(r + 4, c)));
  half8 h;
  __builtin_memcpy(&h, &a, 8);
  __builtin_memcpy((char*)&h + 8, &b, 8);
  return h;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// over lanes l, l ^ 16, l ^ 32, l ^ 48 (the 32- and 16-lane swaps of this
// target: each returns the lane's own value and its partner's, in some order)
__device__ __forceinline__ float sum_x16x32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}
__device__ __forceinline__ float min_x16x32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fminf(__int_as_float(a[0]), __int_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fminf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float max_x16x32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

// element i (a per-lane index) of a 4-vector
__device__ __forceinline__ float pick4(const float4v& v, int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// x as the fp16 pair hi = fp16(x), lo = fp16(x - hi), element i of two arrays
__device__ __forceinline__ void put_hilo(uint16_t* hi, uint16_t* lo, int i, float x) {
  const uint16_t hb = f2h_bits(x);
  hi[i] = hb;
  lo[i] = f2h_bits(x - h2f(hb));
}

// q^2 of a packed operand (exact: |q| <= 31) as fma(q, q, z) with z a zero
// that every pass reads from LDS, so that the compiler forms each square in
// the pass that uses it; the packed FMAs are ordinary instructions, whose
// hazards with the matrix cores the compiler tracks (it inserts the wait
// states a product reading a just-written VGPR needs, and never hands a
// register that an in-flight product will still write to them -- neither
// holds for VGPRs written inside inline asm).
__device__ __forceinline__ half8 sq8(half8 v, half8 z) { return __builtin_elementwise_fma(v, v, z); }

// fp32(d * x) for element e of a packed fp16 operand in one instruction:
// v_fma_mix_f32 reads x as fp16 and adds nz = -0, the identity of every
// product (signed zeros included), so the result is the product rounded once
// to fp32, as a v_mul_f32 after the conversion would give.  Written out (the
// compiler folds a -0 addend into a plain multiply) and volatile, so that the
// second rounding sweep over the tile recomputes y instead of keeping the
// first sweep's 64 values per row alive.
__device__ __forceinline__ float mul_e(float d, const half8& v, int e, float nz) {
  uint4 u;
  __builtin_memcpy(&u, &v, 16);
  const uint32_t wd = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
  float r;
  if (e & 1)
    asm volatile("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(d), "v"(wd), "v"(nz));
  else
    asm volatile("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(d), "v"(wd), "v"(nz));
  return r;
}
// the same product, not volatile: the compiler may share it and move loads
// across it (the value codes' sweep, whose per-row operands come from LDS)
__device__ __forceinline__ float mul_e_pure(float d, const half8& v, int e, float nz) {
  uint4 u;
  __builtin_memcpy(&u, &v, 16);
  const uint32_t wd = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
  float r;
  if (e & 1)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(d), "v"(wd), "v"(nz));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(d), "v"(wd), "v"(nz));
  return r;
}
// -0.0f, opaque to the compiler
__device__ __forceinline__ float neg_zero() {
  float z = -0.0f;
  asm volatile("" : "+v"(z));
  return z;
}

// Eight consecutive b-bit codes (code e at bits b e of an LSB-first stream)
// as the b bytes at p: 8-, 4- and 2-bit groups are aligned words, a 3-bit
// group three bytes (p is then only byte-aligned).
__device__ __forceinline__ void put_codes8(uint8_t* p, const uint32_t (&cq)[8], int bits) {
  uint64_t v = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) v |= (uint64_t)cq[e] << (bits * e);
  if (bits == 8) {
    *(uint2*)p = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
  } else if (bits == 4) {
    *(uint32_t*)p = (uint32_t)v;
  } else if (bits == 2) {
    *(uint16_t*)p = (uint16_t)v;
  } else {
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
  }
}

// Eight codes held as fp32 integers in [0, 2^b - 1] (rounded and clamped),
// stored as put_codes8 does.  4 and 8 bits: bytes formed as exact fp32 sums
// (c0 + 16 c1 for two 4-bit codes) and inserted by v_cvt_pk_u8_f32, whose
// conversion of an integer in [0, 255] is that integer; other widths go
// through 32-bit integers.
template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t* p, const float (&cf)[8], int bits) {
  if constexpr (BITS == 4) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(16.0f, cf[2 * k + 1], cf[2 * k]), k, w);
    *(uint32_t*)p = w;
  } else if constexpr (BITS == 8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w0 = __builtin_amdgcn_cvt_pk_u8_f32(cf[k], k, w0);
      w1 = __builtin_amdgcn_cvt_pk_u8_f32(cf[k + 4], k, w1);
    }
    *(uint2*)p = make_uint2(w0, w1);
  } else {
    uint32_t cq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cq[e] = (uint32_t)cf[e];
    put_codes8(p, cq, bits);
  }
}

template <int SUBW>
struct SealLds {
  uint8_t smem[SealShape<SUBW>::BYTES] __attribute__((aligned(16)));
  // B operands: [q, q^2][hi, lo][SUBW] fp16 of the row pass (c, c^2);
  // [NB][q, q^2][hi, lo][128] of the column pass (d r, (d r)^2)
  uint16_t cfl[2 * 2 * SUBW] __attribute__((aligned(16)));
  uint16_t rfl[SealShape<SUBW>::NB * 2 * 2 * 128] __attribute__((aligned(16)));
  float ds[SealShape<SUBW>::NB][kGroup];     // d_ib
  float lcs[SUBW] __attribute__((aligned(16)));   // ln spread of each column (last column pass)
  float invc[SUBW] __attribute__((aligned(16)));  // fp32(1 / C_j)
  float rinv[kGroup];                       // fp32(1 / S_i)
  float zrow[kGroup];                       // Z_i
  float red[4];
  double red64[4];
  int bad[2];  // fast passes: tile flagged in a pass of this parity
  uint4 zero16;  // fp16 zeros, read every pass (sq8)
};

// Binary64 balancing of a flagged tile, from the start: the passes as
// defined (SJ-KVaRN 2.2: alternating row and column passes, rows first, log
// domain, keep the final scales), y_ij = ((q_ij d_ib) exp(-lr_i)) exp(-lc_j),
// the spread of a row or column the population standard deviation about its
// first element (exactly zero when its values are equal) and zero at or below
// 2^-40 of its RMS, in which case the log scale is kept.  The tile's codes are
// copied from the row-layout registers into an int8 tile in LDS (the factor
// exchange is no longer needed), followed by lr, lc and their exponentials.
// Writes C (fp16) to meta and fp32(1 / C) to invc.
template <int SUBW>
__device__ __forceinline__ void balance_f64(SealLds<SUBW>& L, const half8 (&ar)[2][SUBW / 32], int passes,
                                            uint8_t* meta) {
  using Sh = SealShape<SUBW>;
  constexpr int KR = Sh::KR;
  static_assert(128 * SUBW + 8 * 2 * (128 + SUBW) <= Sh::BYTES, "binary64 state fits the tile's LDS");
  int8_t* qs = (int8_t*)L.smem;                      // [128][SUBW]
  double* lr = (double*)(L.smem + 128 * SUBW);       // [128]
  double* lc = lr + 128;                             // [SUBW]
  double* fr = lc + SUBW;                            // [128] exp(-lr)
  double* fc = fr + 128;                             // [SUBW] exp(-lc)
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      uint32_t wd[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) wd[e >> 2] |= ((uint32_t)(int)(float)ar[t][kk][e] & 0xFFu) << (8 * (e & 3));
      *(uint2*)(qs + (16 * (2 * w + t) + m) * SUBW + 32 * kk + 8 * g) = make_uint2(wd[0], wd[1]);
    }
  for (int i = tid; i < 128 + SUBW; i += 256) lr[i] = 0.0;  // lr and lc are contiguous
  __syncthreads();
  const int hf = tid & 1;
  for (int p = 0; p < passes; ++p) {
    for (int i = tid; i < 128 + SUBW; i += 256) fr[i] = exp(-lr[i]);  // fr, fc mirror lr, lc
    __syncthreads();
    if ((p & 1) == 0) {
      // row tid / 2, columns hf SUBW / 2 .. + SUBW / 2 (one tq6_0 block at 256 wide)
      const int row = tid >> 1, c0 = hf * (SUBW / 2);
      const double frow = fr[row];
      const double ref = ((double)qs[row * SUBW] * (double)L.ds[0][row]) * frow * fc[0];
      double s1 = 0.0, s2 = 0.0, sq = 0.0;
      for (int c = c0; c < c0 + SUBW / 2; c += 4) {
        const double d = (double)L.ds[c / kQBlock][row];
        const char4 q4 = *(const char4*)(qs + row * SUBW + c);
        const int qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double yy = ((double)qv[e] * d) * frow * fc[c + e], dv = yy - ref;
          s1 += dv;
          s2 += dv * dv;
          sq += yy * yy;
        }
      }
      s1 += __shfl_xor(s1, 1, 64);
      s2 += __shfl_xor(s2, 1, 64);
      sq += __shfl_xor(sq, 1, 64);
      const double mean = s1 / SUBW, var = fmax(s2 / SUBW - mean * mean, 0.0), sig = sqrt(var);
      if (hf == 0 && sig > kZeroSpread64 * sqrt(sq / SUBW)) lr[row] += log(sig);
    } else {
      // column tid (256 wide), or tid / 2 with rows hf 64 .. + 64 (128 wide)
      constexpr int TPC = 256 / SUBW, NR = 128 / TPC;
      const int col = tid / TPC, r0 = TPC == 2 ? hf * NR : 0;
      const double dcol0 = (double)L.ds[col / kQBlock][0];
      const double fcol = fc[col];
      const double ref = ((double)qs[col] * dcol0) * fr[0] * fcol;
      double s1 = 0.0, s2 = 0.0, sq = 0.0;
      for (int r = r0; r < r0 + NR; ++r) {
        const double yy = ((double)qs[r * SUBW + col] * (double)L.ds[col / kQBlock][r]) * fr[r] * fcol,
                     dv = yy - ref;
        s1 += dv;
        s2 += dv * dv;
        sq += yy * yy;
      }
      if (TPC == 2) {
        s1 += __shfl_xor(s1, 1, 64);
        s2 += __shfl_xor(s2, 1, 64);
        sq += __shfl_xor(sq, 1, 64);
      }
      const double mean = s1 / kGroup, var = fmax(s2 / kGroup - mean * mean, 0.0), sig = sqrt(var);
      if ((TPC == 1 || hf == 0) && sig > kZeroSpread64 * sqrt(sq / kGroup)) lc[col] += log(sig);
    }
    __syncthreads();
  }
  // centre, clamp to [-9, 9], C = fp16(exp(lc))
  double v = tid < SUBW ? lc[tid] : 0.0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  if (l == 0) L.red64[w] = v;
  __syncthreads();
  const double lmean = (L.red64[0] + L.red64[1] + L.red64[2] + L.red64[3]) / SUBW;
  if (tid < SUBW) {
    const double c = fmin(fmax(lc[tid] - lmean, -9.0), 9.0);
    const half_t ch = (half_t)exp(c);
    uint16_t cb;
    __builtin_memcpy(&cb, &ch, 2);
    ((uint16_t*)meta)[tid] = cb;
    L.invc[tid] = 1.0f / h2f(cb);
  }
  __syncthreads();
}

// One tile; KV (0 keys, 1 values) is a compile-time choice so that the keys'
// path holds one copy of the tile once the balancing is done.  BITS is the
// code width when known at compile time (the 4- and 8-bit bodies: constant
// shifts in the packing), 0 to read it from the layout.
template <int SUBW, int KV, int BITS>
__device__ __forceinline__ void seal_tile(const SealArgs& a, SealLds<SUBW>& L, int r, int sub, int h, int s,
                                          int layer) {
  using Sh = SealShape<SUBW>;
  constexpr int NB = Sh::NB, KR = Sh::KR, CT = Sh::CT;
  constexpr int kv = KV;
  const Layout& y = a.y;
  uint8_t* smem = L.smem;
  auto& ds = L.ds;
  float* lcs = L.lcs;
  float* invc = L.invc;
  float* rinv = L.rinv;
  float* zrow = L.zrow;
  float* red = L.red;
  uint16_t* tile = (uint16_t*)smem;  // q, row-major (tile_half)
  uint16_t* cfl = L.cfl;
  uint16_t* rfl = L.rfl;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int slot0 = (int)(((int64_t)r * kGroup) % y.cap);
  auto slot_of = [&](int row) { const int t = slot0 + row; return t >= y.cap ? t - y.cap : t; };
  // ring rows of this (K|V) head; the sub-tile's channels start at block sub * NB
  const int64_t row_bytes = (int64_t)y.NB * kQBytes;
  const uint8_t* codes = a.arena + rcode_off(y, s, layer, h, kv, 0) + (int64_t)sub * NB * kQBytes;
  const uint8_t* scales = a.arena + rscale_off(y, s, layer, h, kv, 0) + 2 * sub * NB;

  // ---- the tile, row layout: ar[t][kk] = q of row 16 (2w + t) + m, columns
  // 32 kk + 8 g .. + 7 (the A operand of a row pass)
  half8 ar[2][KR];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint8_t* row = codes + (int64_t)slot_of(16 * (2 * w + t) + m) * row_bytes + ((6 * g) & ~3);
    const uint32_t sh = (g & 1) ? 16u : 0u;
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      const uint32_t* p = (const uint32_t*)(row + 24 * kk);
      const uint32_t lo = p[0], hi = p[1];
      ar[t][kk] = codes6_reg(__builtin_amdgcn_alignbit(hi, lo, sh), hi >> sh);
    }
  }
  // the same tile in LDS for the column layout (load_col8)
  auto put_tile = [&]() {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < KR; ++kk) {
        uint4 u;
        __builtin_memcpy(&u, &ar[t][kk], 16);
        *(uint4*)(tile + tile_half<SUBW>(16 * (2 * w + t) + m, 32 * kk + 8 * g)) = u;
      }
  };
  put_tile();
  // block scales d of every row
  for (int i = tid; i < NB * kGroup; i += 256) {
    const int row = i % kGroup, b = i / kGroup;
    ds[b][row] = h2f(*(const uint16_t*)(scales + (int64_t)slot_of(row) * (y.NB * 2) + 2 * b));
  }
  for (int j = tid; j < SUBW; j += 256) {  // first row pass: c = 1, pre-scaled (hi kCScale, lo 0)
    cfl[0 * SUBW + j] = f2h_bits(kCScale);
    cfl[1 * SUBW + j] = 0;
    cfl[2 * SUBW + j] = f2h_bits(kCScale * kCScale);
    cfl[3 * SUBW + j] = 0;
    lcs[j] = 0.0f;
  }
  if (tid < 2) L.bad[tid] = 0;
  if (tid == 0) L.zero16 = make_uint4(0u, 0u, 0u, 0u);
  // q^2 of the row layout (exact: |q| <= 31), the A operand of the row passes'
  // second moments; the column passes square their operands as they load them
  half8 ar2[2][KR];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) ar2[t][kk] = ar[t][kk] * ar[t][kk];
  __syncthreads();

  // B carries the factor's fp16 hi in its even columns and lo in its odd ones
  // (the same 16 values in every column pair), so every lane ends with sums of
  // its rows: lane m of lane group g holds rows 4 g .. + 3 (hi part for even m,
  // lo for odd), and the pair (m, m ^ 1) adds them with one DPP step.  Each
  // lane pair then takes its own row (or columns) for the statistics.
  const int wb = SUBW == 256 ? (w >> 1) : 0;  // the block of this wave's columns
  const int pr = m >> 1;                       // lane pair 0..7
  constexpr int NCL = CT / 2;                  // columns per lane pair in a column pass
  // the factors of this lane pair's row and columns from their last update:
  // a row or column of zeros keeps them (and its log scale)
  float rf_keep = 1.0f, cf_keep[NCL], lc_keep[NCL];
#pragma unroll
  for (int e = 0; e < NCL; ++e) {
    cf_keep[e] = 1.0f;
    lc_keep[e] = 0.0f;
  }

  // d of this lane pair's row in a row pass (row 16 (2w + t) + 4 g + i, t = pr / 4, i = pr % 4)
  float drow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) drow[b] = ds[b][16 * (2 * w + (pr >> 2)) + 4 * g + (pr & 3)];
  bool exact = false;  // flagged: the binary64 passes take the tile
  for (int p = 0; p < a.passes; ++p) {
    bool flag = false;
    const half8 zq = mfma_a(L.zero16);
    if ((p & 1) == 0) {
      // ---- row pass: pair pr takes row 16 (2w + t) + 4 g + i, t = pr / 4, i = pr % 4
      float4v a1[2][NB], a2[2][NB];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) a1[t][b] = a2[t][b] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KR; ++kk) {
        const int b = kk / 4;
        const half8 b1 = mfma_a(*(const uint4*)(cfl + (0 + (m & 1)) * SUBW + 32 * kk + 8 * g));
        const half8 b2 = mfma_a(*(const uint4*)(cfl + (2 + (m & 1)) * SUBW + 32 * kk + 8 * g));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          a1[t][b] = mfma16(ar[t][kk], b1, a1[t][b]);
          a2[t][b] = mfma16(ar2[t][kk], b2, a2[t][b]);
        }
      }
      const int t = pr >> 2, i = pr & 3;
      const int row = 16 * (2 * w + t) + 4 * g + i;
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float x1 = pick4(t ? a1[1][b] : a1[0][b], i), x2 = pick4(t ? a2[1][b] : a2[0][b], i);
        x1 += dpp<0xB1>(x1);  // hi + lo (quad_perm [1, 0, 3, 2])
        x2 += dpp<0xB1>(x2);
        const float d = drow[b];
        s1 = fmaf(d, x1, s1);
        s2 = fmaf(d * d, x2, s2);
      }
      // the sums carry kCScale and its square (exact powers of two)
      const float mean = s1 * (1.0f / (kCScale * SUBW));
      const float ms = s2 * (1.0f / (kCScale * kCScale * SUBW));
      const float var = ms - mean * mean;
      const bool upd = s2 > 0.0f;
      flag = upd && !(var > kIllCond * ms);
      const float rf = upd ? __builtin_amdgcn_rsqf(fmaxf(var, 0.0f)) : rf_keep;
      rf_keep = rf;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float f = drow[b] * rf * kRScale;
        flag = flag || f > kFMax || (f != 0.0f && f < kFMin);
        // both lanes of the pair hold the row's sums: both store (the same
        // halves to the same place), with no branch around the stores
        uint16_t* base = rfl + b * 4 * kGroup;
        put_hilo(base + 0 * kGroup, base + 1 * kGroup, row, f);
        put_hilo(base + 2 * kGroup, base + 3 * kGroup, row, f * f);
      }
    } else {
      // ---- column pass: pair pr takes columns 16 (CT w + ct) + 4 g + i of its
      // NCL slots (ct, i) = (k / 4, k % 4), k = NCL pr + e
      float4v c1[CT], c2[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) c1[ct] = c2[ct] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* base = rfl + wb * 4 * kGroup;
      // software-pipelined over the 4 CT steps (kr, ct): the column operand of
      // step j + 2 (and the factors of its kr) is loaded before the products of
      // step j (the scheduling barriers keep that order), so each product
      // waits for loads issued two steps earlier
      constexpr int NS = 4 * CT, LA = 2;
      half8 op[LA + 1], bf1[2], bf2[2];
      auto load_b = [&](int kr) {
        bf1[kr & 1] = mfma_a(*(const uint4*)(base + (0 + (m & 1)) * kGroup + 32 * kr + 8 * g));
        bf2[kr & 1] = mfma_a(*(const uint4*)(base + (2 + (m & 1)) * kGroup + 32 * kr + 8 * g));
      };
      auto load_op = [&](int j) { op[j % (LA + 1)] = load_col8<SUBW>(tile, 32 * (j / CT), 16 * (CT * w + j % CT), l); };
      load_b(0);
#pragma unroll
      for (int j = 0; j < LA; ++j) load_op(j);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int kr = j / CT, ct = j % CT;
        if (j + LA < NS) {
          if ((j + LA) % CT == 0) load_b((j + LA) / CT);
          load_op(j + LA);
        }
        __builtin_amdgcn_sched_barrier(0);
        const half8 a = op[j % (LA + 1)];
        c1[ct] = mfma16(a, bf1[kr & 1], c1[ct]);
        c2[ct] = mfma16(sq8(a, zq), bf2[kr & 1], c2[ct]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < NCL; ++e) {
        const int k = NCL * pr + e, ct = k >> 2, i = k & 3;
        const int col = 16 * (CT * w + ct) + 4 * g + i;
        float4v v1 = c1[0], v2 = c2[0];
#pragma unroll
        for (int c = 1; c < CT; ++c)
          if (ct == c) {
            v1 = c1[c];
            v2 = c2[c];
          }
        float x1 = pick4(v1, i), x2 = pick4(v2, i);
        x1 += dpp<0xB1>(x1);
        x2 += dpp<0xB1>(x2);
        // the sums carry kRScale and its square
        const float mean = x1 * (1.0f / (kRScale * kGroup));
        const float ms = x2 * (1.0f / (kRScale * kRScale * kGroup));
        const float var = ms - mean * mean;
        const bool upd = x2 > 0.0f;
        const float v0 = fmaxf(var, 0.0f);
        const float cf = upd ? __builtin_amdgcn_rsqf(v0) : cf_keep[e];
        const float lc = upd ? __builtin_amdgcn_logf(v0) * 0.34657359027997264f : lc_keep[e];  // ln sqrt: log2 / 2 ln 2
        cf_keep[e] = cf;
        lc_keep[e] = lc;
        const float c = cf * kCScale;
        flag = flag || (upd && !(var > kIllCond * ms)) || c > kFMax || c < kFMin;
        put_hilo(cfl + 0 * SUBW, cfl + 1 * SUBW, col, c);  // both lanes of the pair, as above
        put_hilo(cfl + 2 * SUBW, cfl + 3 * SUBW, col, c * c);
        lcs[col] = lc;
      }
    }
    if (flag) L.bad[p & 1] = 1;  // read after this pass's barrier, written again two passes on
    // the other side's factors are written; every wave has read the ones the
    // pass used (CF in row passes, RF in column passes)
    __syncthreads();
    if (L.bad[p & 1]) {
      exact = true;
      break;
    }
  }

  // ---- column scales: centre the log scales, clamp, fp16 (thread j: column j)
  const int bits = BITS ? BITS : kv ? y.vbits : y.kbits;
  const float levels = (float)((1 << bits) - 1);
  uint8_t* rec = a.arena + rec_off(y, s, layer, h, r) + (int64_t)sub * y.sub_bytes;
  uint8_t* meta = rec + y.kcode_bytes + y.vcode_bytes + kv * 2 * (SUBW + 2 * kGroup);
  if (exact) {
    balance_f64<SUBW>(L, ar, a.passes, meta);
    if constexpr (kv == 1) put_tile();  // its state took the tile's area; the value codes read the tile
  } else {
    float v = tid < SUBW ? lcs[tid] : 0.0f;
    v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    v = sum_x16x32(v);
    if (l == 0) red[w] = v;
    __syncthreads();
    const float lmean = (red[0] + red[1] + red[2] + red[3]) / (float)SUBW;
    if (tid < SUBW) {
      const float c = fminf(fmaxf(lcs[tid] - lmean, -9.0f), 9.0f);
      const uint16_t cb = f2h_bits(expf(c));
      ((uint16_t*)meta)[tid] = cb;
      invc[tid] = 1.0f / h2f(cb);
    }
    __syncthreads();
  }

  // ---- per-row rounding (row layout): y = x * fp32(1 / C), min and max per row
  const float nz = neg_zero();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 16 * (2 * w + t) + m;
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      const float d = ds[kk / 4][row];
      const float4 i0 = *(const float4*)(invc + 32 * kk + 8 * g), i1 = *(const float4*)(invc + 32 * kk + 8 * g + 4);
      const float ic[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yv = mul_e(d, ar[t][kk], e, nz) * ic[e];
        mn = fminf(mn, yv);
        mx = fmaxf(mx, yv);
      }
    }
    mn = min_x16x32(mn);
    mx = max_x16x32(mx);
    uint16_t Sb = f2h_sat_bits((mx - mn) / levels);
    if (h2f(Sb) == 0.0f) Sb = 0x3C00;  // 1.0
    const uint16_t Zb = f2h_sat_bits(mn);
    const float Zf = h2f(Zb);
    const float inv = 1.0f / h2f(Sb);
    if (g == 0) {
      ((uint16_t*)(meta + 2 * SUBW))[row] = Sb;
      ((uint16_t*)(meta + 2 * SUBW + 2 * kGroup))[row] = Zb;
      rinv[row] = inv;
      zrow[row] = Zf;
    }
    if constexpr (kv == 0) {  // keys: row-major codes, this lane's 8 columns of each k-step
#pragma unroll
      for (int kk = 0; kk < KR; ++kk) {
        const float d = ds[kk / 4][row];
        const float4 i0 = *(const float4*)(invc + 32 * kk + 8 * g), i1 = *(const float4*)(invc + 32 * kk + 8 * g + 4);
        const float ic[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        float cf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float yv = mul_e(d, ar[t][kk], e, nz) * ic[e];
          cf[e] = __builtin_amdgcn_fmed3f(rintf((yv - Zf) * inv), 0.0f, levels);
        }
        store_codes8<BITS>(rec + (int64_t)row * (SUBW * bits / 8) + (32 * kk + 8 * g) * bits / 8, cf, bits);
      }
    }
  }
  if constexpr (kv == 1) {  // values: channel-major codes (column layout), 8 tokens of one channel per dword
    __syncthreads();
    uint8_t* vbase = rec + y.kcode_bytes;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int col = 16 * (CT * w + ct) + m;
      const float ic = invc[col];
#pragma unroll
      for (int kr = 0; kr < 4; ++kr) {
        const half8 ac = load_col8<SUBW>(tile, 32 * kr, 16 * (CT * w + ct), l);
        float cf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = 32 * kr + 8 * g + e;
          const float yv = mul_e_pure(ds[wb][row], ac, e, nz) * ic;
          cf[e] = __builtin_amdgcn_fmed3f(rintf((yv - zrow[row]) * rinv[row]), 0.0f, levels);
        }
        store_codes8<BITS>(vbase + (int64_t)col * (kGroup * bits / 8) + (32 * kr + 8 * g) * bits / 8, cf, bits);
      }
    }
  }
}

template <int SUBW, int KB, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void seal_kernel(SealArgs a) {
  __shared__ SealLds<SUBW> L;
  const int gx = blockIdx.x;
  int ti = 0;
  while (ti + 1 < a.n_tasks && gx >= a.task[ti + 1].first) ++ti;
  const SealTask tk = a.task[ti];
  const int r = tk.rec0 + (gx - tk.first);
  int by = blockIdx.y;
  const int sub = by % a.y.nsub;
  by /= a.y.nsub;
  const int kv = by & 1, h = by >> 1;
  if (kv == 0)
    seal_tile<SUBW, 0, KB>(a, L, r, sub, h, tk.slot, tk.layer);
  else
    seal_tile<SUBW, 1, VB>(a, L, r, sub, h, tk.slot, tk.layer);
}

// ---------------------------------------------------------------------------
// Seal of f16-staged tiles (SJ-KVaRN 4.1: the 16-bit alternative to tq6_0
// staging; KV Cache Precision Tail, section 2: KVarN's exact F16 tail).  The
// ring holds the tokens in the original domain, so the seal first rotates the
// group's rows (SJ-KVaRN 2.2; 128-wide heads: the randomized Walsh-Hadamard
// transform of KV cache math): each row's signed sum of fp16 values is exact
// in binary64 across the wave (the staging encoder's arithmetic) and is
// rounded once to fp32, into an fp32 tile in LDS.  That tile has no integer
// structure for the matrix cores, and this staging serves small caches, so it
// is balanced by the binary64 passes (balance_f64's definition, read from the
// fp32 tile) and rounded in IEEE fp32 exactly as the 6-bit path rounds.
template <int SUBW>
struct SealF16Lds {
  float x[kGroup][SUBW];  // the rotated tile
  double lr[kGroup], lc[SUBW], fr[kGroup], fc[SUBW];
  double red64[4];
  float invc[SUBW], rinv[kGroup], zrow[kGroup];
};

template <int SUBW>
__global__ __launch_bounds__(256) void seal_f16_kernel(SealArgs a) {
  __shared__ SealF16Lds<SUBW> L;
  constexpr int VPL = SUBW / 64;
  const Layout& y = a.y;
  const int gx = blockIdx.x;
  int ti = 0;
  while (ti + 1 < a.n_tasks && gx >= a.task[ti + 1].first) ++ti;
  const SealTask tk = a.task[ti];
  const int r = tk.rec0 + (gx - tk.first);
  int by = blockIdx.y;
  const int sub = by % y.nsub;
  by /= y.nsub;
  const int kv = by & 1, h = by >> 1, s = tk.slot, layer = tk.layer;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int slot0 = (int)(((int64_t)r * kGroup) % y.cap);
  const uint16_t* ring = (const uint16_t*)(a.arena + rcode_off(y, s, layer, h, kv, 0));

  // ---- rotate: wave w takes rows w, w + 4, ...; lane l holds elements VPL l ..
  for (int row = w; row < kGroup; row += 4) {
    int slot = slot0 + row;
    if (slot >= y.cap) slot -= y.cap;
    const uint16_t* src = ring + (int64_t)slot * y.D + sub * SUBW;
    double v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int i = VPL * l + j;
      const double e = (double)h2f(src[i]);
      v[j] = SUBW == 128 && sign_neg(a.signs, i) ? -e : e;
    }
#pragma unroll
    for (int st = 1; st < VPL; st <<= 1)
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (!(j & st)) {
          const double p = v[j], q = v[j + st];
          v[j] = p + q;
          v[j + st] = p - q;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const double o = shfl_xor_d(v[j], m);
        v[j] = (l & m) ? (o - v[j]) : (v[j] + o);
      }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      double e;
      if (SUBW == 128) {
        e = v[j] * kInvSqrt128;
        if (sign_neg(a.signs, 128 + VPL * l + j)) e = -e;
      } else {
        e = v[j] * 0.0625;
      }
      L.x[row][VPL * l + j] = (float)e;
    }
  }
  for (int i = tid; i < kGroup; i += 256) L.lr[i] = 0.0;
  for (int j = tid; j < SUBW; j += 256) L.lc[j] = 0.0;
  __syncthreads();

  // ---- binary64 balancing
  const int hf = tid & 1;
  for (int p = 0; p < a.passes; ++p) {
    for (int i = tid; i < kGroup; i += 256) L.fr[i] = exp(-L.lr[i]);
    for (int j = tid; j < SUBW; j += 256) L.fc[j] = exp(-L.lc[j]);
    __syncthreads();
    if ((p & 1) == 0) {  // row tid / 2, columns hf SUBW / 2 .. + SUBW / 2
      const int row = tid >> 1, c0 = hf * (SUBW / 2);
      const double frow = L.fr[row];
      const double ref = (double)L.x[row][0] * frow * L.fc[0];
      double s1 = 0.0, s2 = 0.0, sq = 0.0;
      for (int c = c0; c < c0 + SUBW / 2; ++c) {
        const double yy = (double)L.x[row][c] * frow * L.fc[c], dv = yy - ref;
        s1 += dv;
        s2 += dv * dv;
        sq += yy * yy;
      }
      s1 += __shfl_xor(s1, 1, 64);
      s2 += __shfl_xor(s2, 1, 64);
      sq += __shfl_xor(sq, 1, 64);
      const double mean = s1 / SUBW, sig = sqrt(fmax(s2 / SUBW - mean * mean, 0.0));
      if (hf == 0 && sig > kZeroSpread64 * sqrt(sq / SUBW)) L.lr[row] += log(sig);
    } else {  // column tid (256 wide), or tid / 2 with rows hf 64 .. + 64 (128 wide)
      constexpr int TPC = 256 / SUBW, NR = kGroup / TPC;
      const int col = tid / TPC, r0 = TPC == 2 ? hf * NR : 0;
      const double fcol = L.fc[col];
      const double ref = (double)L.x[0][col] * L.fr[0] * fcol;
      double s1 = 0.0, s2 = 0.0, sq = 0.0;
      for (int rr = r0; rr < r0 + NR; ++rr) {
        const double yy = (double)L.x[rr][col] * L.fr[rr] * fcol, dv = yy - ref;
        s1 += dv;
        s2 += dv * dv;
        sq += yy * yy;
      }
      if (TPC == 2) {
        s1 += __shfl_xor(s1, 1, 64);
        s2 += __shfl_xor(s2, 1, 64);
        sq += __shfl_xor(sq, 1, 64);
      }
      const double mean = s1 / kGroup, sig = sqrt(fmax(s2 / kGroup - mean * mean, 0.0));
      if ((TPC == 1 || hf == 0) && sig > kZeroSpread64 * sqrt(sq / kGroup)) L.lc[col] += log(sig);
    }
    __syncthreads();
  }

  // ---- column scales
  const int bits = kv ? y.vbits : y.kbits;
  const float levels = (float)((1 << bits) - 1);
  uint8_t* rec = a.arena + rec_off(y, s, layer, h, r) + (int64_t)sub * y.sub_bytes;
  uint8_t* meta = rec + y.kcode_bytes + y.vcode_bytes + kv * 2 * (SUBW + 2 * kGroup);
  {
    double v = tid < SUBW ? L.lc[tid] : 0.0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    if (l == 0) L.red64[w] = v;
    __syncthreads();
    const double lmean = (L.red64[0] + L.red64[1] + L.red64[2] + L.red64[3]) / SUBW;
    if (tid < SUBW) {
      const double c = fmin(fmax(L.lc[tid] - lmean, -9.0), 9.0);
      const half_t ch = (half_t)exp(c);
      uint16_t cb;
      __builtin_memcpy(&cb, &ch, 2);
      ((uint16_t*)meta)[tid] = cb;
      L.invc[tid] = 1.0f / h2f(cb);
    }
    __syncthreads();
  }

  // ---- per-row rounding: row tid / 2, columns hf SUBW / 2 .. + SUBW / 2
  {
    const int row = tid >> 1, c0 = hf * (SUBW / 2);
    float mn = INFINITY, mx = -INFINITY;
    for (int c = c0; c < c0 + SUBW / 2; ++c) {
      const float yv = L.x[row][c] * L.invc[c];
      mn = fminf(mn, yv);
      mx = fmaxf(mx, yv);
    }
    mn = fminf(mn, __shfl_xor(mn, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    uint16_t Sb = f2h_sat_bits((mx - mn) / levels);
    if (h2f(Sb) == 0.0f) Sb = 0x3C00;  // 1.0
    const uint16_t Zb = f2h_sat_bits(mn);
    const float Zf = h2f(Zb), inv = 1.0f / h2f(Sb);
    if (hf == 0) {
      ((uint16_t*)(meta + 2 * SUBW))[row] = Sb;
      ((uint16_t*)(meta + 2 * SUBW + 2 * kGroup))[row] = Zb;
      L.rinv[row] = inv;
      L.zrow[row] = Zf;
    }
    if (kv == 0) {  // keys: row-major, two 4-bit codes per byte (even channel low) or one 8-bit code
      for (int c = c0; c < c0 + SUBW / 2; c += 8) {
        uint32_t cq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float yv = L.x[row][c + e] * L.invc[c + e];
          cq[e] = (uint32_t)__builtin_amdgcn_fmed3f(rintf((yv - Zf) * inv), 0.0f, levels);
        }
        put_codes8(rec + (int64_t)row * (SUBW * bits / 8) + c * bits / 8, cq, bits);
      }
    }
  }
  if (kv == 1) {  // values: channel-major, an LSB-first stream of codes per channel
    __syncthreads();
    uint8_t* vbase = rec + y.kcode_bytes;
    for (int col = tid; col < SUBW; col += 256) {
      const float ic = L.invc[col];
      for (int t0 = 0; t0 < kGroup; t0 += 8) {
        uint32_t cq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = t0 + e;
          const float yv = L.x[row][col] * ic;
          cq[e] = (uint32_t)__builtin_amdgcn_fmed3f(rintf((yv - L.zrow[row]) * L.rinv[row]), 0.0f, levels);
        }
        put_codes8(vbase + (int64_t)col * (kGroup * bits / 8) + t0 * bits / 8, cq, bits);
      }
    }
  }
}

hipError_t launch_seal(const SealArgs& a, hipStream_t stream) {
  dim3 grid(a.total_groups, 2 * a.y.H * a.y.nsub);
  if (a.y.f16ring) {
    if (a.y.sub == 256)
      hipLaunchKernelGGL(seal_f16_kernel<256>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(seal_f16_kernel<128>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  // the 4/4 and 8/4 bodies with constant widths, the lower ones read them
  const bool k4 = a.y.kbits == 4 && a.y.vbits == 4, k8 = a.y.kbits == 8 && a.y.vbits == 4;
  auto kern = a.y.sub == 256 ? (k4 ? seal_kernel<256, 4, 4> : k8 ? seal_kernel<256, 8, 4> : seal_kernel<256, 0, 0>)
                             : (k4 ? seal_kernel<128, 4, 4> : k8 ? seal_kernel<128, 8, 4> : seal_kernel<128, 0, 0>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
