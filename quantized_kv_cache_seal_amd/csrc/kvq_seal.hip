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
// Tile mapping: thread (wave w, lane l = 16 r4 + c16) holds rows 32w + 8r4 + i
// (i < 8) and columns CPT*c16 + j (j < CPT), CPT = SUB/16, in registers for the
// whole seal.  A row reduction is in-thread plus a 16-lane DPP exchange; a
// column reduction is in-thread, a swap exchange across r4, then LDS across
// the four waves.  Each pass computes the spread of x scaled by the other side's
// current factors; the updated side's factor becomes 1/spread (equal to
// exp(-l) of the log-domain update l += ln spread).
//
// The balancing factors (1/spread, ln spread) use the hardware square root,
// reciprocal and log2 (about 1 ulp): only the column scales C leave the
// balancing, and they are rounded to fp16.  Rounding is IEEE fp32 with no
// fused multiply-add (built with -ffp-contract=off): y = x * fp32(1/C), S = fp16((max - min) / (2^b - 1))
// (1.0 if zero), Z = fp16(min), code = clamp(rne((y - Z) * fp32(1/S)), 0, 2^b - 1).
#include "kvq_device.h"

namespace kvq {

// Reductions over the 16 lanes of a row (DPP: quad swaps, then the half-row
// and row mirrors; every lane ends with the result) and over the four rows of
// a wave for the same lane (the 32- and 16-lane swaps of this target: each
// returns the lane's own value and its partner's, in some order).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float min16(float x) {
  x = fminf(x, dpp<0xB1>(x));
  x = fminf(x, dpp<0x4E>(x));
  x = fminf(x, dpp<0x141>(x));
  return fminf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  return fmaxf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

__device__ __forceinline__ uint32_t bits6(const uint32_t* wd, int j) {
  const int p = 6 * j;
  const uint64_t pair = ((uint64_t)wd[(p >> 5) + 1] << 32) | wd[p >> 5];
  return (uint32_t)(pair >> (p & 31)) & 63u;
}

template <int CPT>
__global__ __launch_bounds__(256) void seal_kernel(SealArgs a) {
  constexpr int COLS = 16 * CPT;
  const Layout& y = a.y;
  __shared__ float red[4][COLS][2];

  const int gx = blockIdx.x;
  int ti = 0;
  while (ti + 1 < a.n_tasks && gx >= a.task[ti + 1].first) ++ti;
  const SealTask tk = a.task[ti];
  const int r = tk.rec0 + (gx - tk.first);
  int by = blockIdx.y;
  const int sub = by % y.nsub;
  by /= y.nsub;
  const int kv = by & 1, h = by >> 1;
  const int s = tk.slot, layer = tk.layer;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r4 = l >> 4, c16 = l & 15;
  const int row0 = 32 * w + 8 * r4, col0 = CPT * c16;
  const int slot0 = (int)(((int64_t)r * kGroup) % y.cap);
  const int gch = sub * COLS + col0;
  const int blk = gch / kQBlock, k0 = gch % kQBlock;

  // ---- load the tile: x = d * (u - 32), exact in fp32
  float X[8][CPT];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = slot0 + row0 + i;
    const uint8_t* cp = a.arena + rcode_off(y, s, layer, h, kv, slot) + blk * kQBytes + (k0 * 6) / 8;
    const float d = h2f(*(const uint16_t*)(a.arena + rscale_off(y, s, layer, h, kv, slot) + 2 * blk));
    uint32_t wd[4];
    if constexpr (CPT == 16) {
      const uint32_t* p32 = (const uint32_t*)cp;
      wd[0] = p32[0];
      wd[1] = p32[1];
      wd[2] = p32[2];
      wd[3] = 0;
    } else {
      const uint16_t* p16 = (const uint16_t*)cp;
      wd[0] = (uint32_t)p16[0] | ((uint32_t)p16[1] << 16);
      wd[1] = p16[2];
      wd[2] = 0;
      wd[3] = 0;
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) X[i][j] = d * (float)((int)bits6(wd, j) - 32);
  }

  // ---- Sinkhorn passes
  float cf[CPT], rf[8], lc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    cf[j] = 1.0f;
    lc[j] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) rf[i] = 1.0f;

  for (int p = 0; p < a.passes; ++p) {
    if ((p & 1) == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sm = 0.0f, sq = 0.0f;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const float t = X[i][j] * cf[j];
          sm += t;
          sq = fmaf(t, t, sq);
        }
        sm = sum16(sm);
        sq = sum16(sq);
        const float mean = sm / (float)COLS;
        const float var = fmaxf(sq / (float)COLS - mean * mean, 0.0f);
        rf[i] = __builtin_amdgcn_rcpf(fmaxf(__builtin_amdgcn_sqrtf(var), 1e-30f));
      }
    } else {
      float sm[CPT], sq[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        sm[j] = 0.0f;
        sq[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t = X[i][j] * rf[i];
          sm[j] += t;
          sq[j] = fmaf(t, t, sq[j]);
        }
        sm[j] = sum_rows4(sm[j]);
        sq[j] = sum_rows4(sq[j]);
      }
      if (r4 == 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          red[w][col0 + j][0] = sm[j];
          red[w][col0 + j][1] = sq[j];
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const float ts = red[0][col0 + j][0] + red[1][col0 + j][0] + red[2][col0 + j][0] + red[3][col0 + j][0];
        const float tq = red[0][col0 + j][1] + red[1][col0 + j][1] + red[2][col0 + j][1] + red[3][col0 + j][1];
        const float mean = ts / (float)kGroup;
        const float var = fmaxf(tq / (float)kGroup - mean * mean, 0.0f);
        const float sig = fmaxf(__builtin_amdgcn_sqrtf(var), 1e-30f);
        cf[j] = __builtin_amdgcn_rcpf(sig);
        lc[j] = __builtin_amdgcn_logf(sig) * 0.6931471805599453f;  // log2 -> ln
      }
      __syncthreads();
    }
  }

  // ---- column scales: centre the log scales, clamp, fp16
  float ls = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) ls += lc[j];
  ls = sum16(ls);
  const float lmean = ls / (float)COLS;
  uint16_t Cb[CPT];
  float invC[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const float v = fminf(fmaxf(lc[j] - lmean, -9.0f), 9.0f);
    Cb[j] = f2h_bits(expf(v));
    invC[j] = 1.0f / h2f(Cb[j]);
  }

  // ---- per-row rounding and packing
  const int bits = kv ? y.vbits : y.kbits;
  const float levels = (float)((1 << bits) - 1);
  uint8_t* rec = a.arena + rec_off(y, s, layer, h, r) + (int64_t)sub * y.sub_bytes;
  uint8_t* meta = rec + y.kcode_bytes + y.vcode_bytes + kv * 2 * (COLS + 2 * kGroup);
  uint32_t vw[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) vw[j] = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float yv[CPT];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      yv[j] = X[i][j] * invC[j];
      mn = fminf(mn, yv[j]);
      mx = fmaxf(mx, yv[j]);
    }
    mn = min16(mn);
    mx = max16(mx);
    uint16_t Sb = f2h_sat_bits((mx - mn) / levels);
    if (h2f(Sb) == 0.0f) Sb = 0x3C00;  // 1.0
    const uint16_t Zb = f2h_sat_bits(mn);
    const float Zf = h2f(Zb);
    const float inv = 1.0f / h2f(Sb);
    uint32_t cq[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) cq[j] = (uint32_t)fminf(fmaxf(rintf((yv[j] - Zf) * inv), 0.0f), levels);
    const int row = row0 + i;
    if (kv == 0) {
      if (bits == 4) {
        uint32_t pk[CPT / 8];
#pragma unroll
        for (int q = 0; q < CPT / 8; ++q) {
          pk[q] = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) pk[q] |= cq[8 * q + e] << (4 * e);
        }
        uint32_t* dst = (uint32_t*)(rec + (int64_t)row * (COLS / 2) + col0 / 2);
#pragma unroll
        for (int q = 0; q < CPT / 8; ++q) dst[q] = pk[q];
      } else {
        uint32_t pk[CPT / 4];
#pragma unroll
        for (int q = 0; q < CPT / 4; ++q) {
          pk[q] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[q] |= cq[4 * q + e] << (8 * e);
        }
        uint32_t* dst = (uint32_t*)(rec + (int64_t)row * COLS + col0);
#pragma unroll
        for (int q = 0; q < CPT / 4; ++q) dst[q] = pk[q];
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) vw[j] |= cq[j] << (4 * i);
    }
    if (c16 == 0) {
      ((uint16_t*)(meta + 2 * COLS))[row] = Sb;
      ((uint16_t*)(meta + 2 * COLS + 2 * kGroup))[row] = Zb;
    }
  }
  if (kv == 1) {
    uint8_t* vbase = rec + y.kcode_bytes;
#pragma unroll
    for (int j = 0; j < CPT; ++j) *(uint32_t*)(vbase + (int64_t)(col0 + j) * (kGroup / 2) + row0 / 2) = vw[j];
  }
  if (w == 0 && r4 == 0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) ((uint16_t*)meta)[col0 + j] = Cb[j];
  }
}

hipError_t launch_seal(const SealArgs& a, hipStream_t stream) {
  dim3 grid(a.total_groups, 2 * a.y.H * a.y.nsub);
  if (a.y.sub == 256)
    hipLaunchKernelGGL(seal_kernel<16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(seal_kernel<8>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
