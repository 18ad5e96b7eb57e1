// Matrix-core decode attention over the two exact regions: the fp16 sink and
// the tq6_0 staging ring, plus the per-call query preparation shared with the
// body scan.
//
// SJ-KVaRN 2.1: the sink (first 128 tokens, original domain) and the staging
// ring (the newest tokens, kept in the rotated domain as 6-bit codes with one
// fp16 scale per 128-value block, KV Cache Precision Tail section 3) are read
// in the same decode pass as the sealed body; each workgroup writes one
// split-K partial (m, l, acc[D]) that the merge combines under one softmax.
// KV cache math ("rotate first"): ring scores use the rotated query; the sink
// uses the unrotated one, so its partial needs no inverse rotation.
//
// One workgroup (4 waves) per 128-token chunk of one KV head: chunk 0 is the
// sink, chunks 1.. the ring.  With u the centred code (q in tq6_0 terms) and d
// the block scale, a ring key is d u and
//     score_t = scale * sum_blocks d_t,b (q' . u_t,b)
//     out_j   = sum_t (p_t d^V_t,b(j)) u^V_t,j
// so the codes enter the matrix cores as exact small integers (fp16) and the
// scales are applied outside the products.  The query and the weights p d are
// split into hi + lo fp16 halves (two products each), which keeps fp32-level
// precision in both contractions.
//
// Steps: (1) stage the chunk in LDS (ring: raw codes and scales; sink: the
// value rows transposed); (2) each wave scores two 16-token tiles against the
// G query heads (G <= 16, padded to the 16 columns of the product);
// (3) workgroup max and the weights p, written to LDS as the second operand;
// (4) each wave forms D/64 channel tiles of p V over all 128 tokens.
#include "kvq_mfma.h"

namespace kvq {

constexpr int kStagedTokens = 128;

// ---------------------------------------------------------------------------
// Query preparation: grid (H, n_seqs), 256 threads.  Rotates the G query heads
// of one KV head (R = H/16 for head_dim 256, s2 . H . s1 / sqrt(128) for 128),
// multiplies them by scale * log2(e) so that every product below yields scores
// in log2 units, and writes the operand sets described in kvq_mfma.h.
template <int D>
__global__ __launch_bounds__(256) void decode_qprep_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;
  __shared__ float qraw[kMaxGroup][D];
  __shared__ float qrot[kMaxGroup][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4, G = a.g;
  const float sl = a.scale * kLog2e;  // scores come out in log2 units
  for (int idx = tid; idx < kMaxGroup * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    const float v = i < G ? h2f(a.q[((int64_t)b * a.Hq + h * G + i) * D + j]) * sl : 0.0f;
    qraw[i][j] = v;
    qrot[i][j] = (D == 128 && sign_neg(a.signs, j)) ? -v : v;
  }
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    for (int p = tid; p < kMaxGroup * D / 2; p += 256) {
      const int i = p / (D / 2), pp = p % (D / 2);
      const int j = (pp / st) * 2 * st + (pp % st);
      const float u = qrot[i][j], v = qrot[i][j + st];
      qrot[i][j] = u + v;
      qrot[i][j + st] = u - v;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < kMaxGroup * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    float x = qrot[i][j];
    if (D == 128) {
      x = x * (float)kInvSqrt128;
      if (sign_neg(a.signs, 128 + j)) x = -x;
    } else {
      x = x * 0.0625f;
    }
    qrot[i][j] = x;
  }
  __syncthreads();
  uint4* out = a.qops + ((int64_t)b * a.y.H + h) * kQopsPerHead;
  for (int kk = wave; kk < KK; kk += 4) {
    // natural order: k-step kk, lane group g holds channels 32 kk + 8 g .. + 7;
    // body order: 128 (kk / 4) + 32 g + 8 (kk % 4) .. + 7, the channels of
    // the code dword that lane group reads from a key row
    const int base = 32 * kk + 8 * g;
    const int base0 = 128 * (kk >> 2) + 32 * g + 8 * (kk & 3);
    const float* qr = qrot[q16];
    const float* qw = qraw[q16];
    uint32_t hb[4], lb[4], hr[4], lr[4], hs[4], ls[4];
    for (int pr = 0; pr < 4; ++pr) {
      // body nibble order: slot pairs hold channels (pr, pr + 4); the pairs
      // read from high nibbles (odd pr) carry a factor 1/16
      const float f = (pr & 1) ? 0.0625f : 1.0f;
      split_h2(qr[base0 + pr] * f, qr[base0 + pr + 4] * f, hb[pr], lb[pr]);
      split_h2(qr[base + 2 * pr], qr[base + 2 * pr + 1], hr[pr], lr[pr]);
      split_h2(qw[base + 2 * pr], qw[base + 2 * pr + 1], hs[pr], ls[pr]);
    }
    if (D == 256) {
      out[kk * 64 + lane] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
      out[(8 + kk) * 64 + lane] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
    }
    out[kQopsSet + kk * 64 + lane] = make_uint4(hr[0], hr[1], hr[2], hr[3]);
    out[kQopsSet + (8 + kk) * 64 + lane] = make_uint4(lr[0], lr[1], lr[2], lr[3]);
    out[2 * kQopsSet + kk * 64 + lane] = make_uint4(hs[0], hs[1], hs[2], hs[3]);
    out[2 * kQopsSet + (8 + kk) * 64 + lane] = make_uint4(ls[0], ls[1], ls[2], ls[3]);
  }
}

// ---------------------------------------------------------------------------
// Eight 6-bit codes (48 bits, LSB first) starting at an even byte offset of an
// LDS buffer, as fp16 values u - 32 in [-32, 31] (exact).  Two aligned dword
// reads and a funnel shift; 1024 + u is formed by OR-ing the code into the
// mantissa of 1024, then one packed subtract.
__device__ __forceinline__ half8 codes6(const uint8_t* base, int off) {
  const uint32_t* w = (const uint32_t*)(base + (off & ~3));
  const uint32_t w0 = w[0], w1 = w[1];
  const uint32_t sh = (uint32_t)(off & 2) * 8u;
  const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, sh);
  const uint32_t hi = w1 >> sh;
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

template <int D>
__global__ __launch_bounds__(256) void decode_staged_kernel(DecodeArgs a) {
  constexpr int NB = D / kQBlock;       // tq6_0 blocks per vector
  constexpr int KK = D / 32;            // k-steps of the score product
  constexpr int RT = kStagedTokens;
  constexpr int ROWB = NB * kQBytes;    // code bytes per ring vector
  constexpr int PITCH = RT + 8;         // halves per row of V^T and of the weights
  constexpr int CPW = D / 64;           // channel tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t kraw[RT * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t vraw[RT * ROWB];  // then the weights [NB][hi, lo][16][PITCH]
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * PITCH];
  __shared__ float dks[RT][NB], dvs[RT][NB];
  __shared__ float xm[4][16], xl[4][16];
  static_assert(NB * 2 * 16 * PITCH * 2 <= RT * ROWB, "weights do not fit the raw value area");

  const Layout& y = a.y;
  const DecodeSeq sq = a.seq[blockIdx.z];
  const int c = blockIdx.x;
  if (c > sq.n_ring_chunks) return;
  const bool sink = c == 0;
  const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4, G = a.g;
  const int s = sq.slot, layer = a.layer;
  const int t_begin = sink ? 0 : (c - 1) * RT;
  const int n = sink ? sq.n_sink : min(RT, sq.ring_len - t_begin);
  const uint16_t* ksink = (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, s, layer, h, 0, 0);

  // ---- (1) stage
  if (sink) {
    const uint16_t* vsrc = (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, s, layer, h, 1, 0);
    for (int it = tid; it < (RT / 4) * (D / 8); it += 256) {
      const int tq = it % (RT / 4), c8 = it / (RT / 4);
      uint4 r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tok = 4 * tq + k;
        r[k] = tok < n ? *(const uint4*)(vsrc + (int64_t)tok * D + 8 * c8) : make_uint4(0, 0, 0, 0);
      }
      store_t4x8(vt, PITCH, 8 * c8, 4 * tq, r);
    }
  } else {
    for (int u = tid; u < RT * ROWB / 16; u += 256) {
      const int tok = u / (ROWB / 16), part = u % (ROWB / 16);
      uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
      if (tok < n) {
        const int slot = (sq.ring0 + t_begin + tok) % y.cap;
        kx = *(const uint4*)(a.arena + rcode_off(y, s, layer, h, 0, slot) + 16 * part);
        vx = *(const uint4*)(a.arena + rcode_off(y, s, layer, h, 1, slot) + 16 * part);
      }
      *(uint4*)(kraw + 16 * u) = kx;
      *(uint4*)(vraw + 16 * u) = vx;
    }
    for (int i = tid; i < RT * NB; i += 256) {
      const int tok = i / NB, blk = i % NB;
      float dk = 0.0f, dv = 0.0f;
      if (tok < n) {
        const int slot = (sq.ring0 + t_begin + tok) % y.cap;
        dk = h2f(((const uint16_t*)(a.arena + rscale_off(y, s, layer, h, 0, slot)))[blk]);
        dv = h2f(((const uint16_t*)(a.arena + rscale_off(y, s, layer, h, 1, slot)))[blk]);
      }
      dks[tok][blk] = dk;
      dvs[tok][blk] = dv;
    }
    __syncthreads();
    for (int it = tid; it < (RT / 4) * (D / 8); it += 256) {
      const int tq = it % (RT / 4), c8 = it / (RT / 4);
      uint4 r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const half8 v = codes6(vraw, (4 * tq + k) * ROWB + 6 * c8);
        __builtin_memcpy(&r[k], &v, 16);
      }
      store_t4x8(vt, PITCH, 8 * c8, 4 * tq, r);
    }
  }

  // ---- (2) scores of two 16-token tiles per wave, log2 units
  uint4 qh[KK], ql[KK];
  {
    const uint4* qo = a.qops + ((int64_t)blockIdx.z * y.H + h) * kQopsPerHead + (sink ? 2 : 1) * kQopsSet;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qh[kk] = qo[kk * 64 + lane];
      ql[kk] = qo[(8 + kk) * 64 + lane];
    }
  }
  float sc[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int bb = 2 * wave + i;
    const int arow = 16 * bb + q16;  // token of this lane's A row
    float4v acc[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) acc[blk] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      half8 av;
      if (sink)
        av = mfma_a(*(const uint4*)(ksink + (int64_t)arow * D + 32 * kk + 8 * g));
      else
        av = codes6(kraw, arow * ROWB + 24 * kk + 6 * g);
      const int blk = kk / 4;
      acc[blk] = mfma16(av, mfma_a(qh[kk]), acc[blk]);
      acc[blk] = mfma16(av, mfma_a(ql[kk]), acc[blk]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * bb + 4 * g + r;
      float v = 0.0f;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) v = sink ? v + acc[blk][r] : fmaf(dks[t][blk], acc[blk][r], v);
      v = t < n ? v : -INFINITY;
      sc[i][r] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = xmax4(mx);
  if (g == 0) xm[wave][q16] = mx;
  __syncthreads();

  // ---- (3) weights: p = 2^(s - M); operand p d^V (ring) or p (sink) as hi + lo
  const float M = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16]));  // token 0 is valid
  uint16_t* pw = (uint16_t*)vraw;
  float lp = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int bb = 2 * wave + i;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(sc[i][r] - M);  // -inf for masked tokens gives 0
      lp += p[r];
    }
#pragma unroll
    for (int blk = 0; blk < (sink ? 1 : NB); ++blk) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = sink ? p[r] : p[r] * dvs[16 * bb + 4 * g + r][blk];
      uint2 hi, lo;
      split_h2(x[0], x[1], hi.x, lo.x);
      split_h2(x[2], x[3], hi.y, lo.y);
      *(uint2*)(pw + ((blk * 2 + 0) * 16 + q16) * PITCH + 16 * bb + 4 * g) = hi;
      *(uint2*)(pw + ((blk * 2 + 1) * 16 + q16) * PITCH + 16 * bb + 4 * g) = lo;
    }
  }
  lp = xsum4(lp);
  if (g == 0) xl[wave][q16] = lp;
  __syncthreads();

  // ---- (4) O^T = V^T P'^T for this wave's channel tiles, written as the partial
  float* P = a.part + (((int64_t)blockIdx.z * a.Hq + h * G + q16) * a.max_chunks + c) * (D + 2);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int cb = wave * CPW + i;
    const int blk = sink ? 0 : (16 * cb) / kQBlock;
    float4v o = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < RT / 32; ++j) {
      const half8 av = mfma_a(*(const uint4*)(vt + (16 * cb + q16) * PITCH + 32 * j + 8 * g));
      const half8 bh = mfma_a(*(const uint4*)(pw + ((blk * 2 + 0) * 16 + q16) * PITCH + 32 * j + 8 * g));
      const half8 bl = mfma_a(*(const uint4*)(pw + ((blk * 2 + 1) * 16 + q16) * PITCH + 32 * j + 8 * g));
      o = mfma16(av, bh, o);
      o = mfma16(av, bl, o);
    }
    if (q16 < G) {
      const int ch = 16 * cb + 4 * g;
      P[2 + ch + 0] = o[0];
      P[2 + ch + 1] = o[1];
      P[2 + ch + 2] = o[2];
      P[2 + ch + 3] = o[3];
    }
  }
  if (wave == 0 && g == 0 && q16 < G) {
    P[0] = M * kLn2;
    P[1] = xl[0][q16] + xl[1][q16] + xl[2][q16] + xl[3][q16];
  }
}

hipError_t launch_decode_qprep(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.y.H, a.n_seqs);
  switch (a.y.D) {
    case 128: hipLaunchKernelGGL(decode_qprep_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_qprep_kernel<256>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// grid_x = 1 + the largest ring chunk count of the launch's sequences
hipError_t launch_decode_staged(const DecodeArgs& a, int grid_x, hipStream_t stream) {
  if (a.ring_chunk != kStagedTokens || a.g > 16) return hipErrorInvalidValue;
  dim3 grid(grid_x, a.y.H, a.n_seqs);
  switch (a.y.D) {
    case 128: hipLaunchKernelGGL(decode_staged_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_staged_kernel<256>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
