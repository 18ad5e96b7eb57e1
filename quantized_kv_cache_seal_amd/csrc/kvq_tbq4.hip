// Comparator formats.  TBQ4 (KV cache math: "rotate first" and the format table):
// each 128-value block is rotated by the randomized Walsh-Hadamard transform
// (sign flip, transform, sign flip), its norm is stored in fp16, and each
// rotated value divided by the norm is replaced by the 4-bit index of the
// nearest of 16 centroids fitted to N(0, 1/128).  Block = [fp16 norm]
// [64 bytes of indices, even value in the low nibble], 66 bytes.
//
// Encode arithmetic: the rotation is exact in binary64 and rounded once to
// fp32; the squared norm is summed in binary64 and its square root rounded
// once to fp16 (nearest even); v = y * fp32(1 / norm) in fp32; the index is
// the number of fp32 cell boundaries strictly below v (ties go low).
//
// Fused decode (the rotated-domain principle of the same page): the query is
// rotated once (a prologue kernel into the workspace), every key and value is
// read as centroid x norm in the rotated domain, and each split-K partial is
// rotated back once before the merge.
#include "kvq_device.h"

namespace kvq {

namespace {

constexpr float kLn2f = 0.6931471805599453f;

// fp16 bits of x >= 0 (finite or not), rounded to nearest even straight from
// binary64: scale by the fp16 spacing at x, round to an integer, scale back.
__device__ __forceinline__ uint16_t d2h_bits_nonneg(double x) {
  if (!(x > 0.0)) return 0;
  if (!(x < 65520.0)) return 0x7C00;  // at or past the overflow threshold
  const int e = ilogb(x);                         // x in [2^e, 2^(e+1))
  const int ue = (e < -14 ? -14 : e) - 10;        // fp16 spacing 2^ue
  const double r = rint(ldexp(x, -ue));           // exact scaling, then RNE
  return f2h_bits((float)ldexp(r, ue));           // r 2^ue is an fp16 value
}

// y = R x for one 128-value block held two values per lane (lane l:
// elements 2l, 2l+1): signed sums in binary64 (exact for fp16 inputs), one
// multiply by 1/sqrt(128), the second sign flip, one rounding to fp32.
__device__ __forceinline__ void rwht128_exact(const uint16_t* __restrict__ src, int lane, const uint32_t* signs,
                                              float (&y)[2]) {
  double x[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    double v = (double)h2f(src[2 * lane + j]);
    x[j] = sign_neg(signs, 2 * lane + j) ? -v : v;
  }
  {
    const double p = x[0], q = x[1];
    x[0] = p + q;
    x[1] = p - q;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const double o = shfl_xor_d(x[j], m);
      x[j] = (lane & m) ? (o - x[j]) : (x[j] + o);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const double r = x[j] * kInvSqrt128;
    y[j] = (float)(sign_neg(signs, 128 + 2 * lane + j) ? -r : r);
  }
}

// Forward or inverse rotation of VPL values per lane, one RWHT per 128
// consecutive elements (lane l holds elements VPL l ..): fp32.
template <int VPL, bool kInverse>
__device__ __forceinline__ void rwht128_f32(float (&v)[VPL], int lane, const uint32_t* signs) {
  const int first = kInverse ? 128 : 0, second = kInverse ? 0 : 128;
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if (sign_neg(signs, first + ((VPL * lane + j) & 127))) v[j] = -v[j];
  wave_fwht<VPL, 128>(v, lane);
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    v[j] *= (float)kInvSqrt128;
    if (sign_neg(signs, second + ((VPL * lane + j) & 127))) v[j] = -v[j];
  }
}

}  // namespace

// One wave per block, four blocks per workgroup.
__global__ __launch_bounds__(256) void tbq4_encode_kernel(Tbq4CodecArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= a.n) return;
  float y[2];
  rwht128_exact(a.x + blk * 128, lane, a.signs, y);
  double s = (double)y[0] * (double)y[0] + (double)y[1] * (double)y[1];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s += shfl_xor_d(s, m);  // same sum in every lane
  const uint16_t nb = d2h_bits_nonneg(sqrt(s));
  const float nf = h2f(nb);
  const float inv = nf > 0.0f ? 1.0f / nf : 0.0f;
  uint32_t byte = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float v = y[j] * inv;
    uint32_t k = 0;
#pragma unroll
    for (int t = 0; t < 15; ++t) k += v > a.bnd[t] ? 1u : 0u;
    byte |= k << (4 * j);
  }
  const uint32_t up = __shfl_xor(byte, 1, 64);
  uint8_t* out = a.blocks_out + blk * kTbqBytes;
  if (!(lane & 1)) *(uint16_t*)(out + 2 + lane) = (uint16_t)(byte | (up << 8));
  if (lane == 0) *(uint16_t*)out = nb;
}

// x^ = R^T (centroid[index] * norm) in fp32, one wave per block.
__global__ __launch_bounds__(256) void tbq4_decode_kernel(Tbq4CodecArgs a) {
  __shared__ float cent[16];
  if (threadIdx.x < 16) cent[threadIdx.x] = a.cent[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= a.n) return;
  const uint8_t* in = a.blocks_in + blk * kTbqBytes;
  const float nf = h2f(*(const uint16_t*)in);
  const uint32_t byte = in[2 + lane];
  float v[2] = {cent[byte & 15] * nf, cent[byte >> 4] * nf};
  rwht128_f32<2, true>(v, lane, a.signs);
  *(float2*)(a.y + blk * 128 + 2 * lane) = make_float2(v[0], v[1]);
}

// tqB_0 comparator blocks, B = 5 or 6 bits (SJ-KVaRN section 6 compares
// against the rotated 5-bit format; the 6-bit one is the staging format): the
// 128-point rotation as above, then the symmetric uniform quantiser of the
// staging format with 2^(B-1) - 1 levels a side: d = fp16(amax / L) by IEEE
// fp32 division, q = clamp(rne(y * fp32(1 / d)), -L, L), u = q + 2^(B-1);
// block = [fp16 d][16 B bytes: LSB-first B-bit stream].  One wave per block:
// lane l holds codes 2l and 2l + 1, so four lanes hold B whole bytes.
template <int B>
__global__ __launch_bounds__(256) void tq_encode_kernel(Tbq4CodecArgs a) {
  constexpr int LEVEL = (1 << (B - 1)) - 1, OFF = 1 << (B - 1), BYTES = 2 + 16 * B;
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= a.n) return;
  float y[2];
  rwht128_exact(a.x + blk * 128, lane, a.signs, y);
  float am = fmaxf(fabsf(y[0]), fabsf(y[1]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, shfl_xor_f(am, m));
  const uint16_t dbits = f2h_bits(am / (float)LEVEL);
  const float d = h2f(dbits);
  const float inv = d > 0.0f ? 1.0f / d : 0.0f;
  uint32_t pair = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float q = fminf(fmaxf(rintf(y[j] * inv), -(float)LEVEL), (float)LEVEL);
    pair |= (uint32_t)((int)q + OFF) << (B * j);
  }
  const int g0 = lane & ~3;
  const uint64_t w = (uint64_t)__shfl(pair, g0, 64) | ((uint64_t)__shfl(pair, g0 + 1, 64) << (2 * B)) |
                     ((uint64_t)__shfl(pair, g0 + 2, 64) << (4 * B)) | ((uint64_t)__shfl(pair, g0 + 3, 64) << (6 * B));
  uint8_t* out = a.blocks_out + blk * BYTES;
  if ((lane & 3) == 0) {
#pragma unroll
    for (int k = 0; k < B; ++k) out[2 + B * (lane >> 2) + k] = (uint8_t)(w >> (8 * k));
  }
  if (lane == 0) *(uint16_t*)out = dbits;
}

// x^ = R^T (d (u - 2^(B-1))) in fp32, one wave per block.
template <int B>
__global__ __launch_bounds__(256) void tq_decode_kernel(Tbq4CodecArgs a) {
  constexpr int OFF = 1 << (B - 1), BYTES = 2 + 16 * B;
  constexpr uint32_t MASK = (1u << B) - 1u;
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= a.n) return;
  const uint8_t* in = a.blocks_in + blk * BYTES;
  const float d = h2f(*(const uint16_t*)in);
  const int bit = 2 * B * lane, sh = bit & 7, nbytes = (sh + 2 * B + 7) >> 3;  // 2 or 3, inside the block
  const uint8_t* p = in + 2 + (bit >> 3);
  uint32_t w = p[0] | ((uint32_t)p[1] << 8);
  if (nbytes > 2) w |= (uint32_t)p[2] << 16;
  w >>= sh;
  float v[2] = {d * (float)((int)(w & MASK) - OFF), d * (float)((int)((w >> B) & MASK) - OFF)};
  rwht128_f32<2, true>(v, lane, a.signs);
  *(float2*)(a.y + blk * 128 + 2 * lane) = make_float2(v[0], v[1]);
}

// The query of every (sequence, query head) rotated once and scaled by
// softmax scale x log2(e): fp32 [n_seqs][Hq][D] in the workspace.
template <int D>
__global__ __launch_bounds__(64) void tbq4_rotq_kernel(Tbq4AttnArgs a) {
  constexpr int VPL = D / 64;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.y * a.Hq + blockIdx.x;
  const uint16_t* qp = a.q + row * D + VPL * lane;
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = h2f(qp[j]);
  rwht128_f32<VPL, false>(v, lane, a.signs);
#pragma unroll
  for (int j = 0; j < VPL; ++j) a.qr[row * D + VPL * lane + j] = v[j] * a.scale_log2;
}

// Split-K decode attention over a TBQ4 cache, one wave per (token chunk, KV
// head, sequence), all GM >= g query heads of the group.  Per pass of 64
// tokens: lane = token for the scores (each lane reads its key blocks; the
// rotated queries are the same for every lane), then lane = channel for the
// values (the weights of token j are read from lane j).  Scores are kept in
// log2 units.  The kernel stores to global memory only after its loops.
template <int D, int GM>
__global__ __launch_bounds__(64) void tbq4_attn_kernel(Tbq4AttnArgs a) {
  constexpr int NB = D / 128, VPL = D / 64, TB = 16;
  __shared__ float cent[16];
  const int lane = threadIdx.x, c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t len = a.len[b];
  const int64_t t0 = (int64_t)c * a.chunk;
  if (t0 >= len) return;  // past this sequence's last chunk: the merge reads no row of it
  const int64_t t1 = len < t0 + a.chunk ? len : t0 + a.chunk;
  const int g = a.g;
  if (lane < 16) cent[lane] = a.cent[lane];
  __syncthreads();
  const float* __restrict__ qg = a.qr + ((int64_t)b * a.Hq + h * g) * D;
  const int64_t head_tok0 = ((int64_t)b * a.H + h) * a.cap;
  const int nbl = (VPL * lane) >> 7;                      // the lane's block in the value phase
  const int vbyte = 2 + (((VPL * lane) & 127) >> 1);      // its first index byte there
  float m[GM], l[GM], acc[GM][VPL];
#pragma unroll
  for (int i = 0; i < GM; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[i][j] = 0.0f;
  }
  for (int64_t base = t0; base < t1; base += 64) {
    const int64_t t = base + lane;
    const bool valid = t < t1;
    const int n_here = (int)(t1 - base < 64 ? t1 - base : 64);
    float s[GM], vn[NB];
#pragma unroll
    for (int i = 0; i < GM; ++i) s[i] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vn[nb] = 0.0f;
    if (valid) {
      const uint8_t* kp = a.kb + (head_tok0 + t) * (NB * kTbqBytes);
      const uint8_t* vp = a.vb + (head_tok0 + t) * (NB * kTbqBytes);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint16_t* k16 = (const uint16_t*)(kp + nb * kTbqBytes);
        const float kn = h2f(k16[0]);
        vn[nb] = h2f(*(const uint16_t*)(vp + nb * kTbqBytes));
        float part[GM];
#pragma unroll
        for (int i = 0; i < GM; ++i) part[i] = 0.0f;
#pragma unroll 8
        for (int w = 0; w < 32; ++w) {
          const uint32_t u = k16[1 + w];
          const float c0 = cent[u & 15], c1 = cent[(u >> 4) & 15], c2 = cent[(u >> 8) & 15], c3 = cent[u >> 12];
#pragma unroll
          for (int i = 0; i < GM; ++i) {
            if (i < g) {
              const float* qq = qg + i * D + nb * 128 + 4 * w;
              part[i] = fmaf(qq[0], c0, part[i]);
              part[i] = fmaf(qq[1], c1, part[i]);
              part[i] = fmaf(qq[2], c2, part[i]);
              part[i] = fmaf(qq[3], c3, part[i]);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < GM; ++i) s[i] = fmaf(part[i], kn, s[i]);
      }
    }
    float pr[GM];
#pragma unroll
    for (int i = 0; i < GM; ++i) {
      pr[i] = 0.0f;
      if (i < g) {
        const float si = valid ? s[i] : -INFINITY;
        float mx = si;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
        const float mn = fmaxf(m[i], mx);               // finite: the pass holds a valid token
        const float alpha = exp2f(m[i] - mn);           // 0 before the first pass
        const float p = exp2f(si - mn);
        float ps = p;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) ps += shfl_xor_f(ps, o);
        l[i] = fmaf(l[i], alpha, ps);
#pragma unroll
        for (int j = 0; j < VPL; ++j) acc[i][j] *= alpha;
        m[i] = mn;
        pr[i] = p;
      }
    }
    const uint8_t* vrow = a.vb + (head_tok0 + base) * (NB * kTbqBytes) + nbl * kTbqBytes + vbyte;
    for (int j0 = 0; j0 < n_here; j0 += TB) {
      uint32_t ub[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        ub[u] = 0;
        if (j0 + u < n_here) {
          const uint8_t* ptr = vrow + (int64_t)(j0 + u) * (NB * kTbqBytes);
          ub[u] = VPL == 2 ? (uint32_t)*ptr : (uint32_t)*(const uint16_t*)ptr;
        }
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int j = j0 + u;
        if (j < n_here) {
          float cv[VPL];
#pragma unroll
          for (int e = 0; e < VPL; ++e) cv[e] = cent[(ub[u] >> (4 * e)) & 15];
          float vnj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vn[0]), j));
          if constexpr (NB == 2) {
            const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vn[1]), j));
            vnj = nbl ? v1 : vnj;
          }
#pragma unroll
          for (int i = 0; i < GM; ++i) {
            if (i < g) {
              const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr[i]), j)) * vnj;
#pragma unroll
              for (int e = 0; e < VPL; ++e) acc[i][e] = fmaf(w, cv[e], acc[i][e]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < GM; ++i) {
    if (i < g) {
      float v[VPL];
#pragma unroll
      for (int j = 0; j < VPL; ++j) v[j] = acc[i][j];
      rwht128_f32<VPL, true>(v, lane, a.signs);
      float* P = a.part + (((int64_t)b * a.Hq + h * g + i) * a.max_chunks + c) * part_stride(D);
      float* dst = P + kPartHead + VPL * lane;
      if constexpr (VPL == 2) {
        *(float2*)dst = make_float2(v[0], v[1]);
      } else {
        *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (lane == 0) {
        P[0] = m[i] * kLn2f;
        P[1] = l[i];
      }
    }
  }
}

hipError_t launch_tbq4_encode(const Tbq4CodecArgs& a, hipStream_t stream) {
  const int64_t grid = (a.n + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tbq4_encode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tbq4_decode(const Tbq4CodecArgs& a, hipStream_t stream) {
  const int64_t grid = (a.n + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tbq4_decode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tq_codec(const Tbq4CodecArgs& a, int bits, bool encode, hipStream_t stream) {
  const int64_t grid = (a.n + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), blk(256);
  if (bits == 5 && encode) hipLaunchKernelGGL(tq_encode_kernel<5>, g, blk, 0, stream, a);
  else if (bits == 5) hipLaunchKernelGGL(tq_decode_kernel<5>, g, blk, 0, stream, a);
  else if (bits == 6 && encode) hipLaunchKernelGGL(tq_encode_kernel<6>, g, blk, 0, stream, a);
  else if (bits == 6) hipLaunchKernelGGL(tq_decode_kernel<6>, g, blk, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_d(const Tbq4AttnArgs& a, dim3 grid, hipStream_t stream) {
  if (a.g <= 4)
    hipLaunchKernelGGL((tbq4_attn_kernel<D, 4>), grid, dim3(64), 0, stream, a);
  else if (a.g <= 8)
    hipLaunchKernelGGL((tbq4_attn_kernel<D, 8>), grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((tbq4_attn_kernel<D, 16>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tbq4_attn(const Tbq4AttnArgs& a, int grid_x, hipStream_t stream) {
  if (a.g < 1 || a.g > kMaxGroup) return hipErrorInvalidValue;
  dim3 grid(grid_x, a.H, a.n_seqs), qgrid(a.Hq, a.n_seqs);
  switch (a.D) {
    case 128:
      hipLaunchKernelGGL(tbq4_rotq_kernel<128>, qgrid, dim3(64), 0, stream, a);
      return launch_attn_d<128>(a, grid, stream);
    case 256:
      hipLaunchKernelGGL(tbq4_rotq_kernel<256>, qgrid, dim3(64), 0, stream, a);
      return launch_attn_d<256>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
