// Split-K decode attention over the four regions, vector-ALU path, and the
// merge of all partials under one softmax.
//
// SJ-KVaRN 2.1: one pass reads the sink, the staging ring (the exact tail) and
// the sealed body.  KV Cache Precision Tail section 2: the region results are
// combined under one softmax.  KV cache math ("rotate first"): the query is
// rotated once, ring and body are read in the rotated domain, the output is
// rotated back once.  The sink is kept in the original domain and is scored
// with the unrotated query.
//
// Work split: chunk 0 of a sequence is its sink; then ring chunks of
// ring_chunk tokens; then body chunks (the records split evenly).  Each
// workgroup handles one chunk of one KV head for its g query heads and writes
// an fp32 partial (m, l, acc[D]): m the largest score, l = sum exp(s - m),
// acc = sum exp(s - m) v (in the rotated domain, except for chunk 0).
// The merge kernel combines the partials of one query head, applies R^T to the
// rotated part, adds the sink part and divides by the total weight.
//
// This path dequantises each tile into LDS as fp32 and uses plain fp32 dot
// products: it is the reference the matrix-core body path is checked against.
#include "kvq_device.h"

namespace kvq {

// In-place rotation of one D-vector held in LDS by a 256-thread block.
// forward: R x (signs s1 then transform then s2 for D = 128); inverse: R^T x.
template <int D>
__device__ void lds_rotate(float* v, const uint32_t* signs, bool inverse) {
  const int tid = threadIdx.x;
  if (D == 128) {
    for (int i = tid; i < D; i += 256)
      if (sign_neg(signs, (inverse ? 128 : 0) + i)) v[i] = -v[i];
    __syncthreads();
  }
  constexpr int CH = D == 128 ? 128 : 256;
  for (int st = 1; st < CH; st <<= 1) {
    for (int p = tid; p < D / 2; p += 256) {
      const int i = (p / st) * 2 * st + (p % st);
      const float a = v[i], b = v[i + st];
      v[i] = a + b;
      v[i + st] = a - b;
    }
    __syncthreads();
  }
  for (int i = tid; i < D; i += 256) {
    float x = v[i];
    if (D == 128) {
      x = x * (float)kInvSqrt128;
      if (sign_neg(signs, (inverse ? 0 : 128) + i)) x = -x;
    } else {
      x = x * 0.0625f;
    }
    v[i] = x;
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  constexpr int TS = 8192 / D;  // tokens per LDS tile
  constexpr int DP = D + 1;
  constexpr int CPT = (D + 255) / 256;
  __shared__ float qs[kMaxGroup][D];
  __shared__ float kt[TS][DP];
  __shared__ float vt[TS][DP];
  __shared__ float sc[kMaxGroup][TS];
  __shared__ float ms[kMaxGroup], lsum[kMaxGroup], al[kMaxGroup];

  const Layout& y = a.y;
  const int c = blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const DecodeSeq sq = a.seq[b];
  prof_start(a.prof_ts);
  if (c >= sq.n_chunks) return;
  const int tid = threadIdx.x;
  const int g = a.g;
  const int s = sq.slot, layer = a.layer;
  const int region = c == 0 ? 0 : (c < 1 + sq.n_ring_chunks ? 1 : 2);
  if (!((a.valu_regions >> region) & 1)) return;  // region handled by a matrix-core kernel

  for (int idx = tid; idx < g * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    qs[i][j] = h2f(a.q[((int64_t)b * a.Hq + h * g + i) * D + j]);
  }
  if (tid < kMaxGroup) {
    ms[tid] = -INFINITY;
    lsum[tid] = 0.0f;
  }
  __syncthreads();
  if (region != 0)
    for (int i = 0; i < g; ++i) lds_rotate<D>(qs[i], a.signs, false);

  int t_begin, t_end;
  if (region == 0) {
    t_begin = 0;
    t_end = sq.n_sink;
  } else if (region == 1) {
    t_begin = (c - 1) * a.ring_chunk;
    t_end = min(sq.ring_len, t_begin + a.ring_chunk);
  } else {
    const int cb = c - 1 - sq.n_ring_chunks;  // records split evenly over the body chunks
    t_begin = (int)((int64_t)cb * sq.n_rec / sq.n_body_chunks) * kGroup;
    t_end = (int)((int64_t)(cb + 1) * sq.n_rec / sq.n_body_chunks) * kGroup;
  }

  float acc[kMaxGroup][CPT];
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i)
#pragma unroll
    for (int q = 0; q < CPT; ++q) acc[i][q] = 0.0f;

  const uint16_t* sink = (const uint16_t*)(a.arena + y.off_sink);
  for (int t0 = t_begin; t0 < t_end; t0 += TS) {
    const int nt = min(TS, t_end - t0);
    for (int idx = tid; idx < nt * D; idx += 256) {
      const int t = idx / D, j = idx % D;
      const int tok = t0 + t;
      float kx, vx;
      if (region == 0) {
        kx = h2f(sink[sink_elem(y, s, layer, h, 0, tok) + j]);
        vx = h2f(sink[sink_elem(y, s, layer, h, 1, tok) + j]);
      } else if (region == 1) {
        const int slot = (sq.ring0 + tok) % y.cap;
        const int blk = j / kQBlock, k = j % kQBlock;
        const int bit = 6 * k;
        float xs[2];
        for (int kv = 0; kv < 2; ++kv) {
          const uint8_t* cp = a.arena + rcode_off(y, s, layer, h, kv, slot) + blk * kQBytes + (bit >> 3);
          uint32_t two = cp[0];
          if ((bit & 7) > 2) two |= (uint32_t)cp[1] << 8;  // the code straddles two bytes
          const int u = (int)((two >> (bit & 7)) & 63u);
          const float d = h2f(((const uint16_t*)(a.arena + rscale_off(y, s, layer, h, kv, slot)))[blk]);
          xs[kv] = d * (float)(u - 32);
        }
        kx = xs[0];
        vx = xs[1];
      } else {
        const int r = tok / kGroup, ti = tok % kGroup;
        const int sub = j / y.sub, jj = j % y.sub;
        const uint8_t* rec = a.arena + rec_off(y, s, layer, h, r) + (int64_t)sub * y.sub_bytes;
        const uint8_t* km = rec + y.kcode_bytes + y.vcode_bytes;
        const uint8_t* vm = km + 2 * (y.sub + 2 * kGroup);
        int kc;
        if (y.kbits == 4) {
          const uint8_t byte = rec[(int64_t)ti * (y.sub / 2) + jj / 2];
          kc = (jj & 1) ? (byte >> 4) : (byte & 15);
        } else {
          kc = rec[(int64_t)ti * y.sub + jj];
        }
        const uint8_t vbyte = rec[y.kcode_bytes + (int64_t)jj * (kGroup / 2) + ti / 2];
        const int vc = (ti & 1) ? (vbyte >> 4) : (vbyte & 15);
        const uint16_t* kmh = (const uint16_t*)km;
        const uint16_t* vmh = (const uint16_t*)vm;
        kx = h2f(kmh[jj]) * (h2f(kmh[y.sub + ti]) * (float)kc + h2f(kmh[y.sub + kGroup + ti]));
        vx = h2f(vmh[jj]) * (h2f(vmh[y.sub + ti]) * (float)vc + h2f(vmh[y.sub + kGroup + ti]));
      }
      kt[t][j] = kx;
      vt[t][j] = vx;
    }
    __syncthreads();
    for (int idx = tid; idx < g * nt; idx += 256) {
      const int i = idx / nt, t = idx % nt;
      float dot = 0.0f;
      for (int j = 0; j < D; ++j) dot = fmaf(qs[i][j], kt[t][j], dot);
      sc[i][t] = dot * a.scale;
    }
    __syncthreads();
    if (tid < g) {
      const int i = tid;
      float mx = ms[i];
      for (int t = 0; t < nt; ++t) mx = fmaxf(mx, sc[i][t]);
      const float alpha = expf(ms[i] - mx);
      float sum = 0.0f;
      for (int t = 0; t < nt; ++t) {
        const float p = expf(sc[i][t] - mx);
        sc[i][t] = p;
        sum += p;
      }
      lsum[i] = lsum[i] * alpha + sum;
      ms[i] = mx;
      al[i] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int j = tid + 256 * q;
      if (j < D) {
#pragma unroll
        for (int i = 0; i < kMaxGroup; ++i) {
          if (i < g) {
            float v = acc[i][q] * al[i];
            for (int t = 0; t < nt; ++t) v = fmaf(sc[i][t], vt[t][j], v);
            acc[i][q] = v;
          }
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i) {
    if (i >= g) break;
    float* P = a.part + (((int64_t)b * a.Hq + h * g + i) * a.max_chunks + c) * (D + 2);
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int j = tid + 256 * q;
      if (j < D) P[2 + j] = acc[i][q];
    }
    if (tid == 0) {
      P[0] = ms[i];
      P[1] = lsum[i];
    }
  }
  prof_end(a.prof_ts);
}

// Merge of the split-K partials of one query head (grid Hq x n_seqs, 1024
// threads): one softmax over all chunks, R^T applied to the rotated part
// (chunks 1..), the sink part (chunk 0) added as is, divided by the total
// weight.  The 16 waves split the chunks (more loads in flight than a
// 256-thread block); each lane owns D / 64 channels.
constexpr int kMergeWaves = 16;
constexpr int kMergeUnroll = 8;  // partials per wave and pass, all loaded before any is used

// One workgroup per (sequence, query head).  Wave w takes partials
// w, w + NW, ... in passes of kMergeUnroll: every load of a pass (the rows and
// their (m, l), the latter broadcast to all lanes) is issued before the first
// is used, so a pass costs one memory round trip, and the wave keeps a running
// (M, L, sum e^(m - M) acc) in registers with no cross-lane step.  The waves'
// states meet in LDS; wave 0 rotates the rotated-domain sum back and adds the
// sink's partial (chunk 0, original domain).
template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeArgs a) {
  constexpr int VPL = D / 64, NW = kMergeWaves, U = kMergeUnroll;
  __shared__ float red[NW][D];
  __shared__ float rm[2 * NW];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.n_chunks[b];
  const float* P = a.part + ((int64_t)b * a.Hq + hq) * a.max_chunks * (D + 2);

  float M = -INFINITY, L = 0.0f;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = 0.0f;
  float sink[VPL];
  float m0 = 0.0f;
  if (wave == 0) {
    m0 = P[0];
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i) {
      const float2 x = ((const float2*)(P + 2 + VPL * lane))[i];
      sink[2 * i] = x.x;
      sink[2 * i + 1] = x.y;
    }
  }
  for (int base = 0; base < n; base += NW * U) {
    float2 ml[U];
    float x[U][VPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + wave + NW * u;
      const float* row = P + (int64_t)(c < n ? c : 0) * (D + 2);
      ml[u] = *(const float2*)row;
#pragma unroll
      for (int i = 0; i < VPL / 2; ++i) {
        const float2 t = ((const float2*)(row + 2 + VPL * lane))[i];
        x[u][2 * i] = t.x;
        x[u][2 * i + 1] = t.y;
      }
    }
    float mp = M;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + wave + NW * u < n) mp = fmaxf(mp, ml[u].x);
    const float alpha = M == -INFINITY ? 0.0f : expf(M - mp);  // nothing to rescale before the first partial
    L *= alpha;
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] *= alpha;
    M = mp;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + wave + NW * u;
      if (c < n) {
        const float w = expf(ml[u].x - M);
        L = fmaf(w, ml[u].y, L);
        if (c > 0) {  // chunk 0 (the sink) is in the original domain: added after the rotation
#pragma unroll
          for (int i = 0; i < VPL; ++i) v[i] = fmaf(w, x[u][i], v[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) red[wave][VPL * lane + i] = v[i];
  if (lane == 0) {
    rm[wave] = M;
    rm[NW + wave] = L;
  }
  __syncthreads();
  if (wave != 0) return;
  float Mt = rm[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mt = fmaxf(Mt, rm[w]);
  float Lt = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float s = rm[w] == -INFINITY ? 0.0f : expf(rm[w] - Mt);  // a wave with no partial has M = -inf
    Lt = fmaf(s, rm[NW + w], Lt);
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] = fmaf(s, red[w][VPL * lane + i], v[i]);
  }
  // R^T: head_dim 128: s1 . H . s2 / sqrt(128); 256 and 512: H_256 / 16 per 256-block
  if (D == 128) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (sign_neg(a.signs, 128 + VPL * lane + i)) v[i] = -v[i];
    wave_fwht<VPL, 128>(v, lane);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      v[i] *= (float)kInvSqrt128;
      if (sign_neg(a.signs, VPL * lane + i)) v[i] = -v[i];
    }
  } else {
    wave_fwht<VPL, 256>(v, lane);
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] *= 0.0625f;
  }
  const float w0 = expf(m0 - Mt);
  const float inv_l = 1.0f / Lt;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = VPL * lane + i;
    const float o = fmaf(w0, sink[i], v[i]) * inv_l;
    const int64_t oi = ((int64_t)b * a.Hq + hq) * D + j;
    if (a.out_f16)
      ((uint16_t*)a.out)[oi] = f2h_bits(o);
    else
      ((float*)a.out)[oi] = o;
  }
}

hipError_t launch_decode_valu(const DecodeArgs& a, int grid_x, hipStream_t stream) {
  dim3 grid(grid_x, a.y.H, a.n_seqs);
  switch (a.y.D) {
    case 128: hipLaunchKernelGGL(decode_valu_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_valu_kernel<256>, grid, dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL(decode_valu_kernel<512>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  dim3 grid(a.Hq, a.n_seqs);
  switch (a.D) {
    case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64 * kMergeWaves), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(64 * kMergeWaves), 0, stream, a); break;
    case 512: hipLaunchKernelGGL(merge_kernel<512>, grid, dim3(64 * kMergeWaves), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
