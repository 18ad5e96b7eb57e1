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
// an fp32 partial row (m, l, acc[D]): m the largest score, l = sum exp(s - m),
// acc = sum exp(s - m) v, rotated back to the original domain by the
// workgroup (R^T is linear).  The merge kernel combines the partials of one
// query head under one softmax and divides by the total weight.
//
// This path is the reference the matrix-core path is checked against.  The
// score side runs in binary64: the query is rotated exactly (a signed sum of
// fp16 values), keys are dequantised exactly (fp16 products), the dot products
// and the scores are binary64, so that scores in the thousands (keys near the
// fp16 maximum) keep their fraction; each chunk's reference maximum is rounded
// to fp32 before its weights are taken from it, so that the partial it writes
// is exact relative to the m the merge reads.  Values and weights are fp32.
#include <mutex>

#include "kvq_device.h"

namespace kvq {

// In-place rotation of one D-vector held in LDS by a 256-thread block.
// forward: R x (signs s1 then transform then s2 for D = 128); inverse: R^T x.
template <int D, typename T>
__device__ void lds_rotate(T* v, const uint32_t* signs, bool inverse) {
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
      const T a = v[i], b = v[i + st];
      v[i] = a + b;
      v[i + st] = a - b;
    }
    __syncthreads();
  }
  for (int i = tid; i < D; i += 256) {
    T x = v[i];
    if (D == 128) {
      x = x * (T)kInvSqrt128;
      if (sign_neg(signs, (inverse ? 0 : 128) + i)) x = -x;
    } else {
      x = x * (T)0.0625;
    }
    v[i] = x;
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  constexpr int TS = 4096 / D;  // tokens per LDS tile
  constexpr int DP = D + 1;
  constexpr int CPT = (D + 255) / 256;
  __shared__ double qs[kMaxGroup][D];  // query rows (binary64), later the partial rows
  __shared__ double kt[TS][DP];
  __shared__ float vt[TS][DP];
  __shared__ double sd[kMaxGroup][TS];  // scores
  __shared__ float sc[kMaxGroup][TS];   // weights
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
  // ring (tq6_0 staging) and body are read in the rotated domain; the sink and
  // an f16-staged ring in the original domain
  const bool rotated = region == 2 || (region == 1 && !y.f16ring);

  for (int idx = tid; idx < g * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    qs[i][j] = (double)h2f(a.q[((int64_t)b * a.Hq + h * g + i) * D + j]);
  }
  if (tid < kMaxGroup) {
    ms[tid] = -INFINITY;
    lsum[tid] = 0.0f;
  }
  __syncthreads();
  if (rotated)
    for (int i = 0; i < g; ++i) lds_rotate<D, double>(qs[i], a.signs, false);

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
      double kx;
      float vx;
      if (region == 0) {
        kx = h2f(sink[sink_elem(y, s, layer, h, 0, tok) + j]);
        vx = h2f(sink[sink_elem(y, s, layer, h, 1, tok) + j]);
      } else if (region == 1 && y.f16ring) {
        const int slot = (sq.ring0 + tok) % y.cap;
        kx = h2f(((const uint16_t*)(a.arena + rcode_off(y, s, layer, h, 0, slot)))[j]);
        vx = h2f(((const uint16_t*)(a.arena + rcode_off(y, s, layer, h, 1, slot)))[j]);
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
        // code k of a row: stream bits b k .. b k + b - 1, LSB first
        auto code = [](const uint8_t* row, int k, int bits) {
          const int bit = bits * k;
          uint32_t w = row[bit >> 3];
          if ((bit & 7) + bits > 8) w |= (uint32_t)row[(bit >> 3) + 1] << 8;
          return (int)((w >> (bit & 7)) & ((1u << bits) - 1));
        };
        const int kc = code(rec + (int64_t)ti * (y.sub * y.kbits / 8), jj, y.kbits);
        const int vc = code(rec + y.kcode_bytes + (int64_t)jj * (kGroup * y.vbits / 8), ti, y.vbits);
        const float vmid = (float)(1 << (y.vbits - 1));
        const uint16_t* kmh = (const uint16_t*)km;
        const uint16_t* vmh = (const uint16_t*)vm;
        // keys exact in binary64: C (S n + Z) of fp16 C, S, Z; values centred,
        // C (S (n - mid) + (Z + mid S)) in fp32 (mid = 2^(b-1); Z + mid S exact),
        // so that rows whose range is far above their values do not cancel
        kx = (double)h2f(kmh[jj]) *
             ((double)h2f(kmh[y.sub + ti]) * (double)kc + (double)h2f(kmh[y.sub + kGroup + ti]));
        const float vs = h2f(vmh[y.sub + ti]);
        vx = h2f(vmh[jj]) * fmaf(vs, (float)vc - vmid, fmaf(vmid, vs, h2f(vmh[y.sub + kGroup + ti])));
      }
      kt[t][j] = kx;
      vt[t][j] = vx;
    }
    __syncthreads();
    for (int idx = tid; idx < g * nt; idx += 256) {
      const int i = idx / nt, t = idx % nt;
      double dot = 0.0;
      for (int j = 0; j < D; ++j) dot = fma(qs[i][j], kt[t][j], dot);
      sd[i][t] = dot * (double)a.scale;
    }
    __syncthreads();
    if (tid < g) {
      const int i = tid;
      double mxd = ms[i];
      for (int t = 0; t < nt; ++t) mxd = fmax(mxd, sd[i][t]);
      const float mx = (float)mxd;  // the chunk's reference, as the partial will hold it
      const float alpha = expf(ms[i] - mx);
      float sum = 0.0f;
      for (int t = 0; t < nt; ++t) {
        const float p = (float)exp(sd[i][t] - (double)mx);
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

  // rotated-domain sums back to the original domain (the sink's already are)
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i) {
    if (i >= g) break;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int j = tid + 256 * q;
      if (j < D) qs[i][j] = acc[i][q];
    }
  }
  __syncthreads();
  if (rotated)
    for (int i = 0; i < g; ++i) lds_rotate<D, double>(qs[i], a.signs, true);
  for (int i = 0; i < g; ++i) {
    float* P = a.part + (((int64_t)b * a.Hq + h * g + i) * a.max_chunks + c) * part_stride(D);
    for (int j = tid; j < D; j += 256) P[kPartHead + j] = (float)qs[i][j];
    if (tid == 0) {
      P[0] = ms[i];
      P[1] = lsum[i];
    }
  }
  prof_end(a.prof_ts);
}

// Merge of the split-K partials (all in the original domain): one softmax
// over the chunks of a query row, divided by the total weight.  One
// workgroup per (sequence, query token, query head, 64-channel slice; one
// query token per sequence for decode, the block's n_q for block attention,
// whose partials with l = 0, fully masked, carry a finite m): thread t takes
// channels 4 (t & 15) .. + 3 of the slice and chunks t >> 4, + 16, ...; every
// load of a pass (the rows' float4 and their (m, l)) is issued before any is
// used, so a pass costs one memory round trip, and each thread keeps a
// running (M, L, sum e^(m - M) acc).  The 16 row groups meet in LDS.
constexpr int kMergeUnroll = 8;  // partials per thread and pass

// e^x for x <= 0 by the hardware base-2 exponential (the merge weights need
// fp32 precision, not correct rounding; the partials' m are in natural-log units)
__device__ __forceinline__ float exp_le0(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int NSL = D / 64, U = kMergeUnroll;
  __shared__ float4 red[16][16];
  __shared__ float rm[2][16];
  const int hq = blockIdx.x / NSL, sl = blockIdx.x % NSL, b = blockIdx.z;
  const int64_t row = ((int64_t)b * a.n_rows + blockIdx.y) * a.Hq + hq;  // (sequence, query token, head)
  const int tid = threadIdx.x, rg = tid >> 4, cq = tid & 15;
  const int n = a.n_chunks[b];
  const int ch = 64 * sl + 4 * cq;
  const float* P = a.part + row * a.max_chunks * part_stride(D);

  float M = -INFINITY, L = 0.0f;
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int base = 0; base < n; base += 16 * U) {
    float2 ml[U];
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + rg + 16 * u;
      const float* row = P + (int64_t)(c < n ? c : 0) * part_stride(D);
      ml[u] = *(const float2*)row;
      x[u] = *(const float4*)(row + kPartHead + ch);
    }
    float mp = M;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + rg + 16 * u < n) mp = fmaxf(mp, ml[u].x);
    const float alpha = M == -INFINITY ? 0.0f : exp_le0(M - mp);  // nothing to rescale before the first partial
    L *= alpha;
    v.x *= alpha;
    v.y *= alpha;
    v.z *= alpha;
    v.w *= alpha;
    M = mp;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + rg + 16 * u < n) {
        const float w = exp_le0(ml[u].x - M);
        L = fmaf(w, ml[u].y, L);
        v.x = fmaf(w, x[u].x, v.x);
        v.y = fmaf(w, x[u].y, v.y);
        v.z = fmaf(w, x[u].z, v.z);
        v.w = fmaf(w, x[u].w, v.w);
      }
    }
  }
  red[rg][cq] = v;
  if (cq == 0) {
    rm[0][rg] = M;
    rm[1][rg] = L;
  }
  __syncthreads();
  if (tid >= 16) return;
  float Mt = rm[0][0];
#pragma unroll
  for (int r = 1; r < 16; ++r) Mt = fmaxf(Mt, rm[0][r]);
  float Lt = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float s = rm[0][r] == -INFINITY ? 0.0f : exp_le0(rm[0][r] - Mt);  // a row group with no partial
    Lt = fmaf(s, rm[1][r], Lt);
    const float4 t = red[r][cq];
    o.x = fmaf(s, t.x, o.x);
    o.y = fmaf(s, t.y, o.y);
    o.z = fmaf(s, t.z, o.z);
    o.w = fmaf(s, t.w, o.w);
  }
  const float inv_l = 1.0f / Lt;
  const int64_t oi = row * D + ch;
  if (a.out_f16) {
    uint2 h;
    h.x = (uint32_t)f2h_bits(o.x * inv_l) | ((uint32_t)f2h_bits(o.y * inv_l) << 16);
    h.y = (uint32_t)f2h_bits(o.z * inv_l) | ((uint32_t)f2h_bits(o.w * inv_l) << 16);
    *(uint2*)((uint16_t*)a.out + oi) = h;
  } else {
    *(float4*)((float*)a.out + oi) = make_float4(o.x * inv_l, o.y * inv_l, o.z * inv_l, o.w * inv_l);
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
  if (a.n_rows < 1 || a.n_rows > 65535) return hipErrorInvalidValue;
  dim3 grid(a.Hq * (a.D / 64), a.n_rows, a.n_seqs);
  switch (a.D) {
    case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL(merge_kernel<512>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Device scratch of the allocation-free decode (kvq_attn_decode_noalloc): the
// split-K partial rows of one call.  One array per GPU the library runs on,
// held until the process ends; every call on a GPU shares it, so calls that
// overlap on one GPU race.  Nothing in it needs clearing: every partial row a
// merge reads is written by the same call first.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// The array's device address on the current device.  In host code the name
// `scratch` is a host-side stand-in, not a device address, so the address is
// taken once per device with hipGetSymbolAddress (with that device current)
// and kept; callers pass it to the kernels as they pass a workspace.
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace kvq
