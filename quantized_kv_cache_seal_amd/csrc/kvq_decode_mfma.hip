// Matrix-core scan of sealed body records (256-channel sub-tiles, 4-bit K and
// V): the hot loop of decode attention.
//
// KV cache math ("rotate first"): the query is rotated once and the raw
// blocks are read in the rotated domain, with no dequantise pass.  A record's
// key is k_ij = C_j (S_i code_ij + Z_i) (SJ-KVaRN 2.2: column balance scales
// absorbed, per-row scale and zero point), so for the rotated query q':
//     q'.k_i = S_i (q~ . code_i) + Z_i sigma,   q~_j = q'_j C_j,  sigma = sum_j q~_j
// and for values, with p_i the softmax weights of the record's rows:
//     sum_i p_i v_ij = C_j ( sum_i (p_i S_i) code_ij + sum_i p_i Z_i ).
// Both inner products are dense (16 query rows, the group padded to 16) x
// (32 codes) x (16 tokens or channels) and run on v_mfma_f32_16x16x32_f16.
//
// Codes reach the matrix cores without a conversion loop: one AND-OR per pair
// turns a nibble n into the fp16 1024 + n (low nibble) or 1024 + 16 n (high
// nibble of a byte, left in place); the x16 is folded into the other operand
// (q~/16 or p S/16), and one packed subtract restores exact, centred code
// values, so the fp32 accumulators never carry a large offset term.
//
// Orientation: S^T = K . Q~^T (A = key codes, rows = tokens) and
// O^T = V^T . P'^T (A = value codes, rows = channels), so the score layout that
// comes out of the first product is the operand layout the second needs, with
// no lane exchange.  Token rows are assigned so that lane group g (lanes
// 16g..16g+15) holds the 32 tokens 32g..32g+31 of a record; step t of the
// value product uses tokens 32g + 8t + 0..7, exactly one dword of the
// channel-major value row.
//
// Work split: one workgroup (4 waves) per chunk of records of one KV head;
// each wave takes every fourth record with its own online-softmax state; the
// four states are combined in LDS and written as one fp32 partial
// (m, l, acc[D]) in natural-log units, for the merge kernel.
#include "kvq_device.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ half8 nib8(uint32_t w) {
  // halves: [n0, n4, 16 n1, 16 n5, n2, n6, 16 n3, 16 n7] + 1024
  const uint32_t w8 = w >> 8;
  uint4 u;
  u.x = (w & 0x000F000Fu) | 0x64006400u;
  u.y = (w & 0x00F000F0u) | 0x64006400u;
  u.z = (w8 & 0x000F000Fu) | 0x64006400u;
  u.w = (w8 & 0x00F000F0u) | 0x64006400u;
  half8 h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

// Recentred code values n - 8 (slots of the high nibble: 16 (n - 8)), exact in
// fp16: one packed subtract removes the 1024 exponent offset and the centre.
// Centring matters for precision: with codes in [0, 15] the products carry a
// large common component S * 7.5 that the zero point later cancels, so fp16
// rounding of the weights would be amplified; the centre moves into the zero
// point instead (v = S (n - 8) + (Z + 8 S)).
__device__ __forceinline__ half8 nib8_centred(uint32_t w) {
  half8 h = nib8(w);
  const half8 off = {(_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1152.0f, (_Float16)1152.0f,
                     (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1152.0f, (_Float16)1152.0f};
  return h - off;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return (uint32_t)f2h_bits(lo) | ((uint32_t)f2h_bits(hi) << 16);
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

__device__ __forceinline__ float xsum4(float x) {  // sum over the four lane groups
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
__device__ __forceinline__ float xmax4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

// q~ = q' * C for one operand slot pair, split into hi + lo fp16 so that the
// score keeps fp32-level precision: q' = qh + ql (both fp16), hi = fp16(qh C),
// lo = fp16((qh C - hi) + ql C), with qh C - hi exact in fp32.
__device__ __forceinline__ void qtilde_pair(uint32_t qh2, uint32_t ql2, uint32_t c2, uint32_t& hi2, uint32_t& lo2) {
  const half2v qh = as_h2(qh2), ql = as_h2(ql2), c = as_h2(c2);
  const half2v hi = qh * c;
  float r0 = fmaf((float)qh[0], (float)c[0], -(float)hi[0]);
  float r1 = fmaf((float)qh[1], (float)c[1], -(float)hi[1]);
  r0 = fmaf((float)ql[0], (float)c[0], r0);
  r1 = fmaf((float)ql[1], (float)c[1], r1);
  hi2 = as_u32(hi);
  lo2 = pack_h2(r0, r1);
}

// One wave, one record.  State: m (log2 units), l (partial over this lane's
// tokens), acc[cb][i] = channel 16 cb + 4 g + i for query column q.
__device__ __forceinline__ void body_record(const uint8_t* __restrict__ rec, const uint4* qph, const uint4* qpl,
                                            int lane, float scale_log2, float& m_run, float& l_run, float4v* acc) {
  const int q16 = lane & 15, g = lane >> 4;
  const uint8_t* km = rec + 16384 + 16384;   // K meta: C[256] S[128] Z[128]
  const uint8_t* vm = km + 1024;             // V meta
  // ---- loads: key codes (16 x 16 B), value codes (16 x 16 B)
  uint4 kd[8][2];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    const int t = bb >> 1, hh = bb & 1;
    const int tok = 32 * (q16 >> 2) + 8 * t + 4 * hh + (q16 & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s) kd[bb][s] = *(const uint4*)(rec + tok * 128 + 64 * s + 16 * g);
  }
  uint4 vd[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) vd[cb] = *(const uint4*)(rec + 16384 + (16 * cb + q16) * 64 + 16 * g);

  // ---- S^T = K . Q~^T over 8 blocks of 16 tokens; q~ built per k-step
  float4v sc[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) sc[bb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  float a1 = 0.0f, a16 = 0.0f;
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int s = kk >> 2, e = kk & 3;
    const int base = 128 * s + 32 * g + 8 * e;
    const uint4 c = *(const uint4*)(km + 2 * base);   // C[base .. base+8)
    const uint32_t c04 = __builtin_amdgcn_perm(c.z, c.x, 0x05040100u);
    const uint32_t c15 = __builtin_amdgcn_perm(c.z, c.x, 0x07060302u);
    const uint32_t c26 = __builtin_amdgcn_perm(c.w, c.y, 0x05040100u);
    const uint32_t c37 = __builtin_amdgcn_perm(c.w, c.y, 0x07060302u);
    uint4 hi, lo;
    qtilde_pair(qph[kk].x, qpl[kk].x, c04, hi.x, lo.x);
    qtilde_pair(qph[kk].y, qpl[kk].y, c15, hi.y, lo.y);
    qtilde_pair(qph[kk].z, qpl[kk].z, c26, hi.z, lo.z);
    qtilde_pair(qph[kk].w, qpl[kk].w, c37, hi.w, lo.w);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.x), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.x), ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.y), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.y), ones, a16, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.z), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.z), ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.w), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.w), ones, a16, false);
    half8 bh, bl;
    __builtin_memcpy(&bh, &hi, 16);
    __builtin_memcpy(&bl, &lo, 16);
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const uint32_t w = e == 0 ? kd[bb][s].x : e == 1 ? kd[bb][s].y : e == 2 ? kd[bb][s].z : kd[bb][s].w;
      const half8 av = nib8_centred(w);
      sc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, sc[bb], 0, 0, 0);
      sc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, sc[bb], 0, 0, 0);
    }
  }
  a1 = xsum4(a1);
  a16 = xsum4(a16);
  const float sig_q = a1 + 16.0f * a16;    // sum of q~

  // ---- scores (log2 units): s = scale (S_i M + (Z_i + 8 S_i) sig_q)
  const uint8_t* skz = km + 512;  // S^K[128] then Z^K[128]
  uint4 sk[4], zk[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sk[t] = *(const uint4*)(skz + 2 * (32 * g + 8 * t));
    zk[t] = *(const uint4*)(skz + 256 + 2 * (32 * g + 8 * t));
  }
  float mx = -INFINITY;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    const int t = bb >> 1, hh = bb & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k8 = 4 * hh + i;  // token 32 g + 8 t + k8
      const uint32_t sw = (k8 >> 1) == 0 ? sk[t].x : (k8 >> 1) == 1 ? sk[t].y : (k8 >> 1) == 2 ? sk[t].z : sk[t].w;
      const uint32_t zw = (k8 >> 1) == 0 ? zk[t].x : (k8 >> 1) == 1 ? zk[t].y : (k8 >> 1) == 2 ? zk[t].z : zk[t].w;
      const float S = h2f((uint16_t)(sw >> (16 * (k8 & 1))));
      const float Z = h2f((uint16_t)(zw >> (16 * (k8 & 1))));
      const float v = (S * sc[bb][i] + fmaf(8.0f, S, Z) * sig_q) * scale_log2;
      sc[bb][i] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = xmax4(mx);
  const float m_new = fmaxf(m_run, mx);
  const float alpha = exp2f(m_run - m_new);
  m_run = m_new;
  if (alpha != 1.0f) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] *= alpha;
  }
  l_run *= alpha;

  // ---- P' = p S^V (operand order) and the zero-point term
  const uint8_t* svz = vm + 512;
  uint4 pb[4];
  float zt = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint4 sv = *(const uint4*)(svz + 2 * (32 * g + 8 * t));
    const uint4 zv = *(const uint4*)(svz + 256 + 2 * (32 * g + 8 * t));
    float p[8], S[8], Z[8];
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) {
      S[k8] = h2f((uint16_t)(sw[k8 >> 1] >> (16 * (k8 & 1))));
      Z[k8] = h2f((uint16_t)(zw[k8 >> 1] >> (16 * (k8 & 1))));
      p[k8] = exp2f(sc[2 * t + (k8 >> 2)][k8 & 3] - m_new);
      l_run += p[k8];
      zt = fmaf(p[k8], fmaf(8.0f, S[k8], Z[k8]), zt);
    }
    // operand order: tokens 0,4,1,5,2,6,3,7 with x1, x1, /16, /16, ...
    uint4 r;
    r.x = pack_h2(p[0] * S[0], p[4] * S[4]);
    r.y = pack_h2(p[1] * S[1] * 0.0625f, p[5] * S[5] * 0.0625f);
    r.z = pack_h2(p[2] * S[2], p[6] * S[6]);
    r.w = pack_h2(p[3] * S[3] * 0.0625f, p[7] * S[7] * 0.0625f);
    pb[t] = r;
  }
  const float corr = -xsum4(zt);

  // ---- O^T = V^T . P'^T per block of 16 channels, folded into acc with C^V
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    float4v o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w = t == 0 ? vd[cb].x : t == 1 ? vd[cb].y : t == 2 ? vd[cb].z : vd[cb].w;
      half8 bop;
      __builtin_memcpy(&bop, &pb[t], 16);
      o = __builtin_amdgcn_mfma_f32_16x16x32_f16(nib8_centred(w), bop, o, 0, 0, 0);
    }
    const uint2 cv = *(const uint2*)(vm + 2 * (16 * cb + 4 * g));
    const float c0 = h2f((uint16_t)cv.x), c1 = h2f((uint16_t)(cv.x >> 16));
    const float c2 = h2f((uint16_t)cv.y), c3 = h2f((uint16_t)(cv.y >> 16));
    acc[cb][0] = fmaf(c0, o[0] - corr, acc[cb][0]);
    acc[cb][1] = fmaf(c1, o[1] - corr, acc[cb][1]);
    acc[cb][2] = fmaf(c2, o[2] - corr, acc[cb][2]);
    acc[cb][3] = fmaf(c3, o[3] - corr, acc[cb][3]);
  }
}

__global__ __launch_bounds__(256) void decode_body_mfma_kernel(DecodeArgs a) {
  __shared__ float qrot[kMaxGroup][256];
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float4v wacc[4][16][64];   // [wave][cb][lane]: 64 KB

  const Layout& y = a.y;
  const DecodeSeq sq = a.seq[blockIdx.z];
  const int cbk = blockIdx.x;
  if (cbk >= sq.n_body_chunks) return;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4;
  const int G = a.g;

  // rotated query (fp32, LDS), rows >= G are zero
  for (int idx = tid; idx < kMaxGroup * 256; idx += 256) {
    const int i = idx >> 8, j = idx & 255;
    qrot[i][j] = i < G ? h2f(a.q[((int64_t)blockIdx.z * a.Hq + h * G + i) * 256 + j]) : 0.0f;
  }
  __syncthreads();
  // 256-point Hadamard per row, /16
  for (int st = 1; st < 256; st <<= 1) {
    for (int p = tid; p < kMaxGroup * 128; p += 256) {
      const int i = p >> 7, pp = p & 127;
      const int j = (pp / st) * 2 * st + (pp % st);
      const float u = qrot[i][j], v = qrot[i][j + st];
      qrot[i][j] = u + v;
      qrot[i][j + st] = u - v;
    }
    __syncthreads();
  }
  // this lane's rotated query values in operand order, as hi + lo fp16: the
  // butterflies above leave H q, so x1/16 gives q'; the high-nibble slots take
  // a further /16
  uint4 qph[8], qpl[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int s = kk >> 2, e = kk & 3;
    const int base = 128 * s + 32 * g + 8 * e;
    const float* qr = qrot[q16];
    const int ord[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    uint32_t h[4], l[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const float f = (pr & 1) ? 0.0625f * 0.0625f : 0.0625f;
      const float x0 = qr[base + ord[2 * pr]] * f, x1 = qr[base + ord[2 * pr + 1]] * f;
      h[pr] = pack_h2(x0, x1);
      const float h0 = h2f((uint16_t)h[pr]), h1 = h2f((uint16_t)(h[pr] >> 16));
      l[pr] = pack_h2(x0 - h0, x1 - h1);
    }
    qph[kk] = make_uint4(h[0], h[1], h[2], h[3]);
    qpl[kk] = make_uint4(l[0], l[1], l[2], l[3]);
  }

  const float scale_log2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  float4v acc[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) acc[cb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  const int r0 = cbk * a.rec_per_chunk;
  const int r1 = min(sq.n_rec, r0 + a.rec_per_chunk);
  for (int r = r0 + wave; r < r1; r += 4) {
    const uint8_t* rec = a.arena + rec_off(y, sq.slot, a.layer, h, r);
    body_record(rec, qph, qpl, lane, scale_log2, m_run, l_run, acc);
  }

  // ---- combine the four waves
  l_run = xsum4(l_run);
  if (g == 0) {
    wm[wave][q16] = m_run;
    wl[wave][q16] = l_run;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(wm[0][q16], wm[1][q16]), fmaxf(wm[2][q16], wm[3][q16]));
  const float f = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) wacc[wave][cb][lane] = acc[cb] * f;
  __syncthreads();
  // thread (wave w', lane) sums channel blocks cb = 4 w' .. 4 w' + 3 for its lane
  const int c = 1 + sq.n_ring_chunks + cbk;
  if (q16 < G) {
    float* P = a.part + (((int64_t)blockIdx.z * a.Hq + h * G + q16) * a.max_chunks + c) * (256 + 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cb = 4 * wave + k;
      const float4v s = wacc[0][cb][lane] + wacc[1][cb][lane] + wacc[2][cb][lane] + wacc[3][cb][lane];
      const int ch = 16 * cb + 4 * g;
      P[2 + ch + 0] = s[0];
      P[2 + ch + 1] = s[1];
      P[2 + ch + 2] = s[2];
      P[2 + ch + 3] = s[3];
    }
    if (wave == 0 && g == 0) {
      float L = 0.0f;
      for (int w = 0; w < 4; ++w)
        if (wm[w][q16] != -INFINITY) L += wl[w][q16] * exp2f(wm[w][q16] - M);
      P[0] = M * kLn2;
      P[1] = L;
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int grid_x, hipStream_t stream) {
  if (a.y.D != 256 || a.y.kbits != 4 || a.y.vbits != 4) return hipErrorInvalidValue;
  dim3 grid(grid_x, a.y.H, a.n_seqs);
  hipLaunchKernelGGL(decode_body_mfma_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
