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
// The non-code operand of each (q~, and the weights p S) is split into
// hi + lo fp16 halves, two products each, which keeps fp32-level precision.
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
#include "kvq_mfma.h"

namespace kvq {

// (a & m) | b in one v_and_or_b32.  The masks and the exponent pattern are
// passed in registers: a VOP3 instruction on this target cannot carry two
// literal constants, and the compiler otherwise splits it into an AND and an OR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t b) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(m), "v"(b));
  return d;
}

// Eight 4-bit codes of one dword as exact, centred fp16 values.
// One AND-OR per pair puts a nibble n into the mantissa of 1024 (the high
// nibble of a byte stays in place, i.e. 1024 + 16 n; its 1/16 is folded into
// the query operand) and one packed subtract leaves n - 8 (or 16 (n - 8)).
// Slots: [n0, n4, 16 n1, 16 n5, n2, n6, 16 n3, 16 n7] - centre.
// Centring keeps the fp32 accumulators free of a large common term: with
// codes in [0, 15] the score product carries 7.5 sum(q~), and q~ = q' C
// reaches thousands in outlier channels; the value product carries
// 7.5 sum(p S), hundreds of times the weighted average when attention is
// diffuse.  fp32 rounding of such a term swamps the result.  The centre moves
// into the zero point instead: x = C (S (n - 8) + (Z + 8 S)).
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

// ---------------------------------------------------------------------------
// Streaming kernel.  Each wave scans whole records with its own online-softmax
// state and a private LDS staging area: 32 KB for one record's codes (stored
// in the order the matrix-core operands are read back, so each 16-byte read
// of a 1 KB slice is contiguous and free of bank conflicts) and two 2 KB areas
// for scales.  Per record the wave copies the codes into registers, starts the
// direct global->LDS loads of its next record into the same area, and computes
// the current one from registers and the scale area while those loads land:
// the next record's HBM latency hides behind this record's arithmetic, with
// no workgroup barrier in the loop.  The four waves' states are combined in
// LDS at the end into one partial per query head.

constexpr int kCodeBytes = 32768;     // K and V codes of one 256-channel 4/4 record
constexpr int kMetaBytes = 2048;      // C S Z of K and V
constexpr int kWaveLds = kCodeBytes + 2 * kMetaBytes;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8*)p);
}

// one 16-byte direct global->LDS load per lane: LDS[m0 + 16 lane] <- *src.
// Issued as inline assembly so that the compiler does not add a wait for it in
// front of every later LDS read; completion is awaited explicitly (wait_vm0).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// stage record `rec` into this wave's area: 16 key slices (block bb, half s),
// 16 value slices (channel block cb), then the 2 KB of scales.
__device__ __forceinline__ void stage(const uint8_t* __restrict__ rec, uint32_t codes, uint32_t meta, int lane) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int sl = 0; sl < 16; ++sl) {
    const int bb = sl >> 1, s = sl & 1, t = bb >> 1, hh = bb & 1;
    const int tok = 32 * (m >> 2) + 8 * t + 4 * hh + (m & 3);
    dma16(rec + tok * 128 + 64 * s + 16 * g, codes + sl * 1024);
  }
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) dma16(rec + 16384 + (16 * cb + m) * 64 + 16 * g, codes + (16 + cb) * 1024);
  dma16(rec + 32768 + 16 * lane, meta);
  dma16(rec + 33792 + 16 * lane, meta + 1024);
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// One record from registers (codes) and LDS (scales).  acc[cb][i] holds
// channel 16 cb + 4 g + i for query column q = lane & 15.  The query operands
// already carry the softmax scale and log2(e): scores come out in log2 units.
// m_run is the running maximum, l_part sums this lane's tokens.
__device__ __forceinline__ void record_step(const uint4 (&kd)[8][2], const uint4 (&vd)[16], const uint8_t* km,
                                            const uint4* qph, const uint4* qpl, int lane,
                                            float& m_run, float& l_part, float4v* acc) {
  const int g = lane >> 4;
  const uint8_t* vm = km + 1024;
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  // ---- S^T = K . Q~^T, q~ built per k-step as exact hi + lo
  float4v sc[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) sc[bb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  float a1 = 0.0f, a16 = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int s = kk >> 2, e = kk & 3;
    const uint4 c = *(const uint4*)(km + 2 * (128 * s + 32 * g + 8 * e));
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
    const half8 bh = mfma_a(hi), bl = mfma_a(lo);
    half8 av[8];
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) av[bb] = nib8_centred(pick(kd[bb][s], e));
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) sc[bb] = mfma16(av[bb], bh, sc[bb]);
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) sc[bb] = mfma16(av[bb], bl, sc[bb]);
  }
  a1 = xsum4(a1);
  a16 = xsum4(a16);
  const float sig = a1 + 16.0f * a16;  // sum of q~ over the channels

  // ---- scores S_i M_i + (Z_i + 8 S_i) sigma
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint4 skv = *(const uint4*)(km + 512 + 2 * (32 * g + 8 * t));
    const uint4 zkv = *(const uint4*)(km + 768 + 2 * (32 * g + 8 * t));
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) {
      const float S = (float)as_h2(pick(skv, k8 >> 1))[k8 & 1];
      const float Z = (float)as_h2(pick(zkv, k8 >> 1))[k8 & 1];
      const int bb = 2 * t + (k8 >> 2), i = k8 & 3;
      const float v = fmaf(S, sc[bb][i], fmaf(8.0f, S, Z) * sig);
      sc[bb][i] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = xmax4(mx);
  const float m_new = fmaxf(m_run, mx);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  m_run = m_new;
  if (alpha != 1.0f) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] *= alpha;
  }
  l_part *= alpha;

  // ---- P' = p S^V in operand order, as hi + lo; zero-point term sum p (Z^V + 8 S^V)
  half8 pbh[4], pbl[4];
  float zt = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint4 sv = *(const uint4*)(vm + 512 + 2 * (32 * g + 8 * t));
    const uint4 zv = *(const uint4*)(vm + 768 + 2 * (32 * g + 8 * t));
    float x[8];
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) {
      const _Float16 S = as_h2(pick(sv, k8 >> 1))[k8 & 1];
      const _Float16 Z = as_h2(pick(zv, k8 >> 1))[k8 & 1];
      const float p = __builtin_amdgcn_exp2f(sc[2 * t + (k8 >> 2)][k8 & 3] - m_new);  // argument <= 0
      l_part += p;
      zt = fmaf(p, fmaf(8.0f, (float)S, (float)Z), zt);
      x[k8] = p * (float)S;
    }
    // slot order [0, 4, 1/16 x 1, 1/16 x 5, 2, 6, 1/16 x 3, 1/16 x 7]
    uint4 h, l;
    split_h2(x[0], x[4], h.x, l.x);
    split_h2(x[1] * 0.0625f, x[5] * 0.0625f, h.y, l.y);
    split_h2(x[2], x[6], h.z, l.z);
    split_h2(x[3] * 0.0625f, x[7] * 0.0625f, h.w, l.w);
    pbh[t] = mfma_a(h);
    pbl[t] = mfma_a(l);
  }
  const float corr = xsum4(zt);

  // ---- O^T = V^T . P'^T, four channel blocks at a time, folded into acc with C^V
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    float4v o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8 av = nib8_centred(pick(vd[4 * c4 + j], t));
        o[j] = mfma16(av, pbh[t], o[j]);
        o[j] = mfma16(av, pbl[t], o[j]);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cb = 4 * c4 + j;
      const uint2 cv = *(const uint2*)(vm + 2 * (16 * cb + 4 * g));
      const half2v c01 = as_h2(cv.x), c23 = as_h2(cv.y);
      acc[cb][0] = fmaf((float)c01[0], o[j][0] + corr, acc[cb][0]);
      acc[cb][1] = fmaf((float)c01[1], o[j][1] + corr, acc[cb][1]);
      acc[cb][2] = fmaf((float)c23[0], o[j][2] + corr, acc[cb][2]);
      acc[cb][3] = fmaf((float)c23[1], o[j][3] + corr, acc[cb][3]);
    }
  }
}

__global__ __launch_bounds__(256) void decode_body_stream_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kWaveLds];
  __shared__ float xm[4][16], xl[4][16];

  const Layout& y = a.y;
  const DecodeSeq sq = a.seq[blockIdx.z];
  const int cbk = blockIdx.x;
  if (cbk >= sq.n_body_chunks) return;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4;
  const int G = a.g;

  // ---- rotated query operands (hi, lo), prepared once per call
  uint4 qph[8], qpl[8];
  const uint4* qo = a.qops + ((int64_t)blockIdx.z * y.H + h) * kQopsPerHead;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    qph[kk] = qo[kk * 64 + lane];
    qpl[kk] = qo[(8 + kk) * 64 + lane];
  }

  // ---- this wave's records: r0 + wave, r0 + wave + 4, ...
  uint8_t* mine = lds + wave * kWaveLds;
  const uint32_t codes_lds = lds_addr(mine);
  const uint32_t meta_lds[2] = {lds_addr(mine + kCodeBytes), lds_addr(mine + kCodeBytes + kMetaBytes)};
  const int r0 = cbk * a.rec_per_chunk;
  const int r1 = min(sq.n_rec, r0 + a.rec_per_chunk);
  float m_run = -INFINITY, l_part = 0.0f;
  float4v acc[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) acc[cb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  int r = r0 + wave;
  if (r < r1) stage(a.arena + rec_off(y, sq.slot, a.layer, h, r), codes_lds, meta_lds[0], lane);
  for (int it = 0; r < r1; ++it, r += 4) {
    wait_vm0();
    uint4 kd[8][2], vd[16];
#pragma unroll
    for (int sl = 0; sl < 16; ++sl) kd[sl >> 1][sl & 1] = *(const uint4*)(mine + sl * 1024 + 16 * lane);
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) vd[cb] = *(const uint4*)(mine + (16 + cb) * 1024 + 16 * lane);
    wait_lgkm0();
    if (r + 4 < r1) stage(a.arena + rec_off(y, sq.slot, a.layer, h, r + 4), codes_lds, meta_lds[(it + 1) & 1], lane);
    record_step(kd, vd, mine + kCodeBytes + (it & 1) * kMetaBytes, qph, qpl, lane, m_run, l_part, acc);
  }

  // ---- combine the four waves (codes areas reused as scratch)
  const float lsum = xsum4(l_part);
  if (g == 0) {
    xm[wave][q16] = m_run;
    xl[wave][q16] = lsum;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16]));
  const float f = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
  float4v* wacc = (float4v*)lds;   // [wave][cb][lane]
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) wacc[(wave * 16 + cb) * 64 + lane] = acc[cb] * f;
  __syncthreads();
  if (q16 < G) {
    const int c = 1 + sq.n_ring_chunks + cbk;
    float* P = a.part + (((int64_t)blockIdx.z * a.Hq + h * G + q16) * a.max_chunks + c) * (256 + 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cb = 4 * wave + k;
      const float4v s4 = wacc[(0 * 16 + cb) * 64 + lane] + wacc[(1 * 16 + cb) * 64 + lane] +
                         wacc[(2 * 16 + cb) * 64 + lane] + wacc[(3 * 16 + cb) * 64 + lane];
      const int ch = 16 * cb + 4 * g;
      P[2 + ch + 0] = s4[0];
      P[2 + ch + 1] = s4[1];
      P[2 + ch + 2] = s4[2];
      P[2 + ch + 3] = s4[3];
    }
    if (wave == 0 && g == 0) {
      float L = 0.0f;
      for (int w = 0; w < 4; ++w)
        if (xm[w][q16] != -INFINITY) L += xl[w][q16] * exp2f(xm[w][q16] - M);
      P[0] = M * kLn2;
      P[1] = L;
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int grid_x, hipStream_t stream) {
  if (a.y.D != 256 || a.y.kbits != 4 || a.y.vbits != 4) return hipErrorInvalidValue;
  dim3 grid(grid_x, a.y.H, a.n_seqs);
  hipLaunchKernelGGL(decode_body_stream_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
