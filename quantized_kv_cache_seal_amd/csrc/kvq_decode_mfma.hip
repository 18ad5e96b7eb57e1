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
// O^T = V^T . P'^T (A = value codes, rows = channels): both A operands are
// 16-byte pieces of the record as stored (key rows, channel-major value rows).
// The weights P' pass through LDS between the two products, stored in the
// slot order of the value codes' nibbles.
//
// Work split: one workgroup (4 waves) per chunk of consecutive records of one
// KV head, the four waves sharing each record (see the kernel); one fp32
// partial (m, l, acc[D]) per chunk and query head, m in natural-log units, for
// the merge kernel.
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
// Direct global->LDS loads.
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

__device__ __forceinline__ uint32_t pick(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Cooperative kernel: the four waves of a workgroup share each record.
//   q~:      wave w forms the q~ operands of k-steps 2w, 2w+1 and shares them;
//   scores:  wave w takes token tiles 2w, 2w+1 (32 tokens) over all channels;
//   values:  wave w takes channel tiles 4w..4w+3 (64 channels) over all tokens.
// Records are staged in LDS by direct global->LDS loads into three areas, each
// refilled as soon as its last reader is done, so that every load has about
// half a record of work to land in:
//   key codes    after the scores of record r      -> record r + 1
//   value codes  after the value product of r       -> record r + 1
//   scales (x2)  after the value product of r       -> record r + 2
// Three barriers per record; per-wave state is small (16 accumulators), so
// two workgroups share a compute unit and cover each other's waits.
constexpr int kPPitch = 128 + 8;  // halves per weight row (padding spreads LDS banks)

__device__ __forceinline__ void stage_keys(const uint8_t* __restrict__ rec, uint32_t buf, int wave, int lane) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = wave + 4 * j, bb = sl >> 1, s = sl & 1;  // slice 2 bb + s: tile bb, half s
    dma16(rec + (16 * bb + m) * 128 + 64 * s + 16 * g, __builtin_amdgcn_readfirstlane(buf + sl * 1024));
  }
}
__device__ __forceinline__ void stage_values(const uint8_t* __restrict__ rec, uint32_t buf, int wave, int lane) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cb = wave + 4 * j;
    dma16(rec + 16384 + (16 * cb + m) * 64 + 16 * g, __builtin_amdgcn_readfirstlane(buf + cb * 1024));
  }
}
__device__ __forceinline__ void stage_scales(const uint8_t* __restrict__ rec, uint32_t buf, int wave, int lane) {
  if (wave < 2) dma16(rec + 32768 + wave * 1024 + 16 * lane, __builtin_amdgcn_readfirstlane(buf + wave * 1024));
}
__device__ __forceinline__ void wait_vm4() { __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8)); }

// position of token T in a weight row: the value product's k-step t of lane
// group g takes tokens 32 g + 8 t + [0, 4, 1, 5, 2, 6, 3, 7] in its 8 slots
__device__ __forceinline__ int wpos(int T) {
  const int i = T & 7;
  return (T & ~7) + (i < 4 ? 2 * i : 2 * (i - 4) + 1);
}

// q~ operands (hi, lo) of k-steps 2 wave, 2 wave + 1 from the key scales C,
// and this wave's part of sigma = sum q~
__device__ __forceinline__ void make_qtilde(const uint8_t* km, const uint4 (&qph)[2], const uint4 (&qpl)[2],
                                            uint4 (*qt)[2][64], float (*xs)[16], int wave, int lane) {
  const int g = lane >> 4;
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  float a1 = 0.0f, a16 = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kk = 2 * wave + i, s = kk >> 2, e = kk & 3;
    const uint4 c = *(const uint4*)(km + 2 * (128 * s + 32 * g + 8 * e));
    const uint32_t c04 = __builtin_amdgcn_perm(c.z, c.x, 0x05040100u);
    const uint32_t c15 = __builtin_amdgcn_perm(c.z, c.x, 0x07060302u);
    const uint32_t c26 = __builtin_amdgcn_perm(c.w, c.y, 0x05040100u);
    const uint32_t c37 = __builtin_amdgcn_perm(c.w, c.y, 0x07060302u);
    uint4 hi, lo;
    qtilde_pair(qph[i].x, qpl[i].x, c04, hi.x, lo.x);
    qtilde_pair(qph[i].y, qpl[i].y, c15, hi.y, lo.y);
    qtilde_pair(qph[i].z, qpl[i].z, c26, hi.z, lo.z);
    qtilde_pair(qph[i].w, qpl[i].w, c37, hi.w, lo.w);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.x), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.x), ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.y), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.y), ones, a16, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.z), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.z), ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.w), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.w), ones, a16, false);
    qt[kk][0][lane] = hi;
    qt[kk][1][lane] = lo;
  }
  const float part = xsum4(a1) + 16.0f * xsum4(a16);
  if (g == 0) xs[wave][lane & 15] = part;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_body_coop_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[16 * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[16 * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t mbuf[2][2048];
  __shared__ uint4 qt[8][2][64];
  __shared__ __attribute__((aligned(16))) uint16_t pw[2][16][kPPitch];  // P' hi, lo [query][token slot]
  __shared__ float xm[4][16], xz[4][16], xs[4][16];

  const Layout& y = a.y;
  const DecodeSeq sq = a.seq[blockIdx.z];
  const int cbk = blockIdx.x;
  if (cbk >= sq.n_body_chunks) return;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4;
  const int G = a.g;

  uint4 qph[2], qpl[2];  // this wave's k-steps of the prepared query
  {
    const uint4* qo = a.qops + ((int64_t)blockIdx.z * y.H + h) * kQopsPerHead;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      qph[i] = qo[(2 * wave + i) * 64 + lane];
      qpl[i] = qo[(8 + 2 * wave + i) * 64 + lane];
    }
  }
  const int r0 = cbk * a.rec_per_chunk;
  const int r1 = min(sq.n_rec, r0 + a.rec_per_chunk);
  const uint8_t* rec0 = a.arena + rec_off(y, sq.slot, a.layer, h, 0);
  const uint32_t kb_lds = lds_addr(kbuf), vb_lds = lds_addr(vbuf);
  const uint32_t mb_lds[2] = {lds_addr(mbuf[0]), lds_addr(mbuf[1])};
  float m_run = -INFINITY, l_part = 0.0f;
  float4v acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  // ---- prologue: record r0 whole, q~ of r0, scales of r0 + 1
  stage_scales(rec0 + (int64_t)r0 * y.rec_bytes, mb_lds[0], wave, lane);
  stage_keys(rec0 + (int64_t)r0 * y.rec_bytes, kb_lds, wave, lane);
  stage_values(rec0 + (int64_t)r0 * y.rec_bytes, vb_lds, wave, lane);
  wait_vm0();
  __syncthreads();
  make_qtilde(mbuf[0], qph, qpl, qt, xs, wave, lane);
  __syncthreads();
  if (r0 + 1 < r1) stage_scales(rec0 + (int64_t)(r0 + 1) * y.rec_bytes, mb_lds[1], wave, lane);

  for (int r = r0, it = 0; r < r1; ++r, ++it) {
    const uint8_t* km = mbuf[it & 1];
    const uint8_t* vm = km + 1024;
    const bool more = r + 1 < r1;

    // ---- scores of tiles 2 wave, 2 wave + 1
    uint4 kd[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s) kd[i][s] = *(const uint4*)(kbuf + (2 * (2 * wave + i) + s) * 1024 + 16 * lane);
    float4v sc[2] = {(float4v){0.0f, 0.0f, 0.0f, 0.0f}, (float4v){0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int s = kk >> 2, e = kk & 3;
      const half8 bh = mfma_a(qt[kk][0][lane]), bl = mfma_a(qt[kk][1][lane]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const half8 av = nib8_centred(pick(kd[i][s], e));
        sc[i] = mfma16(av, bh, sc[i]);
        sc[i] = mfma16(av, bl, sc[i]);
      }
    }
    const float sig = xs[0][q16] + xs[1][q16] + xs[2][q16] + xs[3][q16];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int T = 16 * (2 * wave + i) + 4 * g;  // tokens T .. T + 3 of this lane
      const uint2 sk = *(const uint2*)(km + 512 + 2 * T);
      const uint2 zk = *(const uint2*)(km + 768 + 2 * T);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float S = (float)as_h2(j < 2 ? sk.x : sk.y)[j & 1];
        const float Z = (float)as_h2(j < 2 ? zk.x : zk.y)[j & 1];
        const float v = fmaf(S, sc[i][j], fmaf(8.0f, S, Z) * sig);
        sc[i][j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = xmax4(mx);
    if (g == 0) xm[wave][q16] = mx;
    __syncthreads();  // (B2) record maxima; key codes and q~ are free
    if (more) stage_keys(rec0 + (int64_t)(r + 1) * y.rec_bytes, kb_lds, wave, lane);

    const float mrec = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16]));
    const float m_new = fmaxf(m_run, mrec);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first record
    m_run = m_new;
    if (alpha != 1.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    }
    l_part *= alpha;
    float zt = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int T = 16 * (2 * wave + i) + 4 * g;
      const uint2 sv = *(const uint2*)(vm + 512 + 2 * T);
      const uint2 zv = *(const uint2*)(vm + 768 + 2 * T);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float S = (float)as_h2(j < 2 ? sv.x : sv.y)[j & 1];
        const float Z = (float)as_h2(j < 2 ? zv.x : zv.y)[j & 1];
        const float p = __builtin_amdgcn_exp2f(sc[i][j] - m_new);  // argument <= 0
        l_part += p;
        zt = fmaf(p, fmaf(8.0f, S, Z), zt);
        const int Tj = T + j;
        float x = p * S;
        if (Tj & 1) x *= 0.0625f;  // slots of high nibbles carry 1/16
        const uint16_t xh = f2h_bits(x);
        const uint16_t xl = f2h_bits(x - h2f(xh));
        const int pos = wpos(Tj);
        pw[0][q16][pos] = xh;
        pw[1][q16][pos] = xl;
      }
    }
    zt = xsum4(zt);
    if (g == 0) xz[wave][q16] = zt;
    if (more)
      wait_vm4();  // value codes of r and scales of r + 1 in; the 4 key loads of r + 1 may fly
    else
      wait_vm0();
    __syncthreads();  // (B3) weights, zero-point sums, value codes of r, scales of r + 1
    if (more) make_qtilde(mbuf[(it + 1) & 1], qph, qpl, qt, xs, wave, lane);

    const float corr = xz[0][q16] + xz[1][q16] + xz[2][q16] + xz[3][q16];
    half8 pbh[4], pbl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pbh[t] = mfma_a(*(const uint4*)&pw[0][q16][32 * g + 8 * t]);
      pbl[t] = mfma_a(*(const uint4*)&pw[1][q16][32 * g + 8 * t]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cb = 4 * wave + j;
      const uint4 vd = *(const uint4*)(vbuf + cb * 1024 + 16 * lane);
      float4v o = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half8 av = nib8_centred(pick(vd, t));
        o = mfma16(av, pbh[t], o);
        o = mfma16(av, pbl[t], o);
      }
      const uint2 cv = *(const uint2*)(vm + 2 * (16 * cb + 4 * g));
      const half2v c01 = as_h2(cv.x), c23 = as_h2(cv.y);
      acc[j][0] = fmaf((float)c01[0], o[0] + corr, acc[j][0]);
      acc[j][1] = fmaf((float)c01[1], o[1] + corr, acc[j][1]);
      acc[j][2] = fmaf((float)c23[0], o[2] + corr, acc[j][2]);
      acc[j][3] = fmaf((float)c23[1], o[3] + corr, acc[j][3]);
    }
    wait_vm0();       // key codes of r + 1
    __syncthreads();  // (B1) record r done everywhere; key codes and q~ of r + 1 in
    if (more) stage_values(rec0 + (int64_t)(r + 1) * y.rec_bytes, vb_lds, wave, lane);
    if (r + 2 < r1) stage_scales(rec0 + (int64_t)(r + 2) * y.rec_bytes, mb_lds[it & 1], wave, lane);
  }

  // ---- partial of this chunk: every wave holds the same m; l sums over waves
  const float lsum = xsum4(l_part);
  if (g == 0) xm[wave][q16] = lsum;
  __syncthreads();
  if (q16 < G) {
    const int c = 1 + sq.n_ring_chunks + cbk;
    float* P = a.part + (((int64_t)blockIdx.z * a.Hq + h * G + q16) * a.max_chunks + c) * (256 + 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = 16 * (4 * wave + j) + 4 * g;
      P[2 + ch + 0] = acc[j][0];
      P[2 + ch + 1] = acc[j][1];
      P[2 + ch + 2] = acc[j][2];
      P[2 + ch + 3] = acc[j][3];
    }
    if (wave == 0 && g == 0) {
      P[0] = m_run * kLn2;
      P[1] = xm[0][q16] + xm[1][q16] + xm[2][q16] + xm[3][q16];
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int grid_x, hipStream_t stream) {
  if (a.y.D != 256 || a.y.kbits != 4 || a.y.vbits != 4) return hipErrorInvalidValue;
  dim3 grid(grid_x, a.y.H, a.n_seqs);
  hipLaunchKernelGGL(decode_body_coop_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
