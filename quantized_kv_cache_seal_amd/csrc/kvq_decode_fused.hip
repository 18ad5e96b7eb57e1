// Matrix-core decode attention: the sealed body (256-channel 4-bit records),
// the fp16 sink and the tq6_0 staging ring in one launch.
//
// SJ-KVaRN 2.1: one decode pass reads the sink, the staging ring (the exact
// tail) and the sealed body; KV Cache Precision Tail section 2: the region
// results are combined under one softmax (here: split-K partials (m, l, acc)
// merged by the merge kernel).  KV cache math ("rotate first"): the query is
// rotated once, ring and body are read in the rotated domain with no
// dequantise pass, and only the merged output is rotated back; the sink stays
// in the original domain and is scored with the unrotated query.
//
// Body record math (SJ-KVaRN 2.2: column balance scales C absorbed, per-row
// scale S and zero point Z): k_ij = C_j (S_i n_ij + Z_i), so for the rotated
// query q' and q~_j = q'_j C_j, sigma = sum_j q~_j:
//     q'.k_i = S_i (q~ . n_i) + Z_i sigma
//     sum_i p_i v_ij = C_j ( sum_i (p_i S_i) n_ij + sum_i p_i Z_i ).
// Ring math (tq6_0: one fp16 scale d per 128-value block, 6-bit codes u):
//     score_t = sum_blocks d_t,b (q' . u_t,b),   out_j = sum_t (p_t d_t,b(j)) u_t,j.
// Every inner product is dense (16 query columns, the group padded to 16) x
// (32 codes) x (16 tokens or channels) on v_mfma_f32_16x16x32_f16, codes
// entering as exact small integers; the non-code operand (q~, q', the weights)
// is split into hi + lo fp16 halves, two products each, which keeps fp32-level
// precision.  The softmax scale and log2(e) are folded into the query, so
// scores come out in log2 units.
//
// Work items, one workgroup (4 waves) each: body chunks (consecutive records
// of one KV head) first, then the sink and ring chunks of every KV head.
// Each item writes one fp32 partial per query head; partial 0 is the sink,
// 1.. the ring chunks, then the body chunks.
#include <type_traits>

#include "kvq_encode.h"
#include "kvq_mfma.h"

namespace kvq {

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

// Eight 4-bit codes of one dword as exact, centred fp16 values.  One AND-OR
// per pair puts a nibble n into the mantissa of 1024 (the high nibble of a
// byte stays in place, i.e. 1024 + 16 n; its 1/16 is folded into the other
// operand) and one packed subtract leaves n - 8 (or 16 (n - 8)).
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

__device__ __forceinline__ uint32_t pick(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
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
// Query rows: the G query heads of KV head h, times scale * log2(e), rotated
// (R = H/16 for head_dim 256, s2 . H . s1 / sqrt(128) for 128) or not, into
// rows[16][D] of LDS (rows G..15 zero).  Wave w transforms rows w, w + 4, ...
// in registers.  query_load issues the loads (first, ahead of the bulk loads
// of an item, so that waiting for the query does not wait for them);
// query_rows transforms and stores.  The caller synchronises before reading.
template <int D>
struct QueryRaw {
  static constexpr int VPL = D / 64, NR = kMaxGroup / 4;  // values per lane, rows per wave
  static_assert(VPL % 2 == 0, "two fp16 per load");
  uint32_t w[NR][VPL / 2];
};

template <int D>
__device__ __forceinline__ void query_load(const DecodeArgs& a, int b, int h, int wave, int lane, QueryRaw<D>& raw) {
  constexpr int VPL = QueryRaw<D>::VPL, NR = QueryRaw<D>::NR;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int i = wave + 4 * k;
    const int ii = i < a.g ? i : 0;  // rows past the group read row 0 and are zeroed below
    const uint32_t* src = (const uint32_t*)(a.q + ((int64_t)b * a.Hq + h * a.g + ii) * D + VPL * lane);
#pragma unroll
    for (int w = 0; w < VPL / 2; ++w) raw.w[k][w] = src[w];
  }
}

template <int D>
__device__ __forceinline__ void query_rows(const DecodeArgs& a, const QueryRaw<D>& raw, bool rotate, float* rows,
                                           int wave, int lane) {
  constexpr int VPL = QueryRaw<D>::VPL, NR = QueryRaw<D>::NR;
  const float sl = a.scale * kLog2e;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int i = wave + 4 * k;
    const bool live = i < a.g;
    float v[VPL];
#pragma unroll
    for (int w = 0; w < VPL / 2; ++w) {
      const half2v x = as_h2(raw.w[k][w]);
      v[2 * w] = live ? (float)x[0] * sl : 0.0f;
      v[2 * w + 1] = live ? (float)x[1] * sl : 0.0f;
    }
    if (rotate) {
      if (D == 128) {
#pragma unroll
        for (int j = 0; j < VPL; ++j)
          if (sign_neg(a.signs, VPL * lane + j)) v[j] = -v[j];
      }
      wave_fwht<VPL, D>(v, lane);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        if (D == 128) {
          v[j] *= (float)kInvSqrt128;
          if (sign_neg(a.signs, 128 + VPL * lane + j)) v[j] = -v[j];
        } else {
          v[j] *= 0.0625f;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) rows[i * D + VPL * lane + j] = v[j];
  }
}

// ---------------------------------------------------------------------------
// Body role: one chunk of records of one KV head.
//   q~:      wave w forms the q~ operands of k-steps 2w, 2w+1 (live rows) and shares them;
//   scores:  wave w takes token tiles 2w, 2w+1 (32 tokens) over all channels;
//   values:  wave w takes channel tiles 4w..4w+3 (64 channels) over all tokens.
// Key and value codes go from memory straight into the registers of the lane
// that feeds them to the matrix cores (16 bytes per lane and operand), each
// set reloaded as soon as its product is done, so that it has the other half
// of a record's work to land in.  The 2 KB of scales pass through a ring of
// three LDS areas, loaded two records ahead.  Two barriers per record:
//   (B2) after the scores: record maxima exchanged;
//   (B3) after the weights: P', the zero-point sums, q~ and scales of the next
//        record exchanged.
// Token rows are assigned so that the four score rows of a lane are four
// consecutive slots of the value product's operand order (one 8-byte store of
// the weights per tile): position P of a tile holds token
// (P & ~7) + [0, 4, 1, 5, 2, 6, 3, 7][P & 7].
constexpr int kPPitch = 128 + 8;  // halves per weight row (padding spreads LDS banks)
constexpr int kBodyQt = 0, kBodyPw = 16384, kBodyM = kBodyPw + 2 * 16 * kPPitch * 2, kBodyX = kBodyM + 3 * 2048;
constexpr int kBodyLds = kBodyX + 3 * 256;
static_assert(16 * 256 * 4 == 8 * 2 * 64 * 16, "query rows must fit the q~ area");

constexpr int kWOld = 14, kWYoung = 10;  // record shares of the first and second workgroup of a compute unit

__device__ __forceinline__ int slot_token(int p) {  // token at position p (0..7) of an 8-token group
  return (p >> 1) + 4 * (p & 1);
}

// q~ operands (hi, lo) of k-steps 2 wave, 2 wave + 1 from the key scales C,
// for the live query rows only: lane (i, g, kk) = (lane & 7, (lane >> 3) & 3,
// 2 wave + (lane >> 5)) forms the 8 slots of row i (and i + 8 when the group has
// more than 8 heads) that lane group g of k-step kk feeds to the matrix core;
// rows past 8 (or 16) are never written and stay zero.  Also this wave's part
// of sigma = sum q~ per row.
__device__ __forceinline__ void make_qtilde(const uint8_t* km, const uint4 (&qph)[2], const uint4 (&qpl)[2],
                                            uint4 (*qt)[2][64], float (*xs)[16], int G, int wave, int lane) {
  const int i = lane & 7, g = (lane >> 3) & 3, kk = 2 * wave + (lane >> 5);
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  const uint4 c = *(const uint4*)(km + 2 * (128 * (kk >> 2) + 32 * g + 8 * (kk & 3)));
  const uint32_t c04 = __builtin_amdgcn_perm(c.z, c.x, 0x05040100u);
  const uint32_t c15 = __builtin_amdgcn_perm(c.z, c.x, 0x07060302u);
  const uint32_t c26 = __builtin_amdgcn_perm(c.w, c.y, 0x05040100u);
  const uint32_t c37 = __builtin_amdgcn_perm(c.w, c.y, 0x07060302u);
  const int np = G > 8 ? 2 : 1;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p >= np) break;
    uint4 hi, lo;
    qtilde_pair(qph[p].x, qpl[p].x, c04, hi.x, lo.x);
    qtilde_pair(qph[p].y, qpl[p].y, c15, hi.y, lo.y);
    qtilde_pair(qph[p].z, qpl[p].z, c26, hi.z, lo.z);
    qtilde_pair(qph[p].w, qpl[p].w, c37, hi.w, lo.w);
    float a1 = 0.0f, a16 = 0.0f;
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.x), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.x), ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.y), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.y), ones, a16, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.z), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.z), ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.w), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.w), ones, a16, false);
    qt[kk][0][16 * g + i + 8 * p] = hi;
    qt[kk][1][16 * g + i + 8 * p] = lo;
    float part = fmaf(16.0f, a16, a1);
    part += __shfl_xor(part, 8, 64);
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if ((lane >> 3) == 0) xs[wave][i + 8 * p] = part;
  }
}

// dummy: every lane reads the first 16 bytes of `rec` (one line, result unused)
__device__ __forceinline__ void load_keys(const uint8_t* __restrict__ rec, uint4 (&kd)[2][2], int wave, int lane,
                                          bool dummy = false) {
  const int m = lane & 15, g = lane >> 4;
  const int row = (m & 8) + slot_token(m & 7);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      kd[i][s] = *(const uint4*)(rec + (dummy ? 0 : (16 * (2 * wave + i) + row) * 128 + 64 * s + 16 * g));
}
__device__ __forceinline__ void load_values(const uint8_t* __restrict__ rec, uint4 (&vd)[4], int wave, int lane,
                                            bool dummy = false) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) vd[j] = *(const uint4*)(rec + (dummy ? 0 : 16384 + (16 * (4 * wave + j) + m) * 64 + 16 * g));
}

__device__ __forceinline__ void body_role(const DecodeArgs& a, int b, int h, int cbk, uint8_t* smem) {
  const Layout& y = a.y;
  const DecodeSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4;
  const int G = a.g;
  uint4(*qt)[2][64] = (uint4(*)[2][64])(smem + kBodyQt);
  uint16_t(*pw)[16][kPPitch] = (uint16_t(*)[16][kPPitch])(smem + kBodyPw);
  uint8_t* mbuf = smem + kBodyM;  // [3][2048] scales of records r, r + 1, r + 2 (mod 3)
  float(*xm)[16] = (float(*)[16])(smem + kBodyX);
  float(*xz)[16] = (float(*)[16])(smem + kBodyX + 256);
  float(*xs)[16] = (float(*)[16])(smem + kBodyX + 512);

  // Partition of the sequence's records over its chunks.  The first workgroup
  // to land on a compute unit (grid index below n_old) wins the issue
  // arbitration against the second and scans a record ~1.4 times as fast
  // (measured), so it takes kWOld records for every kWYoung of the second,
  // and both end together; with few records per chunk the split is even.
  const int nb = sq.n_body_chunks;
  int r0, r1;
  if (sq.n_rec >= 4 * nb) {
    // chunk c of this pair sits at grid index g_base + c H + h (heads interleaved)
    const int g_base = (int)blockIdx.x - cbk * y.H - h;
    const int n_first = max(0, (a.n_old - g_base - h + y.H - 1) / y.H);  // chunks with g < n_old
    auto wpref = [&](int c) -> int64_t {
      return (int64_t)kWYoung * c + (int64_t)(kWOld - kWYoung) * min(n_first, c);
    };
    const int64_t W = wpref(nb);
    r0 = (int)(wpref(cbk) * sq.n_rec / W);
    r1 = (int)(wpref(cbk + 1) * sq.n_rec / W);
  } else {
    r0 = (int)((int64_t)cbk * sq.n_rec / nb);
    r1 = (int)((int64_t)(cbk + 1) * sq.n_rec / nb);
  }
  const uint8_t* rec0 = a.arena + rec_off(y, sq.slot, a.layer, h, 0);
  auto rec = [&](int r) { return rec0 + (int64_t)r * y.rec_bytes; };
  auto mslot = [&](int r) { return mbuf + ((r - r0) % 3) * 2048; };

  // ---- prologue: the query first, then the scales of r0, r0 + 1 and the key
  // and value codes of r0 in flight while the query is rotated (its rows
  // borrow the q~ area, 16 x 256 floats)
  QueryRaw<256> qraw;
  query_load<256>(a, b, h, wave, lane, qraw);
  uint2 m0 = *(const uint2*)(rec(r0) + 32768 + 8 * tid);
  uint2 m1 = *(const uint2*)(r0 + 1 < r1 ? rec(r0 + 1) + 32768 + 8 * tid : rec0);
  uint4 kd[2][2], vd[4];
  load_keys(rec(r0), kd, wave, lane);
  load_values(rec(r0), vd, wave, lane);
  float* rows = (float*)qt;
  query_rows<256>(a, qraw, true, rows, wave, lane);
  __syncthreads();
  uint4 qph[2], qpl[2];  // q' of this lane's q~ slots (make_qtilde), rows i and i + 8
  {
    const int ui = lane & 7, ug = (lane >> 3) & 3, ukk = 2 * wave + (lane >> 5);
    const int base = 128 * (ukk >> 2) + 32 * ug + 8 * (ukk & 3);  // channels of the key dword of lane group ug
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float* row = rows + (ui + 8 * p) * 256 + base;  // rows past the group are zero
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const float f = (pr & 1) ? 0.0625f : 1.0f;  // pairs read from high nibbles carry 1/16
        split_h2(row[pr] * f, row[pr + 4] * f, hb[pr], lb[pr]);
      }
      qph[p] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
      qpl[p] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
    }
  }
  __syncthreads();  // the query rows are read: the q~ area is cleared (rows make_qtilde skips stay zero)
#pragma unroll
  for (int j = 0; j < 4; ++j) ((uint4*)qt)[tid + 256 * j] = make_uint4(0, 0, 0, 0);
  if (tid < 64) (&xs[0][0])[tid] = 0.0f;
  *(uint2*)(mslot(r0) + 8 * tid) = m0;
  if (r0 + 1 < r1) *(uint2*)(mslot(r0 + 1) + 8 * tid) = m1;
  __syncthreads();
  make_qtilde(mslot(r0), qph, qpl, qt, xs, G, wave, lane);
  uint2 mnext = *(const uint2*)(r0 + 2 < r1 ? rec(r0 + 2) + 32768 + 8 * tid : rec0);
  __syncthreads();

  float m_run = -INFINITY, l_part = 0.0f;
  float4v acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  for (int r = r0; r < r1; ++r) {
    const uint8_t* km = mslot(r);
    const uint8_t* vm = km + 1024;
    const bool more = r + 1 < r1;

    // ---- scores of tiles 2 wave, 2 wave + 1: four independent accumulation
    // chains (tile x hi/lo) keep the matrix core busy between dependent products
    float4v sh[2], sl[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) sh[i] = sl[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
    // q~ operands read from LDS two k-steps ahead of their products
    half8 qb[8][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      qb[kk][0] = mfma_a(qt[kk][0][lane]);
      qb[kk][1] = mfma_a(qt[kk][1][lane]);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int s = kk >> 2, e = kk & 3;
      if (kk + 2 < 8) {
        qb[kk + 2][0] = mfma_a(qt[kk + 2][0][lane]);
        qb[kk + 2][1] = mfma_a(qt[kk + 2][1][lane]);
      }
      const half8 bh = qb[kk][0], bl = qb[kk][1];
      half8 av[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = nib8_centred(pick(kd[i][s], e));
#pragma unroll
      for (int i = 0; i < 2; ++i) sh[i] = mfma16(av[i], bh, sh[i]);
#pragma unroll
      for (int i = 0; i < 2; ++i) sl[i] = mfma16(av[i], bl, sl[i]);
    }
    float4v sc[2] = {sh[0] + sl[0], sh[1] + sl[1]};
    const float sig = xs[0][q16] + xs[1][q16] + xs[2][q16] + xs[3][q16];
    // this lane's rows are positions 16 bb + 4 g + j: tokens base + {0,4,1,5}
    // (g even) or base + {2,6,3,7} (g odd), base = 16 bb + 8 (g / 2)
    const int tb = 8 * (g >> 1) + 2 * (g & 1);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int T = 16 * (2 * wave + i) + tb;
      const uint32_t s01 = *(const uint32_t*)(km + 512 + 2 * T), s45 = *(const uint32_t*)(km + 512 + 2 * T + 8);
      const uint32_t z01 = *(const uint32_t*)(km + 768 + 2 * T), z45 = *(const uint32_t*)(km + 768 + 2 * T + 8);
      const half2v S0 = as_h2(s01), S1 = as_h2(s45), Z0 = as_h2(z01), Z1 = as_h2(z45);
      const float Sj[4] = {(float)S0[0], (float)S1[0], (float)S0[1], (float)S1[1]};
      const float Zj[4] = {(float)Z0[0], (float)Z1[0], (float)Z0[1], (float)Z1[1]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = fmaf(Sj[j], sc[i][j], fmaf(8.0f, Sj[j], Zj[j]) * sig);
        sc[i][j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = xmax4(mx);
    if (g == 0) xm[wave][q16] = mx;
    __syncthreads();  // (B2) record maxima; q~ of r and the key codes are free
    // loads are unconditional (a branch around them makes the compiler's wait
    // counting conservative): past the last record they re-read one 16-byte
    // line of record r0 and are not used
    load_keys(more ? rec(r + 1) : rec0, kd, wave, lane, !more);

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
      const int T = 16 * (2 * wave + i) + tb;
      const uint32_t s01 = *(const uint32_t*)(vm + 512 + 2 * T), s45 = *(const uint32_t*)(vm + 512 + 2 * T + 8);
      const uint32_t z01 = *(const uint32_t*)(vm + 768 + 2 * T), z45 = *(const uint32_t*)(vm + 768 + 2 * T + 8);
      const half2v S0 = as_h2(s01), S1 = as_h2(s45), Z0 = as_h2(z01), Z1 = as_h2(z45);
      const float Sj[4] = {(float)S0[0], (float)S1[0], (float)S0[1], (float)S1[1]};
      const float Zj[4] = {(float)Z0[0], (float)Z1[0], (float)Z0[1], (float)Z1[1]};
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[i][j] - m_new);  // argument <= 0
        l_part += p;
        zt = fmaf(p, fmaf(8.0f, Sj[j], Zj[j]), zt);
        x[j] = p * Sj[j];
      }
      x[2] *= 0.0625f;  // odd tokens sit in the high nibbles: their slots carry 1/16
      x[3] *= 0.0625f;
      uint2 hi, lo;
      split_h2(x[0], x[1], hi.x, lo.x);
      split_h2(x[2], x[3], hi.y, lo.y);
      *(uint2*)&pw[0][q16][16 * (2 * wave + i) + 4 * g] = hi;
      *(uint2*)&pw[1][q16][16 * (2 * wave + i) + 4 * g] = lo;
    }
    zt = xsum4(zt);
    if (g == 0) xz[wave][q16] = zt;
    if (more) make_qtilde(mslot(r + 1), qph, qpl, qt, xs, G, wave, lane);
    if (r + 2 < r1) *(uint2*)(mslot(r + 2) + 8 * tid) = mnext;
    mnext = *(const uint2*)(r + 3 < r1 ? rec(r + 3) + 32768 + 8 * tid : rec0);
    __syncthreads();  // (B3) weights, zero-point sums; q~ and scales of r + 1, r + 2

    const float corr = xz[0][q16] + xz[1][q16] + xz[2][q16] + xz[3][q16];
    half8 pbh[4], pbl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pbh[t] = mfma_a(*(const uint4*)&pw[0][q16][32 * g + 8 * t]);
      pbl[t] = mfma_a(*(const uint4*)&pw[1][q16][32 * g + 8 * t]);
    }
    float4v o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // four channel tiles as independent chains
      half8 av[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = nib8_centred(pick(vd[j], t));
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = mfma16(av[j], pbh[t], o[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = mfma16(av[j], pbl[t], o[j]);
    }
    load_values(more ? rec(r + 1) : rec0, vd, wave, lane, !more);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cb = 4 * wave + j;
      const uint2 cv = *(const uint2*)(vm + 2 * (16 * cb + 4 * g));
      const half2v c01 = as_h2(cv.x), c23 = as_h2(cv.y);
      acc[j][0] = fmaf((float)c01[0], o[j][0] + corr, acc[j][0]);
      acc[j][1] = fmaf((float)c01[1], o[j][1] + corr, acc[j][1]);
      acc[j][2] = fmaf((float)c23[0], o[j][2] + corr, acc[j][2]);
      acc[j][3] = fmaf((float)c23[1], o[j][3] + corr, acc[j][3]);
    }
  }

  // ---- partial of this chunk: every wave holds the same m; l sums over waves
  const float lsum = xsum4(l_part);
  if (g == 0) xm[wave][q16] = lsum;
  __syncthreads();
  if (q16 < G) {
    const int c = 1 + sq.n_ring_chunks + cbk;
    float* P = a.part + (((int64_t)b * a.Hq + h * G + q16) * a.max_chunks + c) * (256 + 2);
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

// ---------------------------------------------------------------------------
// Sink / ring role: chunk c of one KV head, c = 0 the sink (n_sink fp16 tokens,
// original domain), c >= 1 ring tokens [(c - 1) ring_chunk, c ring_chunk).
// The chunk is scanned in steps of 64 tokens with an online softmax:
//   (1) value codes (ring: 6-bit codes decoded; sink: fp16 rows) are written
//       transposed into an fp16 tile V^T in LDS;
//   (2) scores: wave w takes the 16-token tile w over all channels, its key
//       operands read straight from memory;
//   (3) weights p (times d^V per block for the ring) as hi + lo into LDS;
//   (4) values: wave w takes channel tiles D/64 w .. over the 64 tokens,
//       accumulating straight into its running sums.
// Ring steps read memory into registers one step ahead.
constexpr int kStep = 64;           // tokens per step
constexpr int kRPitch = kStep + 8;  // halves per V^T / weight row

template <int D>
struct RingLds {
  static constexpr int NB = D / kQBlock;
  static constexpr int VT = 0, PW = VT + D * kRPitch * 2, QO = PW + NB * 2 * 16 * kRPitch * 2;
  static constexpr int X = QO + (D / 32) * 2 * 64 * 16;
  static constexpr int total = X + 2 * 256;
  static_assert(16 * D * 4 <= D * kRPitch * 2, "query rows must fit the V^T area");
};

// Eight 6-bit codes held as 48 bits (lo, low 16 bits of hi), as fp16 u - 32.
__device__ __forceinline__ half8 codes6_reg(uint32_t lo, uint32_t hi) {
  uint4 u;
  u.x = (lo & 63u) | ((lo << 10) & 0x3F0000u) | 0x64006400u;
  u.y = ((lo >> 12) & 63u) | ((lo >> 2) & 0x3F0000u) | 0x64006400u;
  u.z = ((lo >> 24) & 63u) | ((((lo >> 30) | (hi << 2)) & 63u) << 16) | 0x64006400u;
  u.w = ((hi >> 4) & 63u) | ((hi << 6) & 0x3F0000u) | 0x64006400u;
  const half8 off1056 = {(_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f,
                         (_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f, (_Float16)1056.0f};
  return mfma_a(u) - off1056;
}

// Registers of one ring step for this thread:
//   k[kk]  the two aligned dwords holding the 8 key codes of its A operand
//          (token 16 wave + (lane & 15), channels 32 kk + 8 g ..);
//   dk/dv  the block scales of its 4 output tokens 16 wave + 4 g + r;
//   v      value codes of tokens 4 tq .. 4 tq + 3, channels 16 c16 .. + 15
//          (12 bytes each), tq = tid & 15, c16 = tid >> 4.
template <int D>
struct RingRegs {
  static constexpr int NB = D / kQBlock, KK = D / 32;
  uint2 k[KK];
  uint32_t dk[4], dv[4];
  uint32_t v[4][3];
};

template <int D>
__device__ __forceinline__ void ring_load(const DecodeArgs& a, const DecodeSeq& sq, int h, int t0, int n,
                                          RingRegs<D>& R) {
  constexpr int NB = D / kQBlock, KK = D / 32;
  const Layout& y = a.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  int slot0 = (sq.ring0 + t0) % y.cap;
  auto slot_of = [&](int t) { const int s = slot0 + t; return s >= y.cap ? s - y.cap : s; };
  const uint8_t* kc = a.arena + rcode_off(y, sq.slot, a.layer, h, 0, 0);
  const uint8_t* vc = a.arena + rcode_off(y, sq.slot, a.layer, h, 1, 0);
  const uint8_t* ks = a.arena + rscale_off(y, sq.slot, a.layer, h, 0, 0);
  const uint8_t* vs = a.arena + rscale_off(y, sq.slot, a.layer, h, 1, 0);
  {
    const int t = 16 * wave + m;
    const uint8_t* row = kc + (int64_t)slot_of(t < n ? t : 0) * (NB * kQBytes) + ((6 * g) & ~3);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint32_t* p = (const uint32_t*)(row + 24 * kk);
      R.k[kk] = make_uint2(p[0], p[1]);
    }
  }
  // every load is unconditional (clamped indices, results selected
  // afterwards): loads under branches make the compiler's wait counting
  // conservative across the step loop, which would stall on the prefetch
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wave + 4 * g + r;
    const int sl = slot_of(t < n ? t : 0);
    uint32_t dk, dv;
    if (NB == 2) {
      dk = *(const uint32_t*)(ks + (int64_t)sl * 4);
      dv = *(const uint32_t*)(vs + (int64_t)sl * 4);
    } else {
      dk = *(const uint16_t*)(ks + (int64_t)sl * 2);
      dv = *(const uint16_t*)(vs + (int64_t)sl * 2);
    }
    R.dk[r] = dk;  // a masked token carries the (finite) scales of token 0; its weight is 0
    R.dv[r] = dv;
  }
  const int tq = tid & 15, c16 = (tid >> 4) % (D / 16);  // head_dim 128: two threads per item, one used
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 4 * tq + k;
    const uint32_t* p = (const uint32_t*)(vc + (int64_t)slot_of(t < n ? t : 0) * (NB * kQBytes) + 12 * c16);
    R.v[k][0] = p[0];
    R.v[k][1] = p[1];
    R.v[k][2] = p[2];
  }
}

template <int D>
__device__ __forceinline__ void ring_role(const DecodeArgs& a, int b, int h, int c, uint8_t* smem) {
  using Ly = RingLds<D>;
  constexpr int NB = Ly::NB, KK = D / 32, CPW = D / 64;
  const Layout& y = a.y;
  const DecodeSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4, G = a.g;
  uint16_t* vt = (uint16_t*)(smem + Ly::VT);
  uint16_t* pw = (uint16_t*)(smem + Ly::PW);  // weights [NB][hi, lo][16][kRPitch]
  uint4(*qo)[2][64] = (uint4(*)[2][64])(smem + Ly::QO);  // query operands [kk][hi, lo][lane]
  float(*xm)[16] = (float(*)[16])(smem + Ly::X);
  float(*xl)[16] = (float(*)[16])(smem + Ly::X + 256);

  const bool sink = c == 0;
  const int t_begin = sink ? 0 : (c - 1) * a.ring_chunk;
  const int t_end = sink ? sq.n_sink : min(sq.ring_len, c * a.ring_chunk);

  QueryRaw<D> qraw;
  query_load<D>(a, b, h, wave, lane, qraw);
  RingRegs<D> ra, rb;
  if (!sink) ring_load<D>(a, sq, h, t_begin, t_end - t_begin, ra);

  // ---- query operands in natural channel order, rotated (ring) or not (sink),
  // kept in LDS: wave w forms k-steps w, w + 4, ...
  {
    float* rows = (float*)vt;
    query_rows<D>(a, qraw, !sink, rows, wave, lane);
    __syncthreads();
    for (int kk = wave; kk < KK; kk += 4) {
      const float* r = rows + q16 * D + 32 * kk + 8 * g;
      uint32_t hh[4], ll[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) split_h2(r[2 * pr], r[2 * pr + 1], hh[pr], ll[pr]);
      qo[kk][0][lane] = make_uint4(hh[0], hh[1], hh[2], hh[3]);
      qo[kk][1][lane] = make_uint4(ll[0], ll[1], ll[2], ll[3]);
    }
    __syncthreads();
  }
  const uint16_t* ksink = (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, sq.slot, a.layer, h, 0, 0);
  const uint16_t* vsink = (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, sq.slot, a.layer, h, 1, 0);

  float m_run = -INFINITY, l_part = 0.0f;
  float4v acc[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) acc[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  // one step over tokens t0 .. t0 + 63; the ring step reads `cur` and loads the
  // next step into `nxt` (unconditionally: past the end the clamped loads are
  // harmless), the two register sets alternating so that no copy, and no early
  // wait for the loads in flight, is needed.  The sink and ring steps are
  // compiled separately (no branch around the loads inside a step).
  auto step = [&](auto sink_c, int t0, const RingRegs<D>& cur, RingRegs<D>& nxt) {
    constexpr bool sink = decltype(sink_c)::value;
    const int n = min(kStep, t_end - t0);
    if (!sink) ring_load<D>(a, sq, h, t0 + kStep, t_end - t0 - kStep, nxt);

    // ---- (1) V^T; the sink's key operands are loaded here too, all at once
    uint4 ks_op[KK];
    if (sink) {
      constexpr int ITEMS = (kStep / 4) * (D / 8) / 256;  // 4-token x 8-channel pieces per thread
      uint4 r[ITEMS][4];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        ks_op[kk] = *(const uint4*)(ksink + (int64_t)(t0 + 16 * wave + q16) * D + 32 * kk + 8 * g);
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const int it = tid + 256 * j, tq = it % (kStep / 4), c8 = it / (kStep / 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tok = 4 * tq + k;
          r[j][k] = *(const uint4*)(vsink + (int64_t)(t0 + (tok < n ? tok : 0)) * D + 8 * c8);
        }
      }
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {  // zero the rows past the sink only once everything is in flight
        const int it = tid + 256 * j;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * (it % (kStep / 4)) + k >= n) r[j][k] = make_uint4(0, 0, 0, 0);
        store_t4x8(vt, kRPitch, 8 * (it / (kStep / 4)), 4 * (it % (kStep / 4)), r[j]);
      }
    } else {
      const int tq = tid & 15, c16 = tid >> 4;
      if (c16 < D / 16) {
        uint4 lo8[4], hi8[4];  // channels 16 c16 + 0..7 and + 8..15 of tokens 4 tq + k
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const half8 x0 = codes6_reg(cur.v[k][0], cur.v[k][1]);
          const half8 x1 = codes6_reg(__builtin_amdgcn_alignbit(cur.v[k][2], cur.v[k][1], 16), cur.v[k][2] >> 16);
          __builtin_memcpy(&lo8[k], &x0, 16);
          __builtin_memcpy(&hi8[k], &x1, 16);
        }
        store_t4x8(vt, kRPitch, 16 * c16, 4 * tq, lo8);
        store_t4x8(vt, kRPitch, 16 * c16 + 8, 4 * tq, hi8);
      }
    }

    // ---- (2) scores of tile `wave`
    float4v sacc[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) sacc[blk] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      half8 av;
      if (sink) {
        av = mfma_a(ks_op[kk]);
      } else {
        const uint32_t sh = (g & 1) ? 16u : 0u;
        av = codes6_reg(__builtin_amdgcn_alignbit(cur.k[kk].y, cur.k[kk].x, sh), cur.k[kk].y >> sh);
      }
      const int blk = kk / 4;
      sacc[blk] = mfma16(av, mfma_a(qo[kk][0][lane]), sacc[blk]);
      sacc[blk] = mfma16(av, mfma_a(qo[kk][1][lane]), sacc[blk]);
    }
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * wave + 4 * g + r;
      float v = 0.0f;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
        v = sink ? v + sacc[blk][r] : fmaf((float)as_h2(cur.dk[r])[blk], sacc[blk][r], v);
      v = t < n ? v : -INFINITY;
      sc[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = xmax4(mx);
    if (g == 0) xm[wave][q16] = mx;
    __syncthreads();  // maxima; V^T complete

    // ---- (3) weights
    const float M = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16]));  // token t0 is valid
    const float m_new = fmaxf(m_run, M);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first step
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < CPW; ++i) acc[i] *= alpha;
    l_part *= alpha;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(sc[r] - m_new);  // -inf for masked tokens gives 0
      l_part += p[r];
    }
#pragma unroll
    for (int blk = 0; blk < (sink ? 1 : NB); ++blk) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = sink ? p[r] : p[r] * (float)as_h2(cur.dv[r])[blk];
      uint2 hi, lo;
      split_h2(x[0], x[1], hi.x, lo.x);
      split_h2(x[2], x[3], hi.y, lo.y);
      *(uint2*)(pw + ((blk * 2 + 0) * 16 + q16) * kRPitch + 16 * wave + 4 * g) = hi;
      *(uint2*)(pw + ((blk * 2 + 1) * 16 + q16) * kRPitch + 16 * wave + 4 * g) = lo;
    }
    __syncthreads();  // weights

    // ---- (4) O^T += V^T P'^T over this step's tokens
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int cb = CPW * wave + i;
      const int blk = sink ? 0 : (16 * cb) / kQBlock;
#pragma unroll
      for (int j = 0; j < kStep / 32; ++j) {
        const half8 av = mfma_a(*(const uint4*)(vt + (16 * cb + q16) * kRPitch + 32 * j + 8 * g));
        const half8 bh = mfma_a(*(const uint4*)(pw + ((blk * 2 + 0) * 16 + q16) * kRPitch + 32 * j + 8 * g));
        const half8 bl = mfma_a(*(const uint4*)(pw + ((blk * 2 + 1) * 16 + q16) * kRPitch + 32 * j + 8 * g));
        acc[i] = mfma16(av, bh, acc[i]);
        acc[i] = mfma16(av, bl, acc[i]);
      }
    }
    __syncthreads();  // V^T and the weights are free
  };
  if (sink) {
    for (int t0 = t_begin; t0 < t_end; t0 += kStep) step(std::true_type{}, t0, ra, rb);
  } else {
    for (int t0 = t_begin;;) {
      step(std::false_type{}, t0, ra, rb);
      if ((t0 += kStep) >= t_end) break;
      step(std::false_type{}, t0, rb, ra);
      if ((t0 += kStep) >= t_end) break;
    }
  }

  const float lsum = xsum4(l_part);
  if (g == 0) xl[wave][q16] = lsum;
  __syncthreads();
  if (q16 < G) {
    float* P = a.part + (((int64_t)b * a.Hq + h * G + q16) * a.max_chunks + c) * (D + 2);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int ch = 16 * (CPW * wave + i) + 4 * g;
      P[2 + ch + 0] = acc[i][0];
      P[2 + ch + 1] = acc[i][1];
      P[2 + ch + 2] = acc[i][2];
      P[2 + ch + 3] = acc[i][3];
    }
    if (wave == 0 && g == 0) {
      P[0] = m_run * kLn2;
      P[1] = xl[0][q16] + xl[1][q16] + xl[2][q16] + xl[3][q16];
    }
  }
}

// ---------------------------------------------------------------------------
// Append role (fused decode step): the token appended in the same call, for
// one (sequence, KV head).  Waves 0 and 1 rotate and encode its key and value
// into the staging ring slot (the same encoder and bytes as the append
// kernel; the ring items of this launch stop short of that slot), keeping the
// decoded rotated-domain values d (u - 32).  The token's split-K partial is
// then exact and needs no scan: for each query head of the group the score
// s = q' . k (scale and log2 e folded into q'), m = s, l = 1, acc = v.
__device__ __forceinline__ void append_role(const DecodeArgs& a, int b, int h, uint8_t* smem) {
  const Layout& y = a.y;
  const DecodeSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.g;
  float* rows = (float*)smem;     // [16][256] query rows
  float* kv = rows + 16 * 256;    // [2][256] decoded key and value
  uint8_t* arena = const_cast<uint8_t*>(a.arena);  // the one region this launch writes
  if (wave < 2) {
    const uint16_t* src = (wave ? a.v_new : a.k_new) + ((int64_t)b * y.H + h) * 256;
    uint8_t* codes = arena + rcode_off(y, sq.slot, a.layer, h, wave, sq.app_slot);
    uint16_t* scales = (uint16_t*)(arena + rscale_off(y, sq.slot, a.layer, h, wave, sq.app_slot));
    float deq[4];
    encode_chunk<4>(src, codes, scales, lane, a.signs, false, deq);
#pragma unroll
    for (int j = 0; j < 4; ++j) kv[256 * wave + 4 * lane + j] = deq[j];
  }
  QueryRaw<256> qraw;
  query_load<256>(a, b, h, wave, lane, qraw);
  query_rows<256>(a, qraw, true, rows, wave, lane);
  __syncthreads();
  for (int i = wave; i < G; i += 4) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(rows[i * 256 + 4 * lane + j], kv[4 * lane + j], s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    float* P = a.part + (((int64_t)b * a.Hq + h * G + i) * a.max_chunks + sq.app_chunk) * (256 + 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) P[2 + 4 * lane + j] = kv[256 + 4 * lane + j];
    if (lane == 0) {
      P[0] = s * kLn2;
      P[1] = 1.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels.  Work item i of a launch: append items first (fused decode step),
// then body items (when the launch has them), then sink/ring items, each
// sequence by sequence.

constexpr int kMainLds = kBodyLds > RingLds<256>::total ? kBodyLds : RingLds<256>::total;

// Within a sequence, body items interleave the KV heads (item i: head i mod H,
// chunk i / H), so that every head gets its share of first and second
// workgroups of the compute units; sink/ring items are head-major.
__device__ __forceinline__ bool find_item(const DecodeArgs& a, int item, bool body, int& b, int& h, int& c) {
  if (a.n_seqs == 1) {  // no loop: sequence 0's fields are already in registers
    b = 0;
    const int per = body ? a.seq[0].n_body_chunks : 1 + a.seq[0].n_ring_chunks;
    if (item >= a.y.H * per) return false;
    h = body ? item % a.y.H : item / per;
    c = body ? item / a.y.H : item % per;
    return true;
  }
  for (b = 0; b < a.n_seqs; ++b) {
    const int per = body ? a.seq[b].n_body_chunks : 1 + a.seq[b].n_ring_chunks;
    const int n = a.y.H * per;
    if (item < n) {
      if (body) {
        h = item % a.y.H;
        c = item / a.y.H;
      } else {
        h = item / per;
        c = item % per;
      }
      return true;
    }
    item -= n;
  }
  return false;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_main_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kMainLds];
  int b, h, c;
  int item = blockIdx.x;
  // Each dependent round of kernel-argument loads costs a trip to memory at
  // the start of every workgroup; the fields the work items start from are
  // read in one round (empty asm statements consuming them keep the compiler
  // from spreading the loads over the branches that use them).
  {
    const DecodeSeq& s0 = a.seq[0];
    asm volatile("" ::"s"(a.n_app_items), "s"(a.n_body_items), "s"(a.n_seqs), "s"(a.y.H), "s"(a.y.cap),
                 "s"(s0.slot), "s"(s0.n_sink), "s"(s0.ring_len), "s"(s0.ring0), "s"(s0.n_rec), "s"(s0.n_ring_chunks),
                 "s"(s0.n_body_chunks), "s"(s0.app_slot), "s"(s0.app_chunk));
    asm volatile("" ::"s"(a.arena), "s"(a.q), "s"(a.part), "s"(a.prof_ts), "s"(a.y.off_body), "s"(a.y.rec_bytes),
                 "s"(a.y.max_rec), "s"(a.y.L), "s"(a.layer), "s"(a.Hq), "s"(a.g), "s"(a.scale), "s"(a.max_chunks),
                 "s"(a.n_old), "s"(a.ring_chunk));
  }
  prof_start(a.prof_ts);
  if (item < a.n_app_items) {
    append_role(a, item / a.y.H, item % a.y.H, smem);
    prof_end(a.prof_ts);
    return;
  }
  item -= a.n_app_items;
  if (item < a.n_body_items) {
    if (find_item(a, item, true, b, h, c)) body_role(a, b, h, c, smem);
  } else {
    if (find_item(a, item - a.n_body_items, false, b, h, c)) ring_role<256>(a, b, h, c, smem);
  }
  prof_end(a.prof_ts);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_ring_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RingLds<D>::total];
  int b, h, c;
  if (find_item(a, blockIdx.x, false, b, h, c)) ring_role<D>(a, b, h, c, smem);
}

// Append (optional), body (head_dim 256, 4-bit K and V) and sink/ring items in
// one launch.
hipError_t launch_decode_main(const DecodeArgs& a, int n_items, hipStream_t stream) {
  if (a.y.D != 256 || a.y.kbits != 4 || a.y.vbits != 4 || a.ring_chunk % kStep != 0 || a.g > kMaxGroup)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_main_kernel, dim3(n_items), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Sink/ring items only (head_dim 128 or 256).
hipError_t launch_decode_ring(const DecodeArgs& a, int n_items, hipStream_t stream) {
  if (a.ring_chunk % kStep != 0 || a.g > kMaxGroup) return hipErrorInvalidValue;
  switch (a.y.D) {
    case 128: hipLaunchKernelGGL(decode_ring_kernel<128>, dim3(n_items), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_ring_kernel<256>, dim3(n_items), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
