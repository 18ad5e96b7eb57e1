// Matrix-core decode attention: the sealed body, the fp16 sink and the tq6_0
// staging ring in one launch (body records of 256 channels at 4/4 bits, of
// 128 channels with 8-bit keys, or two 256-channel halves of a 512-wide head).
//
// SJ-KVaRN 2.1: one decode pass reads the sink, the staging ring (the exact
// tail) and the sealed body; KV Cache Precision Tail section 2: the region
// results are combined under one softmax (here: split-K partials (m, l, acc)
// merged by the merge kernel).  KV cache math ("rotate first"): the query is
// rotated once, ring and body are read in the rotated domain with no
// dequantise pass, and each work item rotates its few accumulated rows back
// before writing them (R^T is linear, so the merge of rotated-back partials
// equals the rotated-back merge); the sink stays in the original domain and is
// scored with the unrotated query.
//
// Body record math (SJ-KVaRN 2.2: column balance scales C absorbed, per-row
// scale S and zero point Z): k_ij = C_j (S_i n_ij + Z_i), so for the rotated
// query q' and q~_j = q'_j C_j, sigma = sum_j q~_j:
//     q'.k_i = S_i (q~ . (n_i - mid)) + (Z_i + mid S_i) sigma,   mid = 2^(b_K - 1)
//     sum_i p_i v_ij = C_j ( sum_i (p_i S_i) (n_ij - 8) + sum_i p_i (Z_i + 8 S_i) ).
// Ring math (tq6_0: one fp16 scale d per 128-value block, 6-bit codes u):
//     score_t = sum_blocks d_t,b (q' . u_t,b),   out_j = sum_t (p_t d_t,b(j)) u_t,j.
// Every inner product is dense (16 query columns, the group padded to 16) x
// (32 codes) x (16 tokens or channels) on v_mfma_f32_16x16x32_f16, codes
// entering exactly as centred small integers; the non-code operand (q~, q', the weights)
// is split into hi + lo fp16 halves, two products each, which keeps fp32-level
// precision.  The softmax scale and log2(e) are folded into the query, so
// scores come out in log2 units.
//
// Work items, one workgroup (4 waves) each: the appended token's item (fused
// decode step), body chunks (consecutive records of one KV head), then the
// sink and ring chunks of every KV head.  Each item writes one fp32 partial
// row per query head in the original domain; partial 0 is the sink, 1.. the
// ring chunks, then the body chunks, then the appended token.
#include <type_traits>

#include "kvq_codes.h"
#include "kvq_encode.h"

namespace kvq {

// ---------------------------------------------------------------------------
// Query rows: the G query heads of KV head h, times scale * log2(e), rotated
// (R = H/16 for head_dim 256, s2 . H . s1 / sqrt(128) for 128) or not, into
// rows[16][D] of LDS (rows G..15 zero; 512-wide heads rotate each 256-point
// half on its own).  Wave w transforms rows w, w + 4, ...
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
      wave_fwht<VPL, D == 128 ? 128 : 256>(v, lane);  // 512: two 256-point halves
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

// Partial rows of one work item (chunk c of KV head h): rows[i][D] in LDS
// holds the accumulator of query head i of the group (rotated domain unless
// `rotate` is false), m the running maximum of this lane's column (log2
// units, the same in every wave), xl[w][i] wave w's part of l.  Wave w writes
// rows w, w + 4, ..., rotated back to the original domain when `rotate`.  The
// caller synchronises after filling rows and xl.
template <int D>
__device__ __forceinline__ void write_partial_rows(const DecodeArgs& a, int b, int h, int c, const float* rows,
                                                   float m, const float (*xl)[16], bool rotate, int wave, int lane) {
  constexpr int VPL = D / 64;
  for (int i = wave; i < a.g; i += 4) {
    float v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] = rows[i * D + VPL * lane + j];
    if (rotate) rotate_back<D>(v, lane, a.signs);
    float* P = a.part + (((int64_t)b * a.Hq + h * a.g + i) * a.max_chunks + c) * part_stride(D);
    float* dst = P + kPartHead + VPL * lane;
    if constexpr (VPL == 2) {
      *(float2*)dst = make_float2(v[0], v[1]);
    } else {
#pragma unroll
      for (int j = 0; j < VPL; j += 4) *(float4*)(dst + j) = make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]);
    }
    const float mi = __shfl(m, i, 64);  // lane i holds column i
    if (lane == 0) {
      P[0] = mi * kLn2;
      P[1] = xl[0][i] + xl[1][i] + xl[2][i] + xl[3][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Body role: one chunk of records of one KV head.
//
// Record shapes (compile time, BodyShape): a record is NSUB sub-records of
// SUBW channels, each with its own C, S, Z: 128 or 256 channels, or a 512-wide
// head as two 256-channel sub-records, one per rotation half (SJ-KVaRN section
// 9); 4- or 8-bit keys, 4-bit values.  A key row is 64, 128 or 256 bytes; each
// lane loads 16 bytes of it per 64.  A token's score sums the sub-records'
// terms; each sub-record's values take their own weights p S^V.
//   q~:      wave w forms the q~ operands of its k-steps (2 of 8 per 256-channel
//            sub-record, 1 of 4 at 128 channels) for the live rows and shares them;
//   scores:  wave w takes token tiles 2w, 2w+1 (32 tokens) over all channels;
//   values:  wave w takes SUBW / 64 channel tiles of every sub-record over all tokens.
// Key and value codes go from memory straight into the registers of the lane
// that feeds them to the matrix cores (16 bytes per lane and operand), each
// set reloaded as soon as its product is done, so that it has the other half
// of a record's work to land in.  The scales pass through a ring of three LDS
// areas, loaded two records ahead.  Two barriers per record:
//   (B2) after the scores: record maxima exchanged;
//   (B3) after the weights: P', the zero-point sums, q~ and scales of the next
//        record exchanged.
// Token rows are assigned so that the four score rows of a lane are four
// consecutive slots of the value product's operand order (one 8-byte store of
// the weights per tile): position P of a tile holds token
// (P & ~7) + [0, 4, 1, 5, 2, 6, 3, 7][P & 7].
constexpr int kPPitch = 128 + 8;  // halves per weight row (padding spreads LDS banks)
constexpr int kWOld = 15, kWYoung = 10;  // record shares of the first and second workgroup of a compute unit

template <int D_, int KB_>
struct BodyShape {
  static constexpr int D = D_, KB = KB_;
  static constexpr int SUBW = D == 128 ? 128 : 256;
  static constexpr int NSUB = D / SUBW;
  static constexpr int KK = SUBW / 32;         // k-steps of 32 channels per sub-record
  static constexpr int KPW = KK / 4;           // k-steps whose q~ one wave forms
  static constexpr int NP = KPW == 2 ? 2 : 1;  // q~ rows per lane (i and i + 8, or one)
  static constexpr int VT = SUBW / 64;         // value channel tiles per wave and sub-record
  static constexpr int ROWB = SUBW * KB / 8;   // bytes per key row: 64, 128 or 256
  static constexpr int NKS = ROWB / 64;        // 16-byte key loads per lane and token tile
  static constexpr int KCODE = 128 * ROWB, VCODE = SUBW * 64;
  static constexpr int META = 4 * (SUBW + 256);  // K and V: C[SUBW], S[128], Z[128] fp16
  static constexpr int SUB_BYTES = KCODE + VCODE + META;
  static constexpr int WG_PER_CU = NSUB == 2 ? 1 : 2;  // resident workgroups per compute unit
  // A sub-record's scales in LDS (stage_scales): the key C stays fp16 (the q~
  // products take it as is); the rest is widened to fp32 once, at staging:
  // K S [128], K Z [128], V C [SUBW], V S [128], V Z [128].
  static constexpr int L_KS = 2 * SUBW, L_KZ = L_KS + 512, L_VC = L_KZ + 512, L_VS = L_VC + 4 * SUBW;
  static constexpr int L_VZ = L_VS + 512;
  static constexpr int MSTRIDE = 4096;  // LDS bytes per sub-record's scales
  // LDS: q~ operands [NSUB][KK][hi, lo][64 lanes]; weights [NSUB][hi, lo][16][kPPitch];
  // scales [3][NSUB][MSTRIDE]; exchange xm[4][16], xz[NSUB][4][16], xs[NSUB][4][16]
  static constexpr int QT = 0, PW = QT + NSUB * KK * 2 * 64 * 16, MB = PW + NSUB * 2 * 16 * kPPitch * 2;
  static constexpr int X = MB + 3 * NSUB * MSTRIDE;
  static constexpr int total = X + (1 + 2 * NSUB) * 256;
  static_assert(NKS * 64 == ROWB && (KB == 4 ? KK == 4 * NKS : KK == 2 * NKS), "a lane's key dwords cover its k-steps");
  static_assert(16 * D * 4 <= PW - QT, "query rows must fit the q~ area");
  static_assert(L_VZ + 512 <= MSTRIDE && 2 * SUBW + 2 * (8 * 256 - 2 * SUBW) <= MSTRIDE,
                "scales of a sub-record (and the stores of threads past them) fit one LDS area");
  // first channel of the 8 that lane group g feeds to the score product at k-step kk
  static __device__ __forceinline__ int kbase(int kk, int g) {
    return KB == 4 ? 128 * (kk >> 2) + 32 * g + 8 * (kk & 3) : 64 * (kk >> 1) + 16 * g + 8 * (kk & 1);
  }
};

// q~ operands (hi, lo) of this wave's k-steps of one sub-record from its key
// scales C, for the live query rows only.  Lane (i, g) = (lane & 7,
// (lane >> 3) & 3) forms the 8 slots of row i (and i + 8 when the group has
// more than 8 heads) that lane group g of k-step 2 wave + (lane >> 5) feeds to
// the matrix core; at 128 channels (one k-step per wave) the lane's row is
// i + 8 (lane >> 5).  Rows never written stay zero.  Also this wave's part of
// sigma = sum q~ per row.
// Packed (PK, at most 8 heads): one operand per k-step, hi in columns 0..7
// and lo in columns 8..15; at 128 channels lanes 32..63 form the lo halves of
// the same rows as lanes 0..31.
template <class Sh, bool PK>
__device__ __forceinline__ void make_qtilde(const uint8_t* km, const uint4 (&qph)[Sh::NP], const uint4 (&qpl)[Sh::NP],
                                            uint4 (*qt)[2][64], float (*xs)[16], int G, int wave, int lane) {
  const int i = lane & 7, g = (lane >> 3) & 3, h5 = lane >> 5;
  const int kk = Sh::KPW == 2 ? 2 * wave + h5 : wave;
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  const half2v lo_ones = {(_Float16)kLoUnscale, (_Float16)kLoUnscale};  // lo operands carry 2^11
  const uint4 c = *(const uint4*)(km + 2 * Sh::kbase(kk, g));
  uint32_t cp[4];
  if constexpr (Sh::KB == 4) {  // slot pairs (n0, n4), (n1, n5), (n2, n6), (n3, n7)
    cp[0] = __builtin_amdgcn_perm(c.z, c.x, 0x05040100u);
    cp[1] = __builtin_amdgcn_perm(c.z, c.x, 0x07060302u);
    cp[2] = __builtin_amdgcn_perm(c.w, c.y, 0x05040100u);
    cp[3] = __builtin_amdgcn_perm(c.w, c.y, 0x07060302u);
  } else {  // channel order
    cp[0] = c.x;
    cp[1] = c.y;
    cp[2] = c.z;
    cp[3] = c.w;
  }
  const int np = !PK && Sh::NP == 2 && G > 8 ? 2 : 1;
#pragma unroll
  for (int p = 0; p < Sh::NP; ++p) {
    if (p >= np) break;
    const int row = PK ? i : Sh::KPW == 2 ? i + 8 * p : i + 8 * h5;
    uint4 hi, lo;
    qtilde_pair(qph[p].x, qpl[p].x, cp[0], hi.x, lo.x);
    qtilde_pair(qph[p].y, qpl[p].y, cp[1], hi.y, lo.y);
    qtilde_pair(qph[p].z, qpl[p].z, cp[2], hi.z, lo.z);
    qtilde_pair(qph[p].w, qpl[p].w, cp[3], hi.w, lo.w);
    float a1 = 0.0f, a16 = 0.0f;  // 4-bit keys: slots y and w carry 1/16
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.x), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.x), lo_ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.y), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.y), lo_ones, a16, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.z), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.z), lo_ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.w), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.w), lo_ones, a16, false);
    if (!PK) {
      qt[kk][0][16 * g + row] = hi;
      qt[kk][1][16 * g + row] = lo;
    } else if (Sh::KPW == 2) {
      qt[kk][0][16 * g + row] = hi;
      qt[kk][0][16 * g + 8 + row] = lo;
    } else {
      qt[kk][0][16 * g + 8 * h5 + row] = h5 ? lo : hi;
    }
    float part = Sh::KB == 4 ? fmaf(16.0f, a16, a1) : a1 + a16;
    part = add_x8(part);  // over g: lanes l ^ 8, l ^ 16 (and over the two k-steps: l ^ 32)
    {
      const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(part), __float_as_int(part), false, false);
      part = __int_as_float(b[0]) + __int_as_float(b[1]);
    }
    if (Sh::KPW == 2) {
      const auto c = __builtin_amdgcn_permlane32_swap(__float_as_int(part), __float_as_int(part), false, false);
      part = __int_as_float(c[0]) + __int_as_float(c[1]);
    }
    // packed at 128 channels: lanes 32..63 repeat the rows of lanes 0..31
    if (Sh::KPW == 2 || PK ? (lane >> 3) == 0 : ((lane >> 3) & 3) == 0) xs[wave][row] = part;
  }
}

// Key codes of token tiles 2 wave, 2 wave + 1: lane (m, g) loads 16 bytes at
// 64 s + 16 g of its token's row, s < NKS.  dummy: every lane reads the first
// 16 bytes of `sub` (one line, result unused).
template <class Sh>
__device__ __forceinline__ void load_keys(const uint8_t* __restrict__ sub, uint4 (&kd)[2][Sh::NKS], int wave,
                                          int lane, bool dummy = false) {
  const int m = lane & 15, g = lane >> 4;
  const int row = (m & 8) + slot_token(m & 7);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int s = 0; s < Sh::NKS; ++s)
      kd[i][s] = ld_stream16(sub + (dummy ? 0 : (16 * (2 * wave + i) + row) * Sh::ROWB + 64 * s + 16 * g));
}
template <class Sh>
__device__ __forceinline__ void load_values(const uint8_t* __restrict__ sub, uint4 (&vd)[Sh::VT], int wave, int lane,
                                            bool dummy = false) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < Sh::VT; ++j)
    vd[j] = ld_stream16(sub + (dummy ? 0 : Sh::KCODE + (16 * (Sh::VT * wave + j) + m) * 64 + 16 * g));
}

template <class Sh, bool PK>
__device__ __forceinline__ void body_role(const DecodeArgs& a, int b, int h, int cbk, uint8_t* smem) {
  constexpr int D = Sh::D, SUBW = Sh::SUBW, NSUB = Sh::NSUB, KK = Sh::KK, VT = Sh::VT, NP = Sh::NP;
  constexpr int SB = Sh::SUB_BYTES, MS = Sh::MSTRIDE;
  const Layout& y = a.y;
  const DecodeSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4;
  const int G = a.g;
  uint4(*qt)[KK][2][64] = (uint4(*)[KK][2][64])(smem + Sh::QT);
  uint16_t(*pw)[2][16][kPPitch] = (uint16_t(*)[2][16][kPPitch])(smem + Sh::PW);
  uint8_t* mbuf = smem + Sh::MB;  // scales of records r, r + 1, r + 2 (mod 3)
  float(*xm)[16] = (float(*)[16])(smem + Sh::X);
  float(*xz)[4][16] = (float(*)[4][16])(smem + Sh::X + 256);
  float(*xs)[4][16] = (float(*)[4][16])(smem + Sh::X + 256 + NSUB * 256);

  // Partition of the sequence's records over its chunks.  With two
  // workgroups per compute unit, the first to land on a unit (grid index below
  // n_old) wins the issue arbitration against the second and scans a record
  // ~1.4 times as fast (measured); it takes kWOld records for every kWYoung of
  // the second (1.5: the second also pays the longer tail, measured best), so
  // that both end together; with few records per chunk, or one workgroup per
  // unit, the split is even.
  const int nb = sq.n_body_chunks;
  int r0, r1;
  if (Sh::WG_PER_CU == 2 && sq.n_rec >= 4 * nb) {
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
  auto mslot = [&](int r) { return mbuf + ((r - r0) % 3) * (NSUB * MS); };
  // this thread's 8 bytes of a sub-record's scales (clamped: threads past the
  // end re-read the last 8 bytes and store them where nothing reads)
  const int mo = Sh::KCODE + Sh::VCODE + (Sh::META == 8 * 256 ? 8 * tid : min(8 * tid, Sh::META - 8));

  // ---- prologue: the query first, then the scales of r0, r0 + 1 and the key
  // and value codes of r0 in flight while the query is rotated (its rows
  // borrow the q~ area)
  QueryRaw<D> qraw;
  query_load<D>(a, b, h, wave, lane, qraw);
  uint2 m0[NSUB], m1[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    m0[s] = ld_stream8(rec(r0) + s * SB + mo);
    m1[s] = ld_stream8(r0 + 1 < r1 ? rec(r0 + 1) + s * SB + mo : rec0);
  }
  uint4 kd[NSUB][2][Sh::NKS], vd[NSUB][VT];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) load_keys<Sh>(rec(r0) + s * SB, kd[s], wave, lane);
  float* rows = (float*)qt;
  query_rows<D>(a, qraw, true, rows, wave, lane);
  __syncthreads();
  uint4 qph[NSUB][NP], qpl[NSUB][NP];  // q' of this lane's q~ slots (make_qtilde)
  {
    const int ui = lane & 7, ug = (lane >> 3) & 3, h5 = lane >> 5;
    const int base = Sh::kbase(Sh::KPW == 2 ? 2 * wave + h5 : wave, ug);  // channels of lane group ug's slots
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int row_i = PK ? ui : Sh::KPW == 2 ? ui + 8 * p : ui + 8 * h5;
        const float* row = rows + row_i * D + SUBW * s + base;  // rows past the group are zero
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          if (Sh::KB == 4) {
            const float f = (pr & 1) ? 0.0625f : 1.0f;  // pairs read from high nibbles carry 1/16
            split_h2s(row[pr] * f, row[pr + 4] * f, hb[pr], lb[pr]);
          } else {
            split_h2s(row[2 * pr], row[2 * pr + 1], hb[pr], lb[pr]);
          }
        }
        qph[s][p] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
        qpl[s][p] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
      }
  }
  __syncthreads();  // the query rows are read: the q~ area is cleared (rows make_qtilde skips stay zero)
#pragma unroll
  for (int j = 0; j < NSUB * KK / 2; ++j) ((uint4*)qt)[tid + 256 * j] = make_uint4(0, 0, 0, 0);
  if (tid < 64 * NSUB) (&xs[0][0][0])[tid] = 0.0f;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    stage_scales<Sh>(mslot(r0) + s * MS, m0[s], tid);
    if (r0 + 1 < r1) stage_scales<Sh>(mslot(r0 + 1) + s * MS, m1[s], tid);
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NSUB; ++s) make_qtilde<Sh, PK>(mslot(r0) + s * MS, qph[s], qpl[s], qt[s], xs[s], G, wave, lane);
  // the first record's value codes only now: at the start of the launch every
  // workgroup asks for its first record at once, and keys requested ahead of
  // values arrive ahead of them, so the first scores start sooner
#pragma unroll
  for (int s = 0; s < NSUB; ++s) load_values<Sh>(rec(r0) + s * SB, vd[s], wave, lane);
  uint2 mnext[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) mnext[s] = ld_stream8(r0 + 2 < r1 ? rec(r0 + 2) + s * SB + mo : rec0);
  __syncthreads();

  float m_run = -INFINITY, l_part = 0.0f;
  float4v acc[NSUB][VT];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int i = 0; i < VT; ++i) acc[s][i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  for (int r = r0; r < r1; ++r) {
    const uint8_t* mr = mslot(r);
    const bool more = r + 1 < r1;

    // ---- scores of tiles 2 wave, 2 wave + 1: independent accumulation chains
    // (sub-record x tile x hi/lo) keep the matrix core busy between dependent
    // products; packed, one chain per sub-record and tile carries both halves
    constexpr int NK = NSUB * KK;
    float4v sh[NSUB][2], sl[NSUB][2];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) sh[s][i] = sl[s][i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
    // q~ operands read from LDS two k-steps ahead of their products
    half8 qb[NK][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      qb[k][0] = mfma_a(qt[k / KK][k % KK][0][lane]);
      if (!PK) qb[k][1] = mfma_a(qt[k / KK][k % KK][1][lane]);
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int s = k / KK, kk = k % KK;
      if (k + 2 < NK) {
        qb[k + 2][0] = mfma_a(qt[(k + 2) / KK][(k + 2) % KK][0][lane]);
        if (!PK) qb[k + 2][1] = mfma_a(qt[(k + 2) / KK][(k + 2) % KK][1][lane]);
      }
      const half8 bh = qb[k][0], bl = PK ? bh : qb[k][1];
      half8 av[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (Sh::KB == 4)
          av[i] = nib8_sub(pick(kd[s][i][kk >> 2], kk & 3));
        else
          av[i] = byte8_sub(pick(kd[s][i][kk >> 1], 2 * (kk & 1)), pick(kd[s][i][kk >> 1], 2 * (kk & 1) + 1));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) sh[s][i] = mfma16(av[i], bh, sh[s][i]);
      if (!PK) {
#pragma unroll
        for (int i = 0; i < 2; ++i) sl[s][i] = mfma16(av[i], bl, sl[s][i]);
      }
    }
    // packed: column c + 8 holds the lo half of column c; lanes l and l ^ 8
    // (columns c, c + 8 of the same rows) both get the sum, bit for bit
    if (PK) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) sh[s][i][j] = add_x8_lo(sh[s][i][j], lane);
    }
    // this lane's rows are positions 16 bb + 4 g + j: tokens base + {0,4,1,5}
    // (g even) or base + {2,6,3,7} (g odd), base = 16 bb + 8 (g / 2).  The
    // products hold q~ . n 2^-24 (subnormal key codes); the scores are kept
    // times 2^-24 up to the exponent's argument: S (dot - mid sigma 2^-24) +
    // (Z + mid S) sigma 2^-24, the centre taken off before the scale.
    const int tb = 8 * (g >> 1) + 2 * (g & 1);
    float sc[2][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const uint8_t* km = mr + s * MS;
      const int qr = PK ? q16 & 7 : q16;  // packed: columns c and c + 8 score query row c
      const float sig = (xs[s][0][qr] + xs[s][1][qr] + xs[s][2][qr] + xs[s][3][qr]) * kSub;
      const float cm = (float)(1 << (Sh::KB - 1)) * sig;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int T = 16 * (2 * wave + i) + tb;
        const float2 s01 = *(const float2*)(km + Sh::L_KS + 4 * T), s45 = *(const float2*)(km + Sh::L_KS + 4 * T + 16);
        const float2 z01 = *(const float2*)(km + Sh::L_KZ + 4 * T), z45 = *(const float2*)(km + Sh::L_KZ + 4 * T + 16);
        const float Sj[4] = {s01.x, s45.x, s01.y, s45.y};
        const float Zj[4] = {z01.x, z45.x, z01.y, z45.y};
        const float4v dot = PK ? sh[s][i] : sh[s][i] + sl[s][i] * kLoUnscale;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float zc = fmaf((float)(1 << (Sh::KB - 1)), Sj[j], Zj[j]);  // Z + mid S
          const float v = fmaf(Sj[j], dot[j] - cm, zc * sig);
          sc[i][j] = s == 0 ? v : sc[i][j] + v;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[i][j]);
    mx = xmax4(mx);
    if (g == 0) xm[wave][q16] = mx;
    __syncthreads();  // (B2) record maxima; q~ of r and the key codes are free
    // loads are unconditional (a branch around them makes the compiler's wait
    // counting conservative): past the last record they re-read one 16-byte
    // line of record r0 and are not used
#pragma unroll
    for (int s = 0; s < NSUB; ++s) load_keys<Sh>(more ? rec(r + 1) + s * SB : rec0, kd[s], wave, lane, !more);

    const float mrec = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16])) * kUnSub;
    const float m_new = fmaxf(m_run, mrec);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first record
    // the record's weights are taken relative to its own maximum, so that the
    // fp16 hi/lo weight operands of its significant tokens stay normal (their
    // absolute floor 2^-25 would otherwise grow relative to the weights as the
    // chunk's running maximum climbs); its fp32 contribution and its share of
    // l carry the factor 2^(mrec - m_new) <= 1
    const float frec = __builtin_amdgcn_exp2f(mrec - m_new);
    m_run = m_new;
    if (alpha != 1.0f) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < VT; ++i) acc[s][i] *= alpha;
    }
    l_part *= alpha;
    float p[2][4], lrec = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[i][j] = __builtin_amdgcn_exp2f(fmaf(sc[i][j], kUnSub, -mrec));  // argument <= 0 (exact scaling)
        lrec += p[i][j];
      }
    l_part = fmaf(frec, lrec, l_part);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const uint8_t* vm = mr + s * MS;
      float zt = 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int T = 16 * (2 * wave + i) + tb;
        const float2 s01 = *(const float2*)(vm + Sh::L_VS + 4 * T), s45 = *(const float2*)(vm + Sh::L_VS + 4 * T + 16);
        const float2 z01 = *(const float2*)(vm + Sh::L_VZ + 4 * T), z45 = *(const float2*)(vm + Sh::L_VZ + 4 * T + 16);
        const float Sj[4] = {s01.x, s45.x, s01.y, s45.y};
        const float Zj[4] = {z01.x, z45.x, z01.y, z45.y};
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          zt = fmaf(p[i][j], fmaf(8.0f, Sj[j], Zj[j]), zt);
          x[j] = p[i][j] * Sj[j];
        }
        x[2] *= 0.0625f;  // odd tokens sit in the high nibbles: their slots carry 1/16
        x[3] *= 0.0625f;
        uint2 hi, lo;
        split_h2(x[0], x[1], hi.x, lo.x);
        split_h2(x[2], x[3], hi.y, lo.y);
        if (PK) {  // columns 0..7 take hi, 8..15 lo of the same query rows
          *(uint2*)&pw[s][0][q16][16 * (2 * wave + i) + 4 * g] = q16 < 8 ? hi : lo;
        } else {
          *(uint2*)&pw[s][0][q16][16 * (2 * wave + i) + 4 * g] = hi;
          *(uint2*)&pw[s][1][q16][16 * (2 * wave + i) + 4 * g] = lo;
        }
      }
      zt = xsum4(zt);
      if (g == 0) xz[s][wave][q16] = zt;
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        make_qtilde<Sh, PK>(mslot(r + 1) + s * MS, qph[s], qpl[s], qt[s], xs[s], G, wave, lane);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (r + 2 < r1) stage_scales<Sh>(mslot(r + 2) + s * MS, mnext[s], tid);
      mnext[s] = ld_stream8(r + 3 < r1 ? rec(r + 3) + s * SB + mo : rec0);
    }
    __syncthreads();  // (B3) weights, zero-point sums; q~ and scales of r + 1, r + 2

#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      // packed, the lo columns accumulate apart from the hi columns until the
      // end of the chunk; the zero-point sum goes to the hi columns only
      const float corr = PK && q16 >= 8 ? 0.0f : xz[s][0][q16] + xz[s][1][q16] + xz[s][2][q16] + xz[s][3][q16];
      half8 pbh[4], pbl[4] = {};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        pbh[t] = mfma_a(*(const uint4*)&pw[s][0][q16][32 * g + 8 * t]);
        if (!PK) pbl[t] = mfma_a(*(const uint4*)&pw[s][1][q16][32 * g + 8 * t]);
      }
      float4v o[VT];
#pragma unroll
      for (int j = 0; j < VT; ++j) o[j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // channel tiles as independent chains
        half8 av[VT];
#pragma unroll
        for (int j = 0; j < VT; ++j) av[j] = nib8_centred(pick(vd[s][j], t));
#pragma unroll
        for (int j = 0; j < VT; ++j) o[j] = mfma16(av[j], pbh[t], o[j]);
        if (!PK) {
#pragma unroll
          for (int j = 0; j < VT; ++j) o[j] = mfma16(av[j], pbl[t], o[j]);
        }
      }
      load_values<Sh>(more ? rec(r + 1) + s * SB : rec0, vd[s], wave, lane, !more);
      const uint8_t* vm = mr + s * MS;
#pragma unroll
      for (int j = 0; j < VT; ++j) {
        const int cb = VT * wave + j;
        const float4 c = *(const float4*)(vm + Sh::L_VC + 4 * (16 * cb + 4 * g));
        acc[s][j][0] = fmaf(c.x * frec, o[j][0] + corr, acc[s][j][0]);
        acc[s][j][1] = fmaf(c.y * frec, o[j][1] + corr, acc[s][j][1]);
        acc[s][j][2] = fmaf(c.z * frec, o[j][2] + corr, acc[s][j][2]);
        acc[s][j][3] = fmaf(c.w * frec, o[j][3] + corr, acc[s][j][3]);
      }
    }
  }
  if (PK) {  // lo columns into the hi columns
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[s][j][e] = add_x8(acc[s][j][e]);
  }

  // ---- partial of this chunk: every wave holds the same m; l sums over
  // waves.  The accumulators pass through the q~ area (no wave reads q~ after
  // the last record's scores) to be rotated back row by row.
  const float lsum = xsum4(l_part);
  if (g == 0) xm[wave][q16] = lsum;
  if (q16 < G) {  // rows: the q~ area, as in the prologue
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int j = 0; j < VT; ++j)
        *(float4v*)(rows + q16 * D + SUBW * s + 16 * (VT * wave + j) + 4 * g) = acc[s][j];
  }
  __syncthreads();
  write_partial_rows<D>(a, b, h, 1 + sq.n_ring_chunks + cbk, rows, m_run, xm, true, wave, lane);
}

// ---------------------------------------------------------------------------
// Low-bit body role: 2- or 3-bit keys and values (SJ-KVaRN 2.3: the 3/3 and
// 3/2 scalar bodies; 2/2), 256-wide heads, one chunk of records of one KV
// head.  The same record math and work split as body_role, in natural slot
// order: at k-step kk, lane group g of the score product feeds channels
// 64 g + 8 kk .. + 7 (its 64 channels of a key row are 8 B bytes of the row),
// and of the value product tokens 32 g + 8 t .. + 7 of a channel row (4 B
// bytes); codes are unpacked into exact centred fp16 (c - 2^(B-1)).  The hi
// and lo query and weight operands take separate products.
template <int KB_, int VB_>
struct LbShape {
  static constexpr int KB = KB_, VB = VB_, SUBW = 256, KK = 8, VT = 4;
  static constexpr int KROW = SUBW * KB / 8, VROW = 128 * VB / 8;  // bytes per key / value code row
  static constexpr int KCODE = 128 * KROW, VCODE = SUBW * VROW;
  static constexpr int META = 4 * (SUBW + 256);
  static constexpr int SUB_BYTES = KCODE + VCODE + META;
  static constexpr int KW = 2 * KB, VW = VB;  // dwords per lane of a key row / value row share
  // scales in LDS as stage_scales lays them out
  static constexpr int L_KS = 2 * SUBW, L_KZ = L_KS + 512, L_VC = L_KZ + 512, L_VS = L_VC + 4 * SUBW;
  static constexpr int L_VZ = L_VS + 512, MSTRIDE = 4096;
  // LDS: q~ operands [KK][hi, lo][64 lanes]; weights [hi, lo][16][kPPitch]; scales [3][MSTRIDE];
  // exchange xm[4][16], xz[4][16], xs[4][16]
  static constexpr int QT = 0, PW = QT + KK * 2 * 64 * 16, MB = PW + 2 * 16 * kPPitch * 2;
  static constexpr int X = MB + 3 * MSTRIDE;
  static constexpr int total = X + 3 * 256;
  static_assert(16 * SUBW * 4 <= PW - QT, "query rows fit the q~ area");
};

template <class Sh>
__device__ __forceinline__ void load_keys_lb(const uint8_t* __restrict__ rec, uint32_t (&kd)[2][Sh::KW], int wave,
                                             int lane, bool dummy) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint8_t* p = rec + (dummy ? 0 : (16 * (2 * wave + i) + m) * Sh::KROW + 8 * Sh::KB * g);
#pragma unroll
    for (int j = 0; j < Sh::KW / 2; ++j) {
      const uint2 v = ld_stream8(p + 8 * j);
      kd[i][2 * j] = v.x;
      kd[i][2 * j + 1] = v.y;
    }
  }
}
template <class Sh>
__device__ __forceinline__ void load_values_lb(const uint8_t* __restrict__ rec, uint32_t (&vd)[Sh::VT][Sh::VW],
                                               int wave, int lane, bool dummy) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < Sh::VT; ++j) {
    const uint32_t* p =
        (const uint32_t*)(rec + (dummy ? 0 : Sh::KCODE + (16 * (Sh::VT * wave + j) + m) * Sh::VROW + 4 * Sh::VB * g));
#pragma unroll
    for (int k = 0; k < Sh::VW; ++k) vd[j][k] = p[k];
  }
}

template <class Sh>
__device__ __forceinline__ void body_role_lb(const DecodeArgs& a, int b, int h, int cbk, uint8_t* smem) {
  constexpr int D = 256, SUBW = Sh::SUBW, KK = Sh::KK, VT = Sh::VT, MS = Sh::MSTRIDE;
  constexpr float kMidK = (float)(1 << (Sh::KB - 1)), kMidV = (float)(1 << (Sh::VB - 1));
  const Layout& y = a.y;
  const DecodeSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q16 = lane & 15, g = lane >> 4;
  uint4(*qt)[2][64] = (uint4(*)[2][64])(smem + Sh::QT);
  uint16_t(*pw)[16][kPPitch] = (uint16_t(*)[16][kPPitch])(smem + Sh::PW);
  uint8_t* mbuf = smem + Sh::MB;
  float(*xm)[16] = (float(*)[16])(smem + Sh::X);
  float(*xz)[16] = (float(*)[16])(smem + Sh::X + 256);
  float(*xs)[16] = (float(*)[16])(smem + Sh::X + 512);

  // records of this chunk: the weighted split of body_role (two workgroups per CU)
  const int nb = sq.n_body_chunks;
  int r0, r1;
  if (sq.n_rec >= 4 * nb) {
    const int g_base = (int)blockIdx.x - cbk * y.H - h;
    const int n_first = max(0, (a.n_old - g_base - h + y.H - 1) / y.H);
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
  auto mslot = [&](int r) { return mbuf + ((r - r0) % 3) * MS; };
  const int mo = Sh::KCODE + Sh::VCODE + 8 * tid;  // META is 8 x 256 bytes

  // ---- prologue: query, scales of r0 and r0 + 1, codes of r0
  QueryRaw<D> qraw;
  query_load<D>(a, b, h, wave, lane, qraw);
  const uint2 m0 = ld_stream8(rec(r0) + mo);
  const uint2 m1 = ld_stream8(r0 + 1 < r1 ? rec(r0 + 1) + mo : rec0);
  uint32_t kd[2][Sh::KW], vd[VT][Sh::VW];
  load_keys_lb<Sh>(rec(r0), kd, wave, lane, false);
  float* rows = (float*)qt;
  query_rows<D>(a, qraw, true, rows, wave, lane);
  __syncthreads();
  // q' of this lane's q~ slots: query row q16, channels 64 g + 8 kk .. + 7 for
  // kk = 2 wave, 2 wave + 1, split hi + scaled lo
  uint4 qph[2], qpl[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float* r = rows + q16 * D + 64 * g + 8 * (2 * wave + k);
    uint32_t hh[4], ll[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) split_h2s(r[2 * pr], r[2 * pr + 1], hh[pr], ll[pr]);
    qph[k] = make_uint4(hh[0], hh[1], hh[2], hh[3]);
    qpl[k] = make_uint4(ll[0], ll[1], ll[2], ll[3]);
  }
  __syncthreads();  // the query rows are read
  stage_scales<Sh>(mslot(r0), m0, tid);
  if (r0 + 1 < r1) stage_scales<Sh>(mslot(r0 + 1), m1, tid);
  __syncthreads();
  // q~ of the k-steps 2 wave, 2 wave + 1 for record r (key C fp16 at the start
  // of its scale area) and this wave's part of sigma = sum q~ per query row
  auto make_qt = [&](const uint8_t* km) {
    const half2v lo_ones = {(_Float16)kLoUnscale, (_Float16)kLoUnscale};
    const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int kk = 2 * wave + k;
      const uint4 c = *(const uint4*)(km + 2 * (64 * g + 8 * kk));
      uint4 hi, lo;
      qtilde_pair(qph[k].x, qpl[k].x, c.x, hi.x, lo.x);
      qtilde_pair(qph[k].y, qpl[k].y, c.y, hi.y, lo.y);
      qtilde_pair(qph[k].z, qpl[k].z, c.z, hi.z, lo.z);
      qtilde_pair(qph[k].w, qpl[k].w, c.w, hi.w, lo.w);
      qt[kk][0][lane] = hi;
      qt[kk][1][lane] = lo;
      part = __builtin_amdgcn_fdot2(as_h2(hi.x), ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(hi.y), ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(hi.z), ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(hi.w), ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(lo.x), lo_ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(lo.y), lo_ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(lo.z), lo_ones, part, false);
      part = __builtin_amdgcn_fdot2(as_h2(lo.w), lo_ones, part, false);
    }
    part = xsum4(part);  // over the lane groups: the wave's 64 channels of row q16
    if (g == 0) xs[wave][q16] = part;
  };
  make_qt(mslot(r0));
  load_values_lb<Sh>(rec(r0), vd, wave, lane, false);
  uint2 mnext = ld_stream8(r0 + 2 < r1 ? rec(r0 + 2) + mo : rec0);
  __syncthreads();

  float m_run = -INFINITY, l_part = 0.0f;
  float4v acc[VT];
#pragma unroll
  for (int i = 0; i < VT; ++i) acc[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  for (int r = r0; r < r1; ++r) {
    const uint8_t* mr = mslot(r);
    const bool more = r + 1 < r1;
    // ---- scores of tiles 2 wave, 2 wave + 1: rows are tokens 16 (2 wave + i) + 4 g + j
    float4v sh[2], sl[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) sh[i] = sl[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const half8 bh = mfma_a(qt[kk][0][lane]), bl = mfma_a(qt[kk][1][lane]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const half8 av = codes_lb_sub<Sh::KB>(step_bits<Sh::KB>(kd[i], kk));
        sh[i] = mfma16(av, bh, sh[i]);
        sl[i] = mfma16(av, bl, sl[i]);
      }
    }
    // subnormal key codes: scores times 2^-24 up to the exponent's argument,
    // S (dot - mid sigma 2^-24) + (Z + mid S) sigma 2^-24 (as in body_role)
    const float sig = (xs[0][q16] + xs[1][q16] + xs[2][q16] + xs[3][q16]) * kSub;
    const float cm = kMidK * sig;
    float sc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int T = 16 * (2 * wave + i) + 4 * g;
      const float4 S = *(const float4*)(mr + Sh::L_KS + 4 * T), Z = *(const float4*)(mr + Sh::L_KZ + 4 * T);
      const float Sj[4] = {S.x, S.y, S.z, S.w}, Zj[4] = {Z.x, Z.y, Z.z, Z.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dot = sh[i][j] + sl[i][j] * kLoUnscale;
        sc[i][j] = fmaf(Sj[j], dot - cm, fmaf(kMidK, Sj[j], Zj[j]) * sig);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[i][j]);
    mx = xmax4(mx);
    if (g == 0) xm[wave][q16] = mx;
    __syncthreads();  // (B2) record maxima; q~ of r and the key codes are free
    load_keys_lb<Sh>(more ? rec(r + 1) : rec0, kd, wave, lane, !more);

    const float mrec = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16])) * kUnSub;
    const float m_new = fmaxf(m_run, mrec);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first record
    const float frec = __builtin_amdgcn_exp2f(mrec - m_new);    // the record's weights are relative to mrec
    m_run = m_new;
    if (alpha != 1.0f) {
#pragma unroll
      for (int i = 0; i < VT; ++i) acc[i] *= alpha;
    }
    l_part *= alpha;
    float lrec = 0.0f, zt = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int T = 16 * (2 * wave + i) + 4 * g;
      const float4 S = *(const float4*)(mr + Sh::L_VS + 4 * T), Z = *(const float4*)(mr + Sh::L_VZ + 4 * T);
      const float Sj[4] = {S.x, S.y, S.z, S.w}, Zj[4] = {Z.x, Z.y, Z.z, Z.w};
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[i][j], kUnSub, -mrec));
        lrec += p;
        zt = fmaf(p, fmaf(kMidV, Sj[j], Zj[j]), zt);
        x[j] = p * Sj[j];
      }
      uint2 hi, lo;
      split_h2s(x[0], x[1], hi.x, lo.x);
      split_h2s(x[2], x[3], hi.y, lo.y);
      *(uint2*)&pw[0][q16][T] = hi;
      *(uint2*)&pw[1][q16][T] = lo;
    }
    l_part = fmaf(frec, lrec, l_part);
    zt = xsum4(zt);
    if (g == 0) xz[wave][q16] = zt;
    if (more) make_qt(mslot(r + 1));
    if (r + 2 < r1) stage_scales<Sh>(mslot(r + 2), mnext, tid);
    mnext = ld_stream8(r + 3 < r1 ? rec(r + 3) + mo : rec0);
    __syncthreads();  // (B3) weights, zero-point sums; q~ and scales of r + 1, r + 2

    // ---- values: channel tiles VT wave + j over the record's 128 tokens
    const float corr = xz[0][q16] + xz[1][q16] + xz[2][q16] + xz[3][q16];
    half8 pbh[4], pbl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pbh[t] = mfma_a(*(const uint4*)&pw[0][q16][32 * g + 8 * t]);
      pbl[t] = mfma_a(*(const uint4*)&pw[1][q16][32 * g + 8 * t]);
    }
    float4v oh[VT], ol[VT];
#pragma unroll
    for (int j = 0; j < VT; ++j) oh[j] = ol[j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int j = 0; j < VT; ++j) {
        const half8 av = codes_lb<Sh::VB>(step_bits<Sh::VB>(vd[j], t));
        oh[j] = mfma16(av, pbh[t], oh[j]);
        ol[j] = mfma16(av, pbl[t], ol[j]);
      }
    }
    load_values_lb<Sh>(more ? rec(r + 1) : rec0, vd, wave, lane, !more);
#pragma unroll
    for (int j = 0; j < VT; ++j) {
      const int cb = VT * wave + j;
      const float4 c = *(const float4*)(mr + Sh::L_VC + 4 * (16 * cb + 4 * g));
      const float cc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[j][e] = fmaf(cc[e] * frec, oh[j][e] + ol[j][e] * kLoUnscale + corr, acc[j][e]);
    }
  }

  // ---- partial of this chunk, rotated back row by row through the q~ area
  const float lsum = xsum4(l_part);
  if (g == 0) xm[wave][q16] = lsum;
  if (q16 < a.g) {
#pragma unroll
    for (int j = 0; j < VT; ++j) *(float4v*)(rows + q16 * D + 16 * (VT * wave + j) + 4 * g) = acc[j];
  }
  __syncthreads();
  write_partial_rows<D>(a, b, h, 1 + sq.n_ring_chunks + cbk, rows, m_run, xm, true, wave, lane);
}

// ---------------------------------------------------------------------------
// Sink / ring role: chunk c of one KV head, c = 0 the sink (n_sink fp16 tokens,
// original domain), c >= 1 ring tokens [(c - 1) ring_chunk, c ring_chunk).
// With f16 staging the ring chunks are read as the sink is: fp16 rows in the
// original domain, scored with the unrotated query, their sums not rotated
// back (the rows wrap around the ring's slots).
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

// Registers of one ring step for this thread:
//   k[kk]  the two aligned dwords holding the 8 key codes of its A operand
//          (token 16 wave + (lane & 15), channels 32 kk + 8 g ..);
//   dk/dv  the block scales of its 4 output tokens 16 wave + 4 g + r;
//   v      value codes of tokens 4 tq .. 4 tq + 3, channels 16 c16 .. + 15
//          (12 bytes each), tq = tid & 15, c16 = (tid >> 4) + 16 u (u < NV).
template <int D>
struct RingRegs {
  static constexpr int NB = D / kQBlock, KK = D / 32, NV = D >= 256 ? D / 256 : 1, NS = (NB + 1) / 2;
  uint2 k[KK];
  uint32_t dk[4][NS], dv[4][NS];
  uint32_t v[NV][4][3];
};
template <int D>
__device__ __forceinline__ float block_scale(const uint32_t (&d)[RingRegs<D>::NS], int blk) {
  return (float)as_h2(d[blk >> 1])[blk & 1];
}

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
    // a masked token carries the (finite) scales of token 0; its weight is 0
    if (NB == 1) {
      R.dk[r][0] = *(const uint16_t*)(ks + (int64_t)sl * 2);
      R.dv[r][0] = *(const uint16_t*)(vs + (int64_t)sl * 2);
    } else {
#pragma unroll
      for (int e = 0; e < NB / 2; ++e) {
        R.dk[r][e] = *(const uint32_t*)(ks + (int64_t)sl * 2 * NB + 4 * e);
        R.dv[r][e] = *(const uint32_t*)(vs + (int64_t)sl * 2 * NB + 4 * e);
      }
    }
  }
  constexpr int NV = RingRegs<D>::NV;
  const int tq = tid & 15;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int c16 = ((tid >> 4) + 16 * u) % (D / 16);  // head_dim 128: two threads per item, one used
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = 4 * tq + k;
      const uint32_t* p = (const uint32_t*)(vc + (int64_t)slot_of(t < n ? t : 0) * (NB * kQBytes) + 12 * c16);
      R.v[u][k][0] = p[0];
      R.v[u][k][1] = p[1];
      R.v[u][k][2] = p[2];
    }
  }
}

// PK (at most 8 query heads): the hi and lo halves of the query operands and
// of the weights share one product, hi in columns 0..7 and lo in 8..15, as in
// the body; the value sums keep their lo columns apart until the end.
template <int D, bool PK>
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
  const bool exact = sink || y.f16ring;  // fp16 rows in the original domain
  const int t_begin = sink ? 0 : (c - 1) * a.ring_chunk;
  const int t_end = sink ? sq.n_sink : min(sq.ring_len, c * a.ring_chunk);

  QueryRaw<D> qraw;
  query_load<D>(a, b, h, wave, lane, qraw);
  RingRegs<D> ra, rb;
  if (!exact) ring_load<D>(a, sq, h, t_begin, t_end - t_begin, ra);

  // ---- query operands in natural channel order, rotated (ring) or not (sink),
  // kept in LDS: wave w forms k-steps w, w + 4, ...
  {
    float* rows = (float*)vt;
    query_rows<D>(a, qraw, !exact, rows, wave, lane);
    __syncthreads();
    for (int kk = wave; kk < KK; kk += 4) {
      const float* r = rows + (PK ? q16 & 7 : q16) * D + 32 * kk + 8 * g;
      uint32_t hh[4], ll[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) split_h2s(r[2 * pr], r[2 * pr + 1], hh[pr], ll[pr]);
      const uint4 hi = make_uint4(hh[0], hh[1], hh[2], hh[3]), lo = make_uint4(ll[0], ll[1], ll[2], ll[3]);
      if (PK) {
        qo[kk][0][lane] = q16 < 8 ? hi : lo;
      } else {
        qo[kk][0][lane] = hi;
        qo[kk][1][lane] = lo;
      }
    }
    __syncthreads();
  }
  // fp16 rows: the sink's token t, or the f16 ring's token t at slot ring0 + t
  const uint16_t* ksrc = sink ? (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, sq.slot, a.layer, h, 0, 0)
                              : (const uint16_t*)(a.arena + rcode_off(y, sq.slot, a.layer, h, 0, 0));
  const uint16_t* vsrc = sink ? (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, sq.slot, a.layer, h, 1, 0)
                              : (const uint16_t*)(a.arena + rcode_off(y, sq.slot, a.layer, h, 1, 0));
  auto row16 = [&](int t) -> int64_t {
    if (sink) return (int64_t)t * D;
    int sl = sq.ring0 + t;
    sl = sl >= y.cap ? sl - y.cap : sl;
    sl = sl >= y.cap ? sl - y.cap : sl;
    return (int64_t)sl * D;
  };

  float m_run = -INFINITY, m_ref = -INFINITY, l_part = 0.0f;
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
        ks_op[kk] = *(const uint4*)(ksrc + row16(t0 + 16 * wave + q16) + 32 * kk + 8 * g);
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const int it = tid + 256 * j, tq = it % (kStep / 4), c8 = it / (kStep / 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tok = 4 * tq + k;
          r[j][k] = *(const uint4*)(vsrc + row16(t0 + (tok < n ? tok : 0)) + 8 * c8);
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
      const int tq = tid & 15;
#pragma unroll
      for (int u = 0; u < RingRegs<D>::NV; ++u) {
        const int c16 = (tid >> 4) + 16 * u;
        if (c16 < D / 16) {
          uint4 lo8[4], hi8[4];  // channels 16 c16 + 0..7 and + 8..15 of tokens 4 tq + k
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const half8 x0 = codes6_reg(cur.v[u][k][0], cur.v[u][k][1]);
            const half8 x1 =
                codes6_reg(__builtin_amdgcn_alignbit(cur.v[u][k][2], cur.v[u][k][1], 16), cur.v[u][k][2] >> 16);
            __builtin_memcpy(&lo8[k], &x0, 16);
            __builtin_memcpy(&hi8[k], &x1, 16);
          }
          store_t4x8(vt, kRPitch, 16 * c16, 4 * tq, lo8);
          store_t4x8(vt, kRPitch, 16 * c16 + 8, 4 * tq, hi8);
        }
      }
    }

    // ---- (2) scores of tile `wave`
    float4v sacc[NB], saccl[NB];  // hi and (unpacked) scaled-lo products
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) sacc[blk] = saccl[blk] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
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
      if (!PK) saccl[blk] = mfma16(av, mfma_a(qo[kk][1][lane]), saccl[blk]);
    }
    if (PK) {  // lanes l and l ^ 8 both get the hi + lo sum of their column, bit for bit
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[blk][r] = add_x8_lo(sacc[blk][r], lane);
    } else {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) sacc[blk] += saccl[blk] * kLoUnscale;
    }
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * wave + 4 * g + r;
      float v = 0.0f;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
        v = sink ? v + sacc[blk][r] : fmaf(block_scale<D>(cur.dk[r], blk), sacc[blk][r], v);
      v = t < n ? v : -INFINITY;
      sc[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = xmax4(mx);
    if (g == 0) xm[wave][q16] = mx;
    __syncthreads();  // maxima; V^T complete

    // ---- (3) weights
    const float M = fmaxf(fmaxf(xm[0][q16], xm[1][q16]), fmaxf(xm[2][q16], xm[3][q16]));  // token t0 is valid
    // the step's weights are taken relative to m_ref = max(M, running maximum
    // - 24), not to the running maximum itself: the fp16 hi/lo weight operands
    // then stay in the normal range, where their relative precision holds
    // (tokens more than 24 below the running maximum weigh under 2^-24 of it);
    // the accumulators and l are rescaled from the previous reference, by a
    // factor of at most 2^24
    m_run = fmaxf(m_run, M);
    const float m_new = fmaxf(M, m_run - 24.0f);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 on the first step
    m_ref = m_new;
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
      for (int r = 0; r < 4; ++r) x[r] = sink ? p[r] : p[r] * block_scale<D>(cur.dv[r], blk);
      uint2 hi, lo;
      split_h2(x[0], x[1], hi.x, lo.x);
      split_h2(x[2], x[3], hi.y, lo.y);
      if (PK) {
        *(uint2*)(pw + ((blk * 2 + 0) * 16 + q16) * kRPitch + 16 * wave + 4 * g) = q16 < 8 ? hi : lo;
      } else {
        *(uint2*)(pw + ((blk * 2 + 0) * 16 + q16) * kRPitch + 16 * wave + 4 * g) = hi;
        *(uint2*)(pw + ((blk * 2 + 1) * 16 + q16) * kRPitch + 16 * wave + 4 * g) = lo;
      }
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
        acc[i] = mfma16(av, bh, acc[i]);
        if (!PK) {
          const half8 bl = mfma_a(*(const uint4*)(pw + ((blk * 2 + 1) * 16 + q16) * kRPitch + 32 * j + 8 * g));
          acc[i] = mfma16(av, bl, acc[i]);
        }
      }
    }
    __syncthreads();  // V^T and the weights are free
  };
  if (exact) {
    for (int t0 = t_begin; t0 < t_end; t0 += kStep) step(std::true_type{}, t0, ra, rb);
  } else {
    for (int t0 = t_begin;;) {
      step(std::false_type{}, t0, ra, rb);
      if ((t0 += kStep) >= t_end) break;
      step(std::false_type{}, t0, rb, ra);
      if ((t0 += kStep) >= t_end) break;
    }
  }

  if (PK) {  // lo columns into the hi columns
#pragma unroll
    for (int i = 0; i < CPW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] = add_x8(acc[i][e]);
  }
  // partial rows through the V^T area (free after the last step); the sink's
  // sums are in the original domain already
  const float lsum = xsum4(l_part);
  if (g == 0) xl[wave][q16] = lsum;
  float* rows = (float*)vt;
  if (q16 < G) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) *(float4v*)(rows + q16 * D + 16 * (CPW * wave + i) + 4 * g) = acc[i];
  }
  __syncthreads();
  write_partial_rows<D>(a, b, h, c, rows, m_ref, xl, !exact, wave, lane);
}

// ---------------------------------------------------------------------------
// Append role (fused decode step): the token appended in the same call, for
// one (sequence, KV head).  Waves 0 and 1 rotate and encode its key and value
// into the staging ring slot (the same encoder and bytes as the append
// kernel; the ring items of this launch stop short of that slot), keeping the
// decoded rotated-domain values d (u - 32).  The token's split-K partial is
// then exact and needs no scan: for each query head of the group the score
// s = q' . k (scale and log2 e folded into q'), m = s, l = 1, acc = v.
template <int D>
__device__ __forceinline__ void append_role(const DecodeArgs& a, int b, int h, uint8_t* smem) {
  constexpr int VPL = D / 64;  // elements of the dot product per lane
  const Layout& y = a.y;
  const DecodeSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.g;
  float* rows = (float*)smem;  // [16][D] query rows
  float* kv = rows + 16 * D;   // [2][D] decoded key and value
  uint8_t* arena = const_cast<uint8_t*>(a.arena);  // the one region this launch writes
  if (wave < 2 && y.f16ring) {  // f16 staging: the token as it is, in the original domain
    const uint16_t* src = (wave ? a.v_new : a.k_new) + ((int64_t)b * y.H + h) * D;
    uint16_t* dst = (uint16_t*)(arena + rcode_off(y, sq.slot, a.layer, h, wave, sq.app_slot));
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const uint16_t e = src[VPL * lane + j];
      dst[VPL * lane + j] = e;
      kv[D * wave + VPL * lane + j] = h2f(e);
    }
  } else if (wave < 2) {
    const uint16_t* src = (wave ? a.v_new : a.k_new) + ((int64_t)b * y.H + h) * D;
    uint8_t* codes = arena + rcode_off(y, sq.slot, a.layer, h, wave, sq.app_slot);
    uint16_t* scales = (uint16_t*)(arena + rscale_off(y, sq.slot, a.layer, h, wave, sq.app_slot));
    if (D == 128) {
      float deq[2];
      encode_chunk<2>(src, codes, scales, lane, a.signs, true, deq);
#pragma unroll
      for (int j = 0; j < 2; ++j) kv[D * wave + 2 * lane + j] = deq[j];
    } else {
#pragma unroll
      for (int c = 0; c < D / 256; ++c) {
        float deq[4];
        encode_chunk<4>(src + 256 * c, codes + 2 * kQBytes * c, scales + 2 * c, lane, a.signs, false, deq);
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[D * wave + 256 * c + 4 * lane + j] = deq[j];
      }
    }
  }
  QueryRaw<D> qraw;
  query_load<D>(a, b, h, wave, lane, qraw);
  query_rows<D>(a, qraw, !y.f16ring, rows, wave, lane);
  __syncthreads();
  float vo[VPL];  // the value in the original domain: the same accumulator for every query head
#pragma unroll
  for (int j = 0; j < VPL; ++j) vo[j] = kv[D + VPL * lane + j];
  if (!y.f16ring) rotate_back<D>(vo, lane, a.signs);
  for (int i = wave; i < G; i += 4) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s = fmaf(rows[i * D + VPL * lane + j], kv[VPL * lane + j], s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    float* P = a.part + (((int64_t)b * a.Hq + h * G + i) * a.max_chunks + sq.app_chunk) * part_stride(D);
#pragma unroll
    for (int j = 0; j < VPL; ++j) P[kPartHead + VPL * lane + j] = vo[j];
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

template <int D, int KB>
struct MainLds {
  static constexpr int body = BodyShape<D, KB>::total, ring = RingLds<D>::total, append = (16 + 2) * D * 4;
  static constexpr int m0 = body > ring ? body : ring;
  static constexpr int value = m0 > append ? m0 : append;
};

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

template <int D, int KB>
__device__ __forceinline__ void decode_main(const DecodeArgs& a, uint8_t* smem) {
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
    append_role<D>(a, item / a.y.H, item % a.y.H, smem);
    prof_end(a.prof_ts);
    return;
  }
  item -= a.n_app_items;
  if (item < a.n_body_items) {
    if (find_item(a, item, true, b, h, c)) {
      // packed hi/lo products at 256-channel sub-records only: at 128 channels
      // the shorter product chains leave the combine's wait exposed (measured:
      // 27 % slower at 262,144 tokens with 8-bit keys)
      if (BodyShape<D, KB>::SUBW == 256 && a.g <= 8)
        body_role<BodyShape<D, KB>, true>(a, b, h, c, smem);
      else
        body_role<BodyShape<D, KB>, false>(a, b, h, c, smem);
    }
  } else {
    if (find_item(a, item - a.n_body_items, false, b, h, c)) {
      if (D >= 256 && a.g <= 8)
        ring_role<D, true>(a, b, h, c, smem);
      else
        ring_role<D, false>(a, b, h, c, smem);
    }
  }
  prof_end(a.prof_ts);
}

// Low-bit bodies (2- or 3-bit keys and values), 256-wide heads: the same
// items, the body scanned by body_role_lb.
template <int KB, int VB>
struct MainLdsLb {
  static constexpr int body = LbShape<KB, VB>::total, ring = RingLds<256>::total, append = (16 + 2) * 256 * 4;
  static constexpr int m0 = body > ring ? body : ring;
  static constexpr int value = m0 > append ? m0 : append;
};

template <int KB, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_main_kernel_lb(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[MainLdsLb<KB, VB>::value];
  int b, h, c;
  int item = blockIdx.x;
  prof_start(a.prof_ts);
  if (item < a.n_app_items) {
    append_role<256>(a, item / a.y.H, item % a.y.H, smem);
    prof_end(a.prof_ts);
    return;
  }
  item -= a.n_app_items;
  if (item < a.n_body_items) {
    if (find_item(a, item, true, b, h, c)) body_role_lb<LbShape<KB, VB>>(a, b, h, c, smem);
  } else if (find_item(a, item - a.n_body_items, false, b, h, c)) {
    if (a.g <= 8)
      ring_role<256, true>(a, b, h, c, smem);
    else
      ring_role<256, false>(a, b, h, c, smem);
  }
  prof_end(a.prof_ts);
}

// Two resident workgroups per compute unit (256 registers per lane each),
// or one for 512-wide heads (whose sink/ring scan needs 125 KB of LDS).
#define KVQ_MAIN_KERNEL(NAME, D, KB, W)                                                      \
  __global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W))) void NAME(DecodeArgs a) { \
    __shared__ __attribute__((aligned(1024))) uint8_t smem[MainLds<D, KB>::value];           \
    decode_main<D, KB>(a, smem);                                                             \
  }
KVQ_MAIN_KERNEL(decode_main_kernel, 256, 4, 2)
KVQ_MAIN_KERNEL(decode_main_kernel_d128k8, 128, 8, 2)
KVQ_MAIN_KERNEL(decode_main_kernel_d512, 512, 4, 1)
KVQ_MAIN_KERNEL(decode_main_kernel_d128k4, 128, 4, 2)
KVQ_MAIN_KERNEL(decode_main_kernel_d256k8, 256, 8, 2)
KVQ_MAIN_KERNEL(decode_main_kernel_d512k8, 512, 8, 1)
#undef KVQ_MAIN_KERNEL
static_assert(BodyShape<512, 4>::WG_PER_CU == 1 && BodyShape<512, 8>::WG_PER_CU == 1 &&
                  BodyShape<256, 4>::WG_PER_CU == 2 && BodyShape<256, 8>::WG_PER_CU == 2 &&
                  BodyShape<128, 4>::WG_PER_CU == 2 && BodyShape<128, 8>::WG_PER_CU == 2,
              "launch bounds match the body shapes");

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_ring_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RingLds<D>::total];
  int b, h, c;
  if (find_item(a, blockIdx.x, false, b, h, c)) {
    if (D >= 256 && a.g <= 8)
      ring_role<D, true>(a, b, h, c, smem);
    else
      ring_role<D, false>(a, b, h, c, smem);
  }
}

// Append (optional), body and sink/ring items in one launch: head_dim 128,
// 256 or 512 (two 256-channel sub-records), 4- or 8-bit keys, 4-bit values.
hipError_t launch_decode_main(const DecodeArgs& a, int n_items, hipStream_t stream) {
  if (a.ring_chunk % kStep != 0 || a.g > kMaxGroup) return hipErrorInvalidValue;
  const dim3 grid(n_items), block(256);
  if (a.y.vbits != 4) {  // low-bit bodies: 256-wide heads, 2- or 3-bit keys and values
    if (a.y.D != 256) return hipErrorInvalidValue;
    const int kb = a.y.kbits, vb = a.y.vbits;
    if (kb == 3 && vb == 3)
      hipLaunchKernelGGL((decode_main_kernel_lb<3, 3>), grid, block, 0, stream, a);
    else if (kb == 3 && vb == 2)
      hipLaunchKernelGGL((decode_main_kernel_lb<3, 2>), grid, block, 0, stream, a);
    else if (kb == 2 && vb == 2)
      hipLaunchKernelGGL((decode_main_kernel_lb<2, 2>), grid, block, 0, stream, a);
    else if (kb == 2 && vb == 3)
      hipLaunchKernelGGL((decode_main_kernel_lb<2, 3>), grid, block, 0, stream, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.y.D == 256 && a.y.kbits == 4)
    hipLaunchKernelGGL(decode_main_kernel, grid, block, 0, stream, a);
  else if (a.y.D == 512 && a.y.kbits == 4)
    hipLaunchKernelGGL(decode_main_kernel_d512, grid, block, 0, stream, a);
  else if (a.y.D == 128 && a.y.kbits == 8)
    hipLaunchKernelGGL(decode_main_kernel_d128k8, grid, block, 0, stream, a);
  else if (a.y.D == 128 && a.y.kbits == 4)
    hipLaunchKernelGGL(decode_main_kernel_d128k4, grid, block, 0, stream, a);
  else if (a.y.D == 256 && a.y.kbits == 8)
    hipLaunchKernelGGL(decode_main_kernel_d256k8, grid, block, 0, stream, a);
  else if (a.y.D == 512 && a.y.kbits == 8)
    hipLaunchKernelGGL(decode_main_kernel_d512k8, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
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
