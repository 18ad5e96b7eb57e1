// Block attention on the matrix cores: the queries of the newest n_q cached
// tokens of each sequence (a prefill chunk whose keys and values were appended
// first, or a speculative verify block), each seeing every cached token up to
// its own position, whichever region holds it.
//
// HAL #582 section 3b measures prefill over the same quantised caches (a
// small prefill cost at head_dim 128, a large matrix-core dequantisation cost
// at 512-wide heads); SJ-KVaRN 2.1: one pass reads sink, ring and body; KV
// Cache Precision Tail section 2: one softmax over all regions.
//
// The record and ring math is the decode kernels' (the query rotated once;
// body codes and 6-bit ring codes enter the products as exact centred
// integers; per-token and per-channel scales applied outside the products).
// The query side differs: a work item takes a row block of 16 NT query rows
// (row r = t g + e: token t of the block, query head e of the KV head's
// group), so every key and value code loaded and unpacked once feeds NT
// products instead of one.  Split-K as in decode: a work item is (sequence,
// KV head, row block, chunk), the chunk being the sink, a run of ring tokens
// or a run of records; it writes one partial row per query row and the merge
// combines a row's partials.
//
// Causal mask: the key at position p is seen by the rows of tokens at
// positions >= p.  A masked score takes a finite sentinel and weight 0; a row
// with no visible key in a chunk writes m = sentinel, l = 0, acc = 0.
//
// Precision: as in decode, the query operand of the scores and the weights
// of the value product are split into hi + lo fp16 (two products each), so
// both keep fp32-level precision.  With one fp16 weight per token (relative
// rounding up to 2^-12) the outputs of attention spread over thousands of
// tokens were off by up to ~2e-3 of their RMS (measured): the output shrinks
// like 1/sqrt(tokens) while the rounding errors of the weights do not average
// faster.
#include "kvq_codes.h"

namespace kvq {

namespace {

constexpr float kMaskedScore = -1.0e30f;  // log2 units: exp2 of it, or of it minus a real maximum, is 0
constexpr int kBStep = 64;                // sink / ring tokens per step
constexpr int kBPitch = kBStep + 8;       // halves per V^T / weight row of a step (padding spreads LDS banks)

// This workgroup's item.  Workgroups are dealt to the 8 XCDs round-robin
// (workgroup x to XCD x mod 8); item (x mod 8) (grid / 8) + x / 8 puts
// consecutive items -- the row blocks of one (sequence, KV head, chunk), which
// read the same codes -- on one XCD and its L2.  The grid is a multiple of 8.
__device__ __forceinline__ int block_item() {
  const int per = (int)gridDim.x / 8;
  return (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
}

__device__ __forceinline__ int find_seq(const PrefillArgs& a, int item, bool body) {
  int b = 0;
  while (b + 1 < a.n_seqs && (body ? a.seq[b + 1].body_item0 : a.seq[b + 1].ring_item0) <= item) ++b;
  return b;
}

// Query rows row0 .. row0 + nrows - 1 of the block (rows past its end zero)
// into rows[nrows][D] fp32, times scale log2 e, rotated (R = H/16 per 256-point
// half; s2 . H . s1 / sqrt(128) for 128-wide heads) or not.  Wave w of NW takes
// rows w, w + NW, ...; the caller synchronises before reading.
template <int D, int NW>
__device__ __forceinline__ void block_query_rows(const PrefillArgs& a, int b, int h, int row0, int nrows, bool rotate,
                                                 float* rows) {
  constexpr int VPL = D / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float sl = a.scale * kLog2e;
  const int n_rows = a.n_q * a.g;
  for (int i = wave; i < nrows; i += NW) {
    const int rr = row0 + i;
    float v[VPL];
    if (rr < n_rows) {
      const int t = rr / a.g, e = rr - t * a.g;
      const uint32_t* src = (const uint32_t*)(a.q + (((int64_t)b * a.n_q + t) * a.Hq + h * a.g + e) * D + VPL * lane);
#pragma unroll
      for (int w = 0; w < VPL / 2; ++w) {
        const half2v x = as_h2(src[w]);
        v[2 * w] = (float)x[0] * sl;
        v[2 * w + 1] = (float)x[1] * sl;
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) v[j] = 0.0f;
    }
    if (rotate) {
      if (D == 128) {
#pragma unroll
        for (int j = 0; j < VPL; ++j)
          if (sign_neg(a.signs, VPL * lane + j)) v[j] = -v[j];
      }
      wave_fwht<VPL, D == 128 ? 128 : 256>(v, lane);
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

// Partial rows of a work item: rows[RB][D] fp32 in LDS (the accumulators,
// rotated-domain when `rotate`), mrow[RB] the rows' maxima (log2 units),
// lrow[NW][RB] the waves' parts of l.  Wave w writes rows w, w + NW, ... that
// lie in the block.  The caller synchronises after filling the LDS arrays.
template <int D, int NW>
__device__ __forceinline__ void write_block_partials(const PrefillArgs& a, int b, int h, int rb, int RB, int chunk,
                                                     const float* rows, const float* mrow, const float* lrow,
                                                     bool rotate) {
  constexpr int VPL = D / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_rows = a.n_q * a.g;
  for (int i = wave; i < RB; i += NW) {
    const int rr = rb * RB + i;
    if (rr >= n_rows) break;
    const int t = rr / a.g, e = rr - t * a.g;
    float v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] = rows[i * D + VPL * lane + j];
    if (rotate) rotate_back<D>(v, lane, a.signs);
    float* P = a.part + ((((int64_t)b * a.n_q + t) * a.Hq + h * a.g + e) * a.max_chunks + chunk) * part_stride(D);
    float* dst = P + kPartHead + VPL * lane;
    if constexpr (VPL == 2) {
      *(float2*)dst = make_float2(v[0], v[1]);
    } else {
#pragma unroll
      for (int j = 0; j < VPL; j += 4) *(float4*)(dst + j) = make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]);
    }
    if (lane == 0) {
      float l = 0.0f;
      for (int w = 0; w < NW; ++w) l += lrow[w * RB + i];
      P[0] = fmaxf(mrow[i], kMaskedScore) * kLn2;
      P[1] = l;
    }
  }
}

// A chunk none of whose keys any row of the block sees: (sentinel, 0, 0) rows.
template <int D, int NW>
__device__ __forceinline__ void write_empty_partials(const PrefillArgs& a, int b, int h, int rb, int RB, int chunk) {
  constexpr int VPL = D / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_rows = a.n_q * a.g;
  for (int i = wave; i < RB; i += NW) {
    const int rr = rb * RB + i;
    if (rr >= n_rows) break;
    const int t = rr / a.g, e = rr - t * a.g;
    float* P = a.part + ((((int64_t)b * a.n_q + t) * a.Hq + h * a.g + e) * a.max_chunks + chunk) * part_stride(D);
#pragma unroll
    for (int j = 0; j < VPL; ++j) P[kPartHead + VPL * lane + j] = 0.0f;
    if (lane == 0) {
      P[0] = kMaskedScore * kLn2;
      P[1] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Body role: one run of records of one KV head for one row block.
//
// Record shapes as in decode: NSUB sub-records of SUBW channels (256; 128 for
// 128-wide heads; a 512-wide head is two 256-channel halves), 4- or 8-bit
// keys, 4-bit values, each sub-record with its own C, S, Z.  NW waves (4, or 8
// for 64-row blocks: two waves per SIMD, so that one wave's softmax overlaps
// another's products):
//   q~:     thread (wave w, lane (n, g)) owns the operand units
//           (s, kk, t) = w + NW u (t fastest, then kk): row 16 t + n, the 8
//           slots lane group g feeds at k-step kk of sub-record s.  Their q'
//           (rotated query, hi + lo) stays in registers; per record the thread
//           multiplies in the key C and stores q~ hi, lo to LDS;
//   scores: wave w takes the 16-token tiles TPW w .. (8 / NW of them) against
//           every row tile; a lane's key share is CPL contiguous channels of a
//           token row (k-step kk: channels CPL g + 8 kk ..).  The lo products
//           take the key operand times 2^-11 (exact) and share the hi
//           products' accumulator;
//   values: wave w takes SUBW / (16 NW) channel tiles of each sub-record
//           against every row tile, over the record's 128 tokens.
// With 4-bit values the token order inside a 16-token tile (position P holds
// token (P & ~7) + [0, 4, 1, 5, 2, 6, 3, 7][P & 7]) and the 1/16 of
// high-nibble slots are the decode kernel's: a lane's four score rows are four
// consecutive slots of the value product's operand.  The 2- and 3-bit bodies
// (SJ-KVaRN 2.3: 3/3, 3/2; and 2/2, 2/3) take natural order instead (NAT):
// position P holds token P, k-step kk of a key row feeds channels
// CPL g + 8 kk .. in order, and the codes are unpacked from the b-bit row
// streams (codes_lb), as the decode's low-bit scan does.  Two barriers per
// record.
template <int D_, int KB_, int VB_, int NT_, int NW_>
struct PBody {
  static constexpr int D = D_, KB = KB_, VB = VB_, NT = NT_, NW = NW_, RB = 16 * NT_, NTH = 64 * NW_;
  static constexpr bool NAT = VB != 4;
  static constexpr int SUBW = D == 128 ? 128 : 256, NSUB = D / SUBW;
  static constexpr int KK = SUBW / 32;       // score k-steps per sub-record
  static constexpr int CPL = SUBW / 4;       // key channels per lane group
  static constexpr int KW = CPL * KB / 32;   // dwords of a lane's key-row share
  static constexpr int TPW = 8 / NW;         // 16-token score tiles per wave
  static constexpr int VT = SUBW / 16 / NW;  // value channel tiles per wave and sub-record
  static constexpr int ROWB = SUBW * KB / 8, VROW = 128 * VB / 8;  // bytes per key / value code row
  static constexpr int VW = VB;                                       // dwords of a lane's value-row share
  static constexpr int KCODE = 128 * ROWB, VCODE = SUBW * VROW;
  static constexpr int META = 4 * (SUBW + 256);
  static constexpr int SUB_BYTES = KCODE + VCODE + META;
  static constexpr int L_KS = 2 * SUBW, L_KZ = L_KS + 512, L_VC = L_KZ + 512, L_VS = L_VC + 4 * SUBW;
  static constexpr int L_VZ = L_VS + 512, MSTRIDE = 4096;
  static constexpr int UNITS = NSUB * KK * NT / NW;  // q~ operand units per thread
  // OWN: every unit of a thread is in row tile wave mod NT (NT divides NW), so
  // a row tile's sigma parts come from its NW / NT owning waves; otherwise
  // (three row tiles over eight waves) unit idx is in row tile idx mod NT and
  // every wave writes a part (zero where it has no unit) for every row tile
  static constexpr bool OWN = NW % NT == 0;
  // LDS: q~ [NSUB][KK][NT][hi, lo][64] uint4; weights [NSUB][hi, lo][RB][kPPitch]
  // halves; scales [3][NSUB][MSTRIDE]; per-row exchange of the waves' parts
  // (a row's NW parts contiguous, read as 16-byte vectors): xm[RB][NW],
  // xz[NSUB][RB][NW], xs[NSUB][RB][NW] floats
  static constexpr int kPPitch = 128 + 8;
  static constexpr int QT = 0, PW = QT + NSUB * KK * NT * 2 * 1024;
  static constexpr int MB = PW + NSUB * 2 * RB * kPPitch * 2;
  static constexpr int X = MB + 3 * NSUB * MSTRIDE;
  static constexpr int total = X + (1 + 2 * NSUB) * NW * RB * 4;
  static_assert(NT >= 1 && NT <= 4 && (OWN || NW == 8), "row tiles per block");
  static_assert(UNITS >= 1 && UNITS * NW == NSUB * KK * NT, "q~ units divide over the workgroup");
  static_assert(TPW * NW == 8 && VT * NW * 16 == SUBW, "tiles divide over the waves");
  static_assert(RB * D * 4 <= PW - QT, "query rows (and the partial rows) fit the q~ area");
  static_assert(KW % 2 == 0 && (!NAT || (SUBW == 256 && KB <= 3)), "key shares load as 8-byte pieces");
  static_assert(L_VZ + 512 <= MSTRIDE && META <= 8 * 256, "scales of a sub-record fit one LDS area");
  static __device__ __forceinline__ int kslot(int j) { return KB == 4 ? (j >> 1) + 4 * (j & 1) : j; }
  static __device__ __forceinline__ float kfac(int j) { return KB == 4 && (j & 2) ? 0.0625f : 1.0f; }
  // tile position of a lane's score row jj (lane group g): token tok_base(g) + tok_off(jj)
  static __device__ __forceinline__ int tok_base(int g) { return NAT ? 4 * g : 8 * (g >> 1) + 2 * (g & 1); }
  static __device__ __forceinline__ int tok_off(int jj) { return NAT ? jj : (jj >> 1) + 4 * (jj & 1); }
};

template <class Sh>
__device__ __forceinline__ void pb_load_keys(const uint8_t* __restrict__ sub, uint32_t (&kd)[Sh::TPW][Sh::KW],
                                             int wave, int lane, bool dummy) {
  const int m = lane & 15, g = lane >> 4;
  // position m of the tile holds this token
  const int row = Sh::NAT ? m : (m & 8) + ((m & 7) >> 1) + 4 * (m & 1);
#pragma unroll
  for (int i = 0; i < Sh::TPW; ++i) {
    const uint8_t* p = sub + (dummy ? 0 : (16 * (Sh::TPW * wave + i) + row) * Sh::ROWB + Sh::CPL * Sh::KB / 8 * g);
    if constexpr (Sh::KW % 4 == 0) {
#pragma unroll
      for (int s = 0; s < Sh::KW / 4; ++s) {
        const uint4 v = *(const uint4*)(p + 16 * s);
        kd[i][4 * s] = v.x;
        kd[i][4 * s + 1] = v.y;
        kd[i][4 * s + 2] = v.z;
        kd[i][4 * s + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int s = 0; s < Sh::KW / 2; ++s) {
        const uint2 v = *(const uint2*)(p + 8 * s);
        kd[i][2 * s] = v.x;
        kd[i][2 * s + 1] = v.y;
      }
    }
  }
}
template <class Sh>
__device__ __forceinline__ void pb_load_values(const uint8_t* __restrict__ sub, uint32_t (&vd)[Sh::VT][Sh::VW],
                                               int wave, int lane, bool dummy) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < Sh::VT; ++j) {
    const uint8_t* p = sub + (dummy ? 0 : Sh::KCODE + (16 * (Sh::VT * wave + j) + m) * Sh::VROW + 4 * Sh::VB * g);
    if constexpr (Sh::VW == 4) {
      const uint4 v = *(const uint4*)p;
      vd[j][0] = v.x;
      vd[j][1] = v.y;
      vd[j][2] = v.z;
      vd[j][3] = v.w;
    } else {
#pragma unroll
      for (int k = 0; k < Sh::VW; ++k) vd[j][k] = ((const uint32_t*)p)[k];
    }
  }
}

// Key operand of a token tile at k-step kk, value operand of a channel tile
// at k-step tt (exact centred fp16).
template <class Sh>
__device__ __forceinline__ half8 pb_key_op(const uint32_t (&kd)[Sh::KW], int kk) {
  if constexpr (Sh::KB == 4) {
    return nib8_centred(kd[kk]);
  } else if constexpr (Sh::KB == 8) {
    return byte8_centred(kd[2 * kk], kd[2 * kk + 1]);
  } else {
    return codes_lb<Sh::KB>(step_bits<Sh::KB>(kd, kk));
  }
}
template <class Sh>
__device__ __forceinline__ half8 pb_value_op(const uint32_t (&vd)[Sh::VW], int tt) {
  if constexpr (Sh::VB == 4) {
    return nib8_centred(vd[tt]);
  } else {
    return codes_lb<Sh::VB>(step_bits<Sh::VB>(vd, tt));
  }
}

// q~ = q' C of this thread's units for the record whose scales sit at km
// (NSUB areas of MSTRIDE), into the q~ area; sigma = sum_j q~_j of each
// sub-record's rows: this wave's part, in xs[s][row][wave].
template <class Sh>
__device__ __forceinline__ void pb_make_qtilde(const uint8_t* km, const uint4 (&qh)[Sh::UNITS],
                                               const uint4 (&ql)[Sh::UNITS], uint4* qt, float* xs, int wave, int lane) {
  constexpr int NT = Sh::NT, KK = Sh::KK, NSUB = Sh::NSUB, RB = Sh::RB, NW = Sh::NW;
  const int n = lane & 15, g = lane >> 4;
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  const half2v lo_ones = {(_Float16)kLoUnscale, (_Float16)kLoUnscale};
  constexpr int NTS = Sh::OWN ? 1 : NT;  // sigma parts per sub-record this thread keeps
  float sig[NSUB][NTS];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int t = 0; t < NTS; ++t) sig[s][t] = 0.0f;
#pragma unroll
  for (int u = 0; u < Sh::UNITS; ++u) {
    const int idx = wave + NW * u, kk = (idx / NT) % KK, s = idx / (NT * KK);
    const int t = Sh::OWN ? wave % NT : idx % NT;
    const uint4 c = *(const uint4*)(km + s * Sh::MSTRIDE + 2 * (Sh::CPL * g + 8 * kk));
    uint32_t cp[4];
    if constexpr (Sh::KB == 4) {  // slot pairs (c0, c4), (c1, c5), (c2, c6), (c3, c7)
      cp[0] = __builtin_amdgcn_perm(c.z, c.x, 0x05040100u);
      cp[1] = __builtin_amdgcn_perm(c.z, c.x, 0x07060302u);
      cp[2] = __builtin_amdgcn_perm(c.w, c.y, 0x05040100u);
      cp[3] = __builtin_amdgcn_perm(c.w, c.y, 0x07060302u);
    } else {
      cp[0] = c.x;
      cp[1] = c.y;
      cp[2] = c.z;
      cp[3] = c.w;
    }
    uint4 hi, lo;
    qtilde_pair(qh[u].x, ql[u].x, cp[0], hi.x, lo.x);
    qtilde_pair(qh[u].y, ql[u].y, cp[1], hi.y, lo.y);
    qtilde_pair(qh[u].z, ql[u].z, cp[2], hi.z, lo.z);
    qtilde_pair(qh[u].w, ql[u].w, cp[3], hi.w, lo.w);
    float a1 = 0.0f, a16 = 0.0f;  // 4-bit keys: slots y and w carry 1/16
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.x), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.x), lo_ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.y), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.y), lo_ones, a16, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(hi.z), ones, a1, false);
    a1 = __builtin_amdgcn_fdot2(as_h2(lo.z), lo_ones, a1, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(hi.w), ones, a16, false);
    a16 = __builtin_amdgcn_fdot2(as_h2(lo.w), lo_ones, a16, false);
    sig[s][Sh::OWN ? 0 : t] += Sh::KB == 4 ? fmaf(16.0f, a16, a1) : a1 + a16;
    uint4* dst = qt + (((s * KK + kk) * NT + t) * 2) * 64 + lane;
    dst[0] = hi;
    dst[64] = lo;
  }
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int tt = 0; tt < NTS; ++tt) {
      const int t = Sh::OWN ? wave % NT : tt;
      const float v = xsum4(sig[s][tt]);
      if (g == 0) xs[(s * RB + 16 * t + n) * NW + wave] = v;
    }
}

template <class Sh>
__device__ __forceinline__ void body_block(const PrefillArgs& a, int b, int h, int rb, int cbk, uint8_t* smem) {
  constexpr int D = Sh::D, SUBW = Sh::SUBW, NSUB = Sh::NSUB, KK = Sh::KK, VT = Sh::VT, NT = Sh::NT, RB = Sh::RB;
  constexpr int NW = Sh::NW, TPW = Sh::TPW, SB = Sh::SUB_BYTES, MS = Sh::MSTRIDE, U = Sh::UNITS, KW = Sh::KW;
  constexpr int PP = Sh::kPPitch;
  constexpr float kMid = (float)(1 << (Sh::KB - 1));
  const Layout& y = a.y;
  const PrefillSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  uint4* qt = (uint4*)(smem + Sh::QT);
  uint16_t* pw = (uint16_t*)(smem + Sh::PW);  // [NSUB][hi, lo][RB][PP]
  uint8_t* mbuf = smem + Sh::MB;
  float* xm = (float*)(smem + Sh::X);            // [RB][NW]
  float* xz = xm + NW * RB;                      // [NSUB][RB][NW]
  float* xs = xz + NSUB * NW * RB;               // [NSUB][RB][NW]
  // sum / maximum of a row's NW parts (16-byte reads)
  auto sum_nw = [&](const float* p) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; k += 4) {
      const float4 q = *(const float4*)(p + k);
      v += (q.x + q.y) + (q.z + q.w);
    }
    return v;
  };
  auto max_nw = [&](const float* p) {
    float v = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; k += 4) {
      const float4 q = *(const float4*)(p + k);
      v = fmaxf(v, fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)));
    }
    return v;
  };

  const int chunk = 1 + sq.n_ring_chunks + cbk;
  const int r0 = (int)((int64_t)cbk * sq.n_rec / sq.n_body_chunks);
  const int r1 = (int)((int64_t)(cbk + 1) * sq.n_rec / sq.n_body_chunks);
  const int n_rows = a.n_q * a.g, row0 = rb * RB;
  const int pmin = sq.p0 + row0 / a.g;
  const int pmax = sq.p0 + (min(n_rows, row0 + RB) - 1) / a.g;
  if (r1 <= r0 || kSink + kGroup * r0 > pmax) {
    write_empty_partials<D, NW>(a, b, h, rb, RB, chunk);
    return;
  }
  int prow[NT];  // positions of this lane's rows (16 t + n); -1 past the block
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rr = row0 + 16 * t + n;
    prow[t] = rr < n_rows ? sq.p0 + rr / a.g : -1;
  }

  const uint8_t* rec0 = a.arena + rec_off(y, sq.slot, a.layer, h, 0);
  auto rec = [&](int r) { return rec0 + (int64_t)r * y.rec_bytes; };
  auto mslot = [&](int r) { return mbuf + ((r - r0) % 3) * (NSUB * MS); };
  // the first 256 threads stage the scales, 8 bytes each (clamped: threads
  // past the end re-read the last 8 bytes and store them where nothing reads)
  const bool stager = tid < 256;
  const int mo = Sh::KCODE + Sh::VCODE + min(8 * (tid & 255), Sh::META - 8);

  // ---- prologue: scales of r0, r0 + 1 and the keys of r0 in flight while the
  // query rows are rotated into the q~ area and split into this thread's units
  uint2 m0[NSUB], m1[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    m0[s] = *(const uint2*)(rec(r0) + s * SB + mo);
    m1[s] = *(const uint2*)(r0 + 1 < r1 ? rec(r0 + 1) + s * SB + mo : rec0);
  }
  uint32_t kd[NSUB][TPW][KW], vd[NSUB][VT][Sh::VW];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) pb_load_keys<Sh>(rec(r0) + s * SB, kd[s], wave, lane, false);
  float* rows = (float*)qt;
  block_query_rows<D, NW>(a, b, h, row0, RB, true, rows);
  __syncthreads();
  uint4 qh[U], ql[U];
  {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = wave + NW * u, kk = (idx / NT) % KK, s = idx / (NT * KK);
      const int t = Sh::OWN ? wave % NT : idx % NT;
      const float* rp = rows + (16 * t + n) * D + SUBW * s + Sh::CPL * g + 8 * kk;
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const int j0 = 2 * pr, j1 = 2 * pr + 1;
        split_h2s(rp[Sh::kslot(j0)] * Sh::kfac(j0), rp[Sh::kslot(j1)] * Sh::kfac(j1), hb[pr], lb[pr]);
      }
      qh[u] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
      ql[u] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
    }
  }
  __syncthreads();  // the query rows are read: the q~ area is free
  if (stager) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      stage_scales<Sh>(mslot(r0) + s * MS, m0[s], tid);
      if (r0 + 1 < r1) stage_scales<Sh>(mslot(r0 + 1) + s * MS, m1[s], tid);
    }
  }
  __syncthreads();
  pb_make_qtilde<Sh>(mslot(r0), qh, ql, qt, xs, wave, lane);
#pragma unroll
  for (int s = 0; s < NSUB; ++s) pb_load_values<Sh>(rec(r0) + s * SB, vd[s], wave, lane, false);
  uint2 mnext[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) mnext[s] = *(const uint2*)(r0 + 2 < r1 ? rec(r0 + 2) + s * SB + mo : rec0);
  __syncthreads();

  float m_run[NT], l_part[NT];
  float4v acc[NSUB][VT][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_part[t] = 0.0f;
  }
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int j = 0; j < VT; ++j)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[s][j][t] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  // this lane's score rows are tile positions 4 g + j: tokens tb + {0, 4, 1, 5}
  const int tb = Sh::tok_base(g);
  const half2v lo_a = {(_Float16)kLoUnscale, (_Float16)kLoUnscale};

  for (int r = r0; r < r1; ++r) {
    const uint8_t* mr = mslot(r);
    const bool more = r + 1 < r1;
    const bool masked = kSink + kGroup * r + kGroup - 1 > pmin;  // some key of the record is after some row

    // ---- scores of this wave's tiles against every row tile
    float sc[TPW][NT][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      float4v sh[TPW][NT];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) sh[i][t] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        half8 av[TPW], al[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          av[i] = pb_key_op<Sh>(kd[s][i], kk);
          const half2v* p = (const half2v*)&av[i];
          half2v q[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = p[e] * lo_a;  // exact: small integers times 2^-11
          __builtin_memcpy(&al[i], q, 16);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4* op = qt + (((s * KK + kk) * NT + t) * 2) * 64 + lane;
          const half8 bh = mfma_a(op[0]), bl = mfma_a(op[64]);
#pragma unroll
          for (int i = 0; i < TPW; ++i) sh[i][t] = mfma16(av[i], bh, sh[i][t]);
#pragma unroll
          for (int i = 0; i < TPW; ++i) sh[i][t] = mfma16(al[i], bl, sh[i][t]);
        }
      }
      const uint8_t* km = mr + s * MS;
      float zc[TPW][4], Sk[TPW][4];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int T = 16 * (TPW * wave + i) + tb;
        float Zk[4];
        if constexpr (Sh::NAT) {  // tokens T .. T + 3
          const float4 s4 = *(const float4*)(km + Sh::L_KS + 4 * T), z4 = *(const float4*)(km + Sh::L_KZ + 4 * T);
          Sk[i][0] = s4.x;
          Sk[i][1] = s4.y;
          Sk[i][2] = s4.z;
          Sk[i][3] = s4.w;
          Zk[0] = z4.x;
          Zk[1] = z4.y;
          Zk[2] = z4.z;
          Zk[3] = z4.w;
        } else {  // tokens T + {0, 4, 1, 5}
          const float2 s01 = *(const float2*)(km + Sh::L_KS + 4 * T), s45 = *(const float2*)(km + Sh::L_KS + 4 * T + 16);
          const float2 z01 = *(const float2*)(km + Sh::L_KZ + 4 * T), z45 = *(const float2*)(km + Sh::L_KZ + 4 * T + 16);
          Sk[i][0] = s01.x;
          Sk[i][1] = s45.x;
          Sk[i][2] = s01.y;
          Sk[i][3] = s45.y;
          Zk[0] = z01.x;
          Zk[1] = z45.x;
          Zk[2] = z01.y;
          Zk[3] = z45.y;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) zc[i][j] = fmaf(kMid, Sk[i][j], Zk[j]);  // Z + mid S: exact
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // sigma of row tile t: the parts of the waves w = t mod NT, which own its
        // units (OWN), or of every wave
        const float* xr = xs + (s * RB + 16 * t + n) * NW;
        float sig = 0.0f;
        if constexpr (Sh::OWN) {
#pragma unroll
          for (int w = t; w < NW; w += NT) sig += xr[w];
        } else {
          sig = sum_nw(xr);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = fmaf(Sk[i][j], sh[i][t][j], zc[i][j] * sig);
            sc[i][t][j] = s == 0 ? v : sc[i][t][j] + v;
          }
      }
    }
    if (masked) {
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pos = kSink + kGroup * r + 16 * (TPW * wave + i) + tb + Sh::tok_off(j);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (pos > prow[t]) sc[i][t][j] = -INFINITY;
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float mx = sc[0][t][0];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[i][t][j]);
      mx = xmax4(mx);
      if (g == 0) xm[(16 * t + n) * NW + wave] = mx;
    }
    __syncthreads();  // (B2) record maxima; q~ of r and the key codes are free
#pragma unroll
    for (int s = 0; s < NSUB; ++s) pb_load_keys<Sh>(more ? rec(r + 1) + s * SB : rec0, kd[s], wave, lane, !more);

    float frec[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row = 16 * t + n;
      // a row that sees no key of the record: weights exp2(-inf) = 0
      const float mrec = fmaxf(max_nw(xm + row * NW), kMaskedScore);
      const float m_new = fmaxf(m_run[t], mrec);
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_new);  // 0 on the first record
      frec[t] = __builtin_amdgcn_exp2f(mrec - m_new);
      m_run[t] = m_new;
      if (alpha != 1.0f) {  // skipped by every lane whose maximum held
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
          for (int j = 0; j < VT; ++j) acc[s][j][t] *= alpha;
      }
      // the record's weights are taken relative to its own maximum, so that the
      // fp16 hi/lo weight operands of its significant tokens stay normal; its
      // value sums enter the running ones times 2^(mrec - m_new) <= 1
      float lrec = 0.0f;
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(sc[i][t][j] - mrec);
          sc[i][t][j] = p;  // the weight from here on
          lrec += p;
        }
      l_part[t] = fmaf(frec[t], lrec, l_part[t] * alpha);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const uint8_t* vm = mr + s * MS;
      float zt[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) zt[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int T = 16 * (TPW * wave + i) + tb;
        constexpr float kMidV = (float)(1 << (Sh::VB - 1));
        float Sj[4], zc[4];
        if constexpr (Sh::NAT) {  // tokens T .. T + 3
          const float4 s4 = *(const float4*)(vm + Sh::L_VS + 4 * T), z4 = *(const float4*)(vm + Sh::L_VZ + 4 * T);
          Sj[0] = s4.x;
          Sj[1] = s4.y;
          Sj[2] = s4.z;
          Sj[3] = s4.w;
          zc[0] = fmaf(kMidV, s4.x, z4.x);
          zc[1] = fmaf(kMidV, s4.y, z4.y);
          zc[2] = fmaf(kMidV, s4.z, z4.z);
          zc[3] = fmaf(kMidV, s4.w, z4.w);
        } else {  // tokens T + {0, 4, 1, 5}
          const float2 s01 = *(const float2*)(vm + Sh::L_VS + 4 * T), s45 = *(const float2*)(vm + Sh::L_VS + 4 * T + 16);
          const float2 z01 = *(const float2*)(vm + Sh::L_VZ + 4 * T), z45 = *(const float2*)(vm + Sh::L_VZ + 4 * T + 16);
          // odd tokens sit in the high nibbles: their slots (2 and 3 here) carry 1/16
          Sj[0] = s01.x;
          Sj[1] = s45.x;
          Sj[2] = s01.y * 0.0625f;
          Sj[3] = s45.y * 0.0625f;
          zc[0] = fmaf(kMidV, s01.x, z01.x);
          zc[1] = fmaf(kMidV, s45.x, z45.x);
          zc[2] = fmaf(kMidV, s01.y, z01.y);
          zc[3] = fmaf(kMidV, s45.y, z45.y);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            zt[t] = fmaf(sc[i][t][j], zc[j], zt[t]);
            x[j] = sc[i][t][j] * Sj[j];
          }
          uint2 hi, lo;
          split_h2(x[0], x[1], hi.x, lo.x);
          split_h2(x[2], x[3], hi.y, lo.y);
          uint16_t* dst = pw + ((2 * s) * RB + 16 * t + n) * PP + 16 * (TPW * wave + i) + 4 * g;
          *(uint2*)dst = hi;
          *(uint2*)(dst + RB * PP) = lo;
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v = xsum4(zt[t]);
        if (g == 0) xz[(s * RB + 16 * t + n) * NW + wave] = v;
      }
    }
    if (more) pb_make_qtilde<Sh>(mslot(r + 1), qh, ql, qt, xs, wave, lane);
    if (stager) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (r + 2 < r1) stage_scales<Sh>(mslot(r + 2) + s * MS, mnext[s], tid);
        mnext[s] = *(const uint2*)(r + 3 < r1 ? rec(r + 3) + s * SB + mo : rec0);
      }
    }
    __syncthreads();  // (B3) weights, zero-point sums; q~ and scales of r + 1, r + 2

#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      half8 av[VT][4];
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) av[j][tt] = pb_value_op<Sh>(vd[s][j], tt);
      pb_load_values<Sh>(more ? rec(r + 1) + s * SB : rec0, vd[s], wave, lane, !more);
      const uint8_t* vm = mr + s * MS;
      float4 cv[VT];
#pragma unroll
      for (int j = 0; j < VT; ++j) cv[j] = *(const float4*)(vm + Sh::L_VC + 4 * (16 * (VT * wave + j) + 4 * g));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = 16 * t + n;
        const float corr = sum_nw(xz + (s * RB + row) * NW);
        const uint16_t* src = pw + ((2 * s) * RB + row) * PP + 32 * g;
        float4v o[VT];
#pragma unroll
        for (int j = 0; j < VT; ++j) o[j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const half8 bh = mfma_a(*(const uint4*)(src + 8 * tt));
          const half8 bl = mfma_a(*(const uint4*)(src + RB * PP + 8 * tt));
#pragma unroll
          for (int j = 0; j < VT; ++j) o[j] = mfma16(av[j][tt], bh, o[j]);
#pragma unroll
          for (int j = 0; j < VT; ++j) o[j] = mfma16(av[j][tt], bl, o[j]);
        }
#pragma unroll
        for (int j = 0; j < VT; ++j) {
          acc[s][j][t][0] = fmaf(cv[j].x * frec[t], o[j][0] + corr, acc[s][j][t][0]);
          acc[s][j][t][1] = fmaf(cv[j].y * frec[t], o[j][1] + corr, acc[s][j][t][1]);
          acc[s][j][t][2] = fmaf(cv[j].z * frec[t], o[j][2] + corr, acc[s][j][t][2]);
          acc[s][j][t][3] = fmaf(cv[j].w * frec[t], o[j][3] + corr, acc[s][j][t][3]);
        }
      }
    }
  }

  // ---- partial rows through the q~ area and l through the sigma area (no
  // wave reads either after the last record's scores; slower waves may still
  // read the zero-point sums); m is the same in every wave, l sums over them
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lsum = xsum4(l_part[t]);
    if (g == 0) {
      xs[wave * RB + 16 * t + n] = lsum;
      if (wave == 0) xm[16 * t + n] = m_run[t];
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int j = 0; j < VT; ++j)
        *(float4v*)(rows + (16 * t + n) * D + SUBW * s + 16 * (VT * wave + j) + 4 * g) = acc[s][j][t];
  }
  __syncthreads();
  write_block_partials<D, NW>(a, b, h, rb, RB, chunk, rows, xm, xs, true);
}

// 8 waves (two per SIMD) wherever the q~ units go round them (at least one
// per thread): all but 16-row blocks of 128-wide heads, which take 4
template <int D, int NT>
constexpr int body_waves() {
  return (D == 128 ? 4 : 8 * (D / 256)) * NT >= 8 ? 8 : 4;
}

template <int D, int KB, int VB, int NT>
__global__ __launch_bounds__((64 * body_waves<D, NT>())) void prefill_body_kernel(PrefillArgs a) {
  using Sh = PBody<D, KB, VB, NT, body_waves<D, NT>()>;
  extern __shared__ __align__(16) uint8_t smem[];
  prof_start(a.prof_ts);
  const int item = block_item();
  if (item >= a.n_items) return;
  const int b = find_seq(a, item, true);
  const PrefillSeq& sq = a.seq[b];
  int j = item - sq.body_item0;
  const int rb = j % a.n_rb;
  j /= a.n_rb;
  const int c = j % sq.n_body_chunks, h = j / sq.n_body_chunks;
  body_block<Sh>(a, b, h, rb, c, smem);
  prof_end(a.prof_ts);
}

// ---------------------------------------------------------------------------
// Sink and ring role: one chunk of the sink (chunk 0) or of the ring of one KV
// head for one row block, in steps of 64 tokens.  Per step:
//   (1) values into an fp16 tile V^T in LDS (tq6_0: the codes u - 32; the
//       sink and the f16 ring: the fp16 rows), transposed;
//   (2) scores: wave w takes the 16-token tile w against every row tile, its
//       key operands read straight from memory (tq6_0: exact u - 32 with the
//       block scales d applied per token after the product; fp16 rows as they
//       are, scored with the unrotated query);
//   (3) weights p (times d^V per 128-channel block for tq6_0) into LDS;
//   (4) values: wave w takes channel tiles D/64 w .. against every row tile,
//       accumulating straight into its running sums.
// Tokens after a row's position (and past the chunk) are masked; steps after
// the block's last position are not scanned.  Three barriers per step.
template <int D_, int NT_>
struct PRing {
  static constexpr int D = D_, NT = NT_, RB = 16 * NT_;
  static constexpr int NB = D / kQBlock, KK = D / 32, CPW = D / 64;
  // LDS: V^T [D][kBPitch] halves; weights [NB][hi, lo][RB][kBPitch] halves;
  // query operands [KK][NT][hi, lo][64] uint4; xm[4][RB], xl[4][RB] floats
  static constexpr int VT = 0, PW = VT + D * kBPitch * 2, QO = PW + NB * 2 * RB * kBPitch * 2;
  static constexpr int X = QO + KK * NT * 2 * 1024;
  static constexpr int total = X + 2 * 4 * RB * 4;
  static_assert(16 * D * 4 <= PW - VT, "one row tile of query rows fits the V^T area");
  static_assert(RB * D * 4 <= X - QO, "the partial rows fit the query operand area");
};

template <int D, int NT>
__device__ __forceinline__ void ring_block(const PrefillArgs& a, int b, int h, int rb, int c, uint8_t* smem) {
  using Ly = PRing<D, NT>;
  constexpr int NB = Ly::NB, KK = Ly::KK, CPW = Ly::CPW, RB = Ly::RB;
  const Layout& y = a.y;
  const PrefillSeq& sq = a.seq[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  uint16_t* vt = (uint16_t*)(smem + Ly::VT);
  uint16_t* pw = (uint16_t*)(smem + Ly::PW);  // [NB][hi, lo][RB][kBPitch]
  uint4* qo = (uint4*)(smem + Ly::QO);        // [KK][NT][2][64]
  float* xm = (float*)(smem + Ly::X);         // [4][RB]
  float* xl = xm + 4 * RB;                    // [4][RB]

  const bool sink = c == 0;
  const bool exact = sink || y.f16ring;  // fp16 rows in the original domain
  const int t_begin = sink ? 0 : (c - 1) * sq.ring_chunk;
  const int t_end = sink ? sq.n_sink : min(sq.ring_len, c * sq.ring_chunk);
  const int pos0 = sink ? 0 : kSink + kGroup * sq.n_rec;  // position of token 0 of the region
  const int n_rows = a.n_q * a.g, row0 = rb * RB;
  const int pmax = sq.p0 + (min(n_rows, row0 + RB) - 1) / a.g;
  if (t_begin >= t_end || pos0 + t_begin > pmax) {
    write_empty_partials<D, 4>(a, b, h, rb, RB, c);
    return;
  }
  const int t_stop = min(t_end, pmax - pos0 + 1);  // later tokens are after every row
  int prow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rr = row0 + 16 * t + n;
    prow[t] = rr < n_rows ? sq.p0 + rr / a.g : -1;
  }

  // ---- query operands in natural channel order, one row tile at a time
  // through the V^T area: k-step kk, lane (n, g): channels 32 kk + 8 g ..
  for (int t = 0; t < NT; ++t) {
    float* rows = (float*)vt;
    block_query_rows<D, 4>(a, b, h, row0 + 16 * t, 16, !exact, rows);
    __syncthreads();
    for (int kk = wave; kk < KK; kk += 4) {
      const float* r = rows + n * D + 32 * kk + 8 * g;
      uint32_t hh[4], ll[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) split_h2s(r[2 * pr], r[2 * pr + 1], hh[pr], ll[pr]);
      uint4* dst = qo + ((kk * NT + t) * 2) * 64 + lane;
      dst[0] = make_uint4(hh[0], hh[1], hh[2], hh[3]);
      dst[64] = make_uint4(ll[0], ll[1], ll[2], ll[3]);
    }
    __syncthreads();
  }

  // sources: fp16 rows (sink token t; f16 ring token t at slot ring0 + t) or tq6_0 codes and scales
  const uint16_t* ksrc = sink ? (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, sq.slot, a.layer, h, 0, 0)
                              : (const uint16_t*)(a.arena + rcode_off(y, sq.slot, a.layer, h, 0, 0));
  const uint16_t* vsrc = sink ? (const uint16_t*)(a.arena + y.off_sink) + sink_elem(y, sq.slot, a.layer, h, 1, 0)
                              : (const uint16_t*)(a.arena + rcode_off(y, sq.slot, a.layer, h, 1, 0));
  const uint8_t* kc = a.arena + rcode_off(y, sq.slot, a.layer, h, 0, 0);
  const uint8_t* vc = a.arena + rcode_off(y, sq.slot, a.layer, h, 1, 0);
  const uint8_t* ks = a.arena + rscale_off(y, sq.slot, a.layer, h, 0, 0);
  const uint8_t* vs = a.arena + rscale_off(y, sq.slot, a.layer, h, 1, 0);
  auto slot_of = [&](int t) {  // ring slot of ring token t (t < ring_len <= cap)
    const int s = sq.ring0 + t;
    return s >= y.cap ? s - y.cap : s;
  };
  auto row16 = [&](int t) -> int64_t { return (int64_t)(sink ? t : slot_of(t)) * D; };

  float m_run[NT], l_part[NT];
  float4v acc[CPW][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_part[t] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < CPW; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  for (int t0 = t_begin; t0 < t_stop; t0 += kBStep) {
    const int nv = min(kBStep, t_end - t0);  // tokens of the chunk in this step

    // ---- (1) V^T (tokens past the chunk: zero rows, or finite codes of token t0 with weight 0)
    if (exact) {
      constexpr int ITEMS = (kBStep / 4) * (D / 8) / 256;  // 4-token x 8-channel pieces per thread
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const int it = tid + 256 * j, tq = it % (kBStep / 4), c8 = it / (kBStep / 4);
        uint4 r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tok = 4 * tq + k;
          r[k] = *(const uint4*)(vsrc + row16(t0 + (tok < nv ? tok : 0)) + 8 * c8);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * tq + k >= nv) r[k] = make_uint4(0, 0, 0, 0);
        store_t4x8(vt, kBPitch, 8 * c8, 4 * tq, r);
      }
    } else {
      const int tq = tid & 15;
      for (int c16 = tid >> 4; c16 < D / 16; c16 += 16) {
        uint4 lo8[4], hi8[4];  // channels 16 c16 + 0..7 and + 8..15 of tokens 4 tq + k
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tok = 4 * tq + k;
          const uint32_t* p = (const uint32_t*)(vc + (int64_t)slot_of(t0 + (tok < nv ? tok : 0)) * (NB * kQBytes) +
                                                12 * c16);
          const uint32_t w0 = p[0], w1 = p[1], w2 = p[2];
          const half8 x0 = codes6_reg(w0, w1);
          const half8 x1 = codes6_reg(__builtin_amdgcn_alignbit(w2, w1, 16), w2 >> 16);
          __builtin_memcpy(&lo8[k], &x0, 16);
          __builtin_memcpy(&hi8[k], &x1, 16);
        }
        store_t4x8(vt, kBPitch, 16 * c16, 4 * tq, lo8);
        store_t4x8(vt, kBPitch, 16 * c16 + 8, 4 * tq, hi8);
      }
    }

    // ---- (2) scores of tile `wave` (token t0 + 16 wave + m in operand row m)
    const int tk = 16 * wave + n;                   // this lane's operand token
    const int tks = t0 + (tk < nv ? tk : 0);        // clamped: a finite row
    half8 ka[KK];
    if (exact) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) ka[kk] = mfma_a(*(const uint4*)(ksrc + row16(tks) + 32 * kk + 8 * g));
    } else {
      const uint8_t* row = kc + (int64_t)slot_of(tks) * (NB * kQBytes) + ((6 * g) & ~3);
      const uint32_t sh = (g & 1) ? 16u : 0u;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t* p = (const uint32_t*)(row + 24 * kk);
        const uint32_t w0 = p[0], w1 = p[1];
        ka[kk] = codes6_reg(__builtin_amdgcn_alignbit(w1, w0, sh), w1 >> sh);
      }
    }
    // block scales of this lane's 4 output tokens t0 + 16 wave + 4 g + r
    float dk[4][NB], dv[4][NB];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 16 * wave + 4 * g + r;
      const int sl = slot_of(t0 + (tok < nv ? tok : 0));
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        dk[r][blk] = exact ? 1.0f : h2f(*(const uint16_t*)(ks + ((int64_t)sl * NB + blk) * 2));
        dv[r][blk] = exact ? 1.0f : h2f(*(const uint16_t*)(vs + ((int64_t)sl * NB + blk) * 2));
      }
    }
    float sc[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float4v shb[NB], slb[NB];
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) shb[blk] = slb[blk] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4* op = qo + ((kk * NT + t) * 2) * 64 + lane;
        const int blk = kk / 4;
        shb[blk] = mfma16(ka[kk], mfma_a(op[0]), shb[blk]);
        slb[blk] = mfma16(ka[kk], mfma_a(op[64]), slb[blk]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.0f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) v = fmaf(dk[r][blk], shb[blk][r] + slb[blk][r] * kLoUnscale, v);
        const int tok = 16 * wave + 4 * g + r;
        const bool seen = tok < nv && pos0 + t0 + tok <= prow[t];
        sc[t][r] = seen ? v : kMaskedScore;
      }
      float mx = fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3]));
      mx = xmax4(mx);
      if (g == 0) xm[wave * RB + 16 * t + n] = mx;
    }
    __syncthreads();  // (B1) maxima; V^T complete

    // ---- (3) weights relative to the running maximum
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row = 16 * t + n;
      const float M = fmaxf(fmaxf(xm[row], xm[RB + row]), fmaxf(xm[2 * RB + row], xm[3 * RB + row]));
      const float m_new = fmaxf(m_run[t], M);
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_new);  // 0 on the first step
      m_run[t] = m_new;
#pragma unroll
      for (int i = 0; i < CPW; ++i) acc[i][t] *= alpha;
      float p[4], ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = sc[t][r] == kMaskedScore ? 0.0f : __builtin_amdgcn_exp2f(sc[t][r] - m_new);
        ls += p[r];
      }
      l_part[t] = fmaf(l_part[t], alpha, ls);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        if (exact && blk > 0) break;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = p[r] * dv[r][blk];
        uint2 hi, lo;
        split_h2(x[0], x[1], hi.x, lo.x);
        split_h2(x[2], x[3], hi.y, lo.y);
        uint16_t* dst = pw + ((2 * blk) * RB + row) * kBPitch + 16 * wave + 4 * g;
        *(uint2*)dst = hi;
        *(uint2*)(dst + RB * kBPitch) = lo;
      }
    }
    __syncthreads();  // (B2) weights

    // ---- (4) O^T += V^T P^T over the step's tokens
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int cb = CPW * wave + i;
      const int blk = exact ? 0 : (16 * cb) / kQBlock;
#pragma unroll
      for (int j = 0; j < kBStep / 32; ++j) {
        const half8 av = mfma_a(*(const uint4*)(vt + (16 * cb + n) * kBPitch + 32 * j + 8 * g));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint16_t* src = pw + ((2 * blk) * RB + 16 * t + n) * kBPitch + 32 * j + 8 * g;
          acc[i][t] = mfma16(av, mfma_a(*(const uint4*)src), acc[i][t]);
          acc[i][t] = mfma16(av, mfma_a(*(const uint4*)(src + RB * kBPitch)), acc[i][t]);
        }
      }
    }
    __syncthreads();  // (B3) V^T and the weights are free
  }

  // ---- partial rows through the query operand area (free after the last step)
  float* rows = (float*)qo;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lsum = xsum4(l_part[t]);
    if (g == 0) {
      xl[wave * RB + 16 * t + n] = lsum;
      if (wave == 0) xm[16 * t + n] = m_run[t];
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) *(float4v*)(rows + (16 * t + n) * D + 16 * (CPW * wave + i) + 4 * g) = acc[i][t];
  }
  __syncthreads();
  write_block_partials<D, 4>(a, b, h, rb, RB, c, rows, xm, xl, !exact);
}

template <int D, int NT>
__global__ __launch_bounds__(256) void prefill_ring_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int item = block_item();
  if (item >= a.n_items) return;
  const int b = find_seq(a, item, false);
  const PrefillSeq& sq = a.seq[b];
  int j = item - sq.ring_item0;
  const int rb = j % a.n_rb;
  j /= a.n_rb;
  const int nc = 1 + sq.n_ring_chunks;
  const int c = j % nc, h = j / nc;
  ring_block<D, NT>(a, b, h, rb, c, smem);
}

template <class K>
hipError_t launch_lds(K kernel, int n_items, int lds, int threads, const PrefillArgs& a, hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = (n_items + 7) / 8 * 8;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

template <int D, int KB, int VB, int NT>
hipError_t launch_body_t(const PrefillArgs& a, hipStream_t stream) {
  using Sh = PBody<D, KB, VB, NT, body_waves<D, NT>()>;
  return launch_lds(prefill_body_kernel<D, KB, VB, NT>, a.n_items, Sh::total, Sh::NTH, a, stream);
}
template <int D, int NT>
hipError_t launch_ring_t(const PrefillArgs& a, hipStream_t stream) {
  return launch_lds(prefill_ring_kernel<D, NT>, a.n_items, PRing<D, NT>::total, 256, a, stream);
}

}  // namespace

// LDS bytes of the body (body = true) or sink/ring workgroup of a launch.
int prefill_lds_bytes(int D, int kb, int nt, bool body) {
#define KVQ_LDS(DD, NTT)                                                                            \
  if (D == DD && nt == NTT)                                                                         \
    return body ? (kb == 8 ? PBody<DD, 8, 4, NTT, body_waves<DD, NTT>()>::total                                  \
                           : PBody<DD, 4, 4, NTT, body_waves<DD, NTT>()>::total)                                 \
                : PRing<DD, NTT>::total;
  KVQ_LDS(128, 1) KVQ_LDS(128, 2) KVQ_LDS(128, 4)
  KVQ_LDS(256, 1) KVQ_LDS(256, 2) KVQ_LDS(256, 4)
  if (D == 256 && nt == 3 && body)
    return kb == 8 ? PBody<256, 8, 4, 3, body_waves<256, 3>()>::total : PBody<256, 4, 4, 3, body_waves<256, 3>()>::total;
  KVQ_LDS(512, 1)
  if (D == 512 && nt == 2 && body)
    return kb == 8 ? PBody<512, 8, 4, 2, body_waves<512, 2>()>::total
                   : PBody<512, 4, 4, 2, body_waves<512, 2>()>::total;
#undef KVQ_LDS
  return 0;
}

// Row tiles of 16 query rows per work item for n_q g rows.  Record items:
// 1, 2, 3 (256-wide heads: the three tiles of a 48-row verify block, where
// four would leave a quarter of the block empty) or 4 (512-wide heads: at
// most 2, for LDS).  Sink/ring items: one tile for blocks of up to 64 rows
// (their 16-row items fit two workgroups per compute unit and the launch has
// more of them: an 8-token block at g = 6 took 11 % less time per step than
// with 64-row items), else as the records (512-wide heads: 1).
int prefill_row_tiles(int D, int rows, bool body) {
  if (!body) return D == 512 || rows <= 64 ? 1 : 4;
  const int nt = rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 48 && D == 256 ? 3 : 4;
  return D == 512 ? (nt > 2 ? 2 : nt) : nt;
}

// The body launch: PrefillArgs.n_items body items, each (sequence, KV head,
// body chunk, row block); nt = prefill_row_tiles(D, n_q g, true).
hipError_t launch_prefill_body(const PrefillArgs& a, int nt, hipStream_t stream) {
  const int D = a.y.D, kb = a.y.kbits, vb = a.y.vbits;
#define KVQ_BODY(DD, KBB, VBB)                                                         \
  if (D == DD && kb == KBB && vb == VBB) {                                             \
    if (nt == 1) return launch_body_t<DD, KBB, VBB, 1>(a, stream);                     \
    if (nt == 2) return launch_body_t<DD, KBB, VBB, 2>(a, stream);                     \
    if (nt == 4 && DD != 512) return launch_body_t<DD, KBB, VBB, (DD == 512 ? 2 : 4)>(a, stream); \
  }
  KVQ_BODY(128, 4, 4)
  KVQ_BODY(128, 8, 4)
  KVQ_BODY(256, 4, 4)
  KVQ_BODY(256, 8, 4)
  KVQ_BODY(512, 4, 4)
  KVQ_BODY(512, 8, 4)
  KVQ_BODY(256, 3, 3)
  KVQ_BODY(256, 3, 2)
  KVQ_BODY(256, 2, 2)
  KVQ_BODY(256, 2, 3)
#undef KVQ_BODY
  // three row tiles: 256-wide heads only (eight waves, three q~ units each)
  if (nt == 3 && D == 256) {
    if (kb == 4 && vb == 4) return launch_body_t<256, 4, 4, 3>(a, stream);
    if (kb == 8 && vb == 4) return launch_body_t<256, 8, 4, 3>(a, stream);
    if (kb == 3 && vb == 3) return launch_body_t<256, 3, 3, 3>(a, stream);
    if (kb == 3 && vb == 2) return launch_body_t<256, 3, 2, 3>(a, stream);
    if (kb == 2 && vb == 2) return launch_body_t<256, 2, 2, 3>(a, stream);
    if (kb == 2 && vb == 3) return launch_body_t<256, 2, 3, 3>(a, stream);
  }
  return hipErrorInvalidValue;
}

// The sink and ring launch: items (sequence, KV head, chunk 0 (sink) or ring
// chunk, row block); nt = prefill_row_tiles(D, n_q g, false).
hipError_t launch_prefill_ring(const PrefillArgs& a, int nt, hipStream_t stream) {
  switch (a.y.D) {
    case 128:
      return nt == 1 ? launch_ring_t<128, 1>(a, stream) : nt == 2 ? launch_ring_t<128, 2>(a, stream)
                                                                  : launch_ring_t<128, 4>(a, stream);
    case 256:
      return nt == 1 ? launch_ring_t<256, 1>(a, stream) : nt == 2 ? launch_ring_t<256, 2>(a, stream)
                                                                  : launch_ring_t<256, 4>(a, stream);
    case 512:
      return nt == 1 ? launch_ring_t<512, 1>(a, stream) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
