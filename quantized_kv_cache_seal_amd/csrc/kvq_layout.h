// Device-memory layout of one cache arena and the by-value kernel arguments.
//
// Arena (every region 256-byte aligned), S = max_seqs, L = layers, H = KV heads,
// D = head_dim, NB = D / 128 tq6_0 blocks per vector, CAP = ring slots:
//   sink        fp16  [S][L][H][2 (K,V)][128][D]            original domain
//   ring codes  u8    [S][L][H][2][CAP][NB][96]             6-bit LSB-first codes
//   ring scales fp16  [S][L][H][2][CAP][NB]                 d of each block
// or, with f16 staging, the ring as fp16 [S][L][H][2][CAP][D] in the original
// domain (the codes' place; no scales).
//   body        u8    [S][L][H][MAX_REC][REC_BYTES]         sealed records
// A record is NSUB sub-records of SUB channels (SUB = 256, or 128 for 128-wide
// heads), each [K codes 128 x SUB row-major][V codes SUB x 128 channel-major]
// [K: C[SUB] S[128] Z[128] fp16][V: C S Z], codes packed two per byte (even
// element in the low nibble) at 4 bits or one per byte at 8 bits.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kvq {

constexpr int kSink = 128;        // sink tokens (SJ-KVaRN 2.1, item 1)
constexpr int kGroup = 128;       // tokens per sealed record (SJ-KVaRN 2)
constexpr int kQBlock = 128;      // values per tq6_0 block
constexpr int kQBytes = 96;       // code bytes per tq6_0 block (128 x 6 bits)
constexpr int kMaxLaunchSeqs = 32;
constexpr int kMaxSealTasks = 64;
constexpr int kMaxGroup = 16;     // query heads per KV head
constexpr int kMaxChunks = 4096;  // split-K partials per (sequence, query head)
// Bytes of the per-GPU scratch array that holds the partials of the
// allocation-free decode (8 MiB: the matrix-core plans of the benchmarked
// workloads need at most ~4.2 MB).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr int kReadProbeBlocks = 16384;  // workgroups of the read probe (4 waves, one output word each)
// A split-K partial row: [m, l, 0, 0, acc[D]] fp32, acc 16-byte aligned and in
// the original domain (the producer rotates its rotated-domain sums back).
constexpr int kPartHead = 4;
__host__ __device__ inline int part_stride(int D) { return D + kPartHead; }

struct Layout {
  int32_t S, L, H, D, NB, cap, nsub, sub, kbits, vbits, max_rec, f16ring;  // f16ring: f16 staging
  int64_t sub_bytes, rec_bytes, kcode_bytes, vcode_bytes;
  int64_t off_sink, off_rcode, off_rscale, off_body, total;
};

// (seq, layer, head) flattened
__host__ __device__ inline int64_t slh(const Layout& y, int s, int l, int h) {
  return ((int64_t)s * y.L + l) * y.H + h;
}
// fp16 element index of sink[s][l][h][kv][t][0]
__host__ __device__ inline int64_t sink_elem(const Layout& y, int s, int l, int h, int kv, int t) {
  return ((slh(y, s, l, h) * 2 + kv) * kSink + t) * (int64_t)y.D;
}
// bytes of one ring row (one token of one head, K or V): tq6_0 codes, or fp16
__host__ __device__ inline int ring_row_bytes(const Layout& y) { return y.f16ring ? 2 * y.D : y.NB * kQBytes; }
// byte offset (from arena) of ring codes[s][l][h][kv][slot][0] (with f16
// staging: of the slot's fp16 row)
__host__ __device__ inline int64_t rcode_off(const Layout& y, int s, int l, int h, int kv, int slot) {
  return y.off_rcode + ((slh(y, s, l, h) * 2 + kv) * y.cap + slot) * (int64_t)ring_row_bytes(y);
}
// byte offset of ring scales[s][l][h][kv][slot][0]
__host__ __device__ inline int64_t rscale_off(const Layout& y, int s, int l, int h, int kv, int slot) {
  return y.off_rscale + ((slh(y, s, l, h) * 2 + kv) * y.cap + slot) * (int64_t)(y.NB * 2);
}
// byte offset of body record r of (s, l, h)
__host__ __device__ inline int64_t rec_off(const Layout& y, int s, int l, int h, int64_t r) {
  return y.off_body + (slh(y, s, l, h) * y.max_rec + r) * y.rec_bytes;
}

struct AppendArgs {
  const uint16_t* k;  // fp16 [n_seqs][n_tok][H][D]
  const uint16_t* v;
  uint8_t* arena;
  Layout y;
  int32_t layer, n_tok, n_seqs, pad;
  uint32_t signs[8];  // bit i set: entry i of [s1 (128); s2 (128)] is -1
  int32_t slot[kMaxLaunchSeqs];
  int64_t pos0[kMaxLaunchSeqs];
};

struct SealTask {
  int32_t slot, layer, rec0, n_groups, first;  // first = index of its first group in the grid
};

struct SealArgs {
  uint8_t* arena;
  Layout y;
  int32_t passes, n_tasks, total_groups, pad;
  uint32_t signs[8];  // f16 staging, 128-wide heads: the rotation's sign flips
  SealTask task[kMaxSealTasks];
};

struct DecodeSeq {
  int32_t slot;      // sequence index in the arena
  int32_t n_sink;    // tokens in the sink (1..128)
  int32_t ring_len;  // tokens in the ring
  int32_t ring0;     // ring slot of the oldest unsealed token
  int32_t n_rec;     // sealed records
  int32_t n_ring_chunks, n_body_chunks, n_chunks;  // body chunks split the records evenly
  int32_t app_slot;   // fused decode step: ring slot the new token is written to
  int32_t app_chunk;  // fused decode step: partial index of the new token (the last one)
};

struct DecodeArgs {
  const uint8_t* arena;
  Layout y;
  const uint16_t* q;  // fp16 [n_seqs][Hq][D]
  const uint16_t* k_new;  // fused decode step: fp16 [n_seqs][H][D] token appended first, or null
  const uint16_t* v_new;
  float* part;        // [n_seqs][Hq][max_chunks][part_stride(D)] split-K partial rows
  float scale;
  int32_t layer, Hq, g, n_seqs, max_chunks;
  int32_t ring_chunk;    // ring tokens per chunk
  int32_t n_app_items;   // fused decode step: one append item per (sequence, KV head), first
  int32_t n_body_items;  // matrix-core launch: body items, after the append items
  int32_t n_old;         // matrix-core launch: workgroups 0 .. n_old - 1 are the first resident on
                         // their compute unit (issue priority): they take more records
  int32_t valu_regions;  // bit r set: the vector-ALU kernel scans region r (0 sink, 1 ring, 2 body)
  uint32_t signs[8];
  unsigned long long* prof_ts;  // profiling: {first start, last end} wall-clock stamps, or null
  DecodeSeq seq[kMaxLaunchSeqs];
};

struct MergeArgs {
  const float* part;  // [n_seqs][n_rows][Hq][max_chunks][part_stride(D)]
  void* out;          // [n_seqs][n_rows][Hq][D] fp32 or fp16
  int32_t D, Hq, n_seqs, max_chunks, out_f16;
  int32_t n_rows;     // query tokens per sequence: 1 for decode, n_q for block attention
  int32_t n_chunks[kMaxLaunchSeqs];  // partials per row of each sequence
};

// Block attention (prefill chunks, verify blocks): the queries of the newest
// n_q cached tokens of each sequence, each seeing the tokens up to its own
// position.  The rows of a (sequence, KV head) are r = t g + e (token t of
// the block, query head e of the group), taken 16 NT at a time (a row block).
constexpr int kMaxBlock = 4096;       // n_q limit
constexpr int kMaxBlockChunks = 64;   // ring chunks, and record chunks, per row (each at most this)
struct PrefillSeq {
  int32_t slot, n_sink, ring_len, ring0, n_rec;
  int32_t p0;          // position of the block's first token
  int32_t ring_chunk;  // ring tokens per chunk (a multiple of 64)
  int32_t n_ring_chunks, n_body_chunks, n_chunks;  // partial 0: sink; 1 ..: ring chunks; then body chunks
  int32_t body_item0, ring_item0;  // this sequence's first item in the body / sink-and-ring launch
};
struct PrefillArgs {
  const uint8_t* arena;
  Layout y;
  const uint16_t* q;  // fp16 [n_seqs][n_q][Hq][D]
  float* part;        // [n_seqs][n_q][Hq][max_chunks][part_stride(D)]
  float scale;
  int32_t layer, Hq, g, n_seqs, n_q, max_chunks;
  int32_t n_rb;       // row blocks per (sequence, KV head)
  int32_t n_items;    // work items of the launch (the grid is rounded up to a multiple of 8)
  uint32_t signs[8];
  unsigned long long* prof_ts;  // profiling: {first start, last end} wall-clock stamps, or null
  PrefillSeq seq[kMaxLaunchSeqs + 1];  // seq[n_seqs].*_item0: the launch's item counts
};

// TBQ4 comparator block (KV cache math): [fp16 norm][64 bytes of 4-bit
// indices, even value in the low nibble] per 128 rotated values.
constexpr int kTbqBytes = 66;

struct Tbq4CodecArgs {
  const uint16_t* x;         // encode input: fp16 [n][128]
  uint8_t* blocks_out;       // encode output: [n][66]
  const uint8_t* blocks_in;  // decode input: [n][66]
  float* y;                  // decode output: fp32 [n][128], original domain
  int64_t n;
  float cent[16];            // centroids, ascending
  float bnd[16];             // cell boundaries (15 used)
  uint32_t signs[8];         // bit i set: entry i of [s1 (128); s2 (128)] is -1
};

struct Tbq4AttnArgs {
  const uint16_t* q;         // fp16 [n_seqs][Hq][D]
  const uint8_t* kb;         // [n_seqs][H][cap][D / 128][66]
  const uint8_t* vb;
  float* qr;                 // workspace: rotated, scaled queries fp32 [n_seqs][Hq][D]
  float* part;               // [n_seqs][Hq][max_chunks][part_stride(D)]
  int64_t cap;
  float scale_log2;          // softmax scale times log2(e)
  int32_t D, H, Hq, g, n_seqs, max_chunks, chunk, pad;
  float cent[16];
  uint32_t signs[8];
  int64_t len[kMaxLaunchSeqs];  // tokens per sequence (1 .. cap)
};

}  // namespace kvq
