/*
 * kvq.h -- C ABI of an MI355X (gfx950) quantized KV cache: a 128-token fp16
 * sink, a staging ring holding the exact tail (rotated 6-bit, or fp16), and
 * sealed body records (4/4, 8/4, 3/3, 3/2, 2/2 or 2/3 bits per key/value
 * code), read by one split-K decode-attention pass, or by block attention
 * for prefill chunks and verify blocks.
 *
 * The method is SJ-KVaRN (page "SJ-KVaRN", sections 2-4) built on KVarN:
 *   - section 2.1 "The life of a token": sink, staging, exact tail, seal;
 *   - section 2.2: Hadamard rotation, Sinkhorn-style balancing, per-row
 *     rounding with fp16 scale and zero point;
 *   - section 4.3 "Adaptive tail": the tail grows from tail_min to tail_max,
 *     then every full 128-token group older than the newest tail_min tokens
 *     is sealed in one batch; an idle server seals back to tail_min;
 *   - section 10: sealed records cannot be partly rewritten.
 * Page "KV cache math": the randomized Walsh-Hadamard transform on 128
 * values (sign flip, transform, sign flip) and the fused rotated-domain
 * attention (rotate the query once, read raw blocks, rotate the output back).
 *
 * Conventions for every call:
 *   - Every function returns a kvq_status; no C++ exception crosses the ABI.
 *   - Argument, capacity and state errors are detected on the host before
 *     anything is enqueued, and then leave the cache unchanged.
 *   - "device" pointers are HIP device memory owned by the caller; they must
 *     stay valid until the work enqueued on `stream` has finished.  "host"
 *     pointers are read or written before the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; the hot path (append, seal,
 *     decode) never waits for the device.
 *   - A cache handle is not thread-safe: use one handle per host thread.
 *   - kvq_last_error() returns a thread-local message for the last failure.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,     /* bad argument, shape or configuration            */
  KVQ_ERR_CAPACITY = -2,    /* context beyond max_ctx, or arena too small      */
  KVQ_ERR_RING_FULL = -3,   /* staging ring cannot take the tokens: seal first */
  KVQ_ERR_SEALED = -4,      /* would rewrite part of a sealed record           */
  KVQ_ERR_DEVICE = -5,      /* a HIP call failed (detail in kvq_last_error)    */
  KVQ_ERR_UNSUPPORTED = -6  /* valid but not supported by this build / mode    */
} kvq_status;

enum { KVQ_SEAL_IF_FULL = 0, KVQ_SEAL_TO_MIN = 1 };
enum { KVQ_REGION_SINK = 0, KVQ_REGION_RING = 1, KVQ_REGION_BODY = 2 };
enum { KVQ_OUT_F32 = 0, KVQ_OUT_F16 = 1 };
enum { KVQ_PATH_AUTO = 0, KVQ_PATH_VALU = 1, KVQ_PATH_MFMA = 2 };
enum { KVQ_FLAG_PLAN_ONLY = 1 };   /* metadata only: no arena, no kernels */
/* Staging precision of the ring (SJ-KVaRN section 4.1): tq6_0, the rotated
 * 6-bit format (98 bytes per 128 values), or f16, the tokens kept exact in
 * the original domain (the KVarN-style exact F16 tail: KV Cache Precision
 * Tail, section 2), rotated when their group is sealed. */
enum { KVQ_STAGE_TQ6 = 0, KVQ_STAGE_F16 = 1 };

/* Sizes are in tokens unless noted.  Constraints checked by every call:
 *   head_dim in {128, 256, 512}; n_q_heads a multiple of n_kv_heads with
 *   n_q_heads / n_kv_heads <= 16; (k_bits, v_bits) in {(4, 4), (8, 4)}, or
 *   k_bits and v_bits both in {2, 3} (SJ-KVaRN 2.3: 3/3, 3/2; and 2/2, 2/3);
 *   tail_min a multiple of 128, 128 <= tail_min <= tail_max;
 *   margin >= 0; max_ctx >= 1; 0 <= sinkhorn_passes <= 64.
 * Ring capacity = round_up(tail_max + margin, 128) token slots, allocated up
 * front (SJ-KVaRN section 3).  Body capacity = (max_ctx - 128) / 128 records
 * per (sequence, layer, KV head). */
typedef struct {
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_q_heads;
  int32_t max_seqs;
  int32_t tail_min;
  int32_t tail_max;
  int32_t margin;
  int64_t max_ctx;          /* tokens per sequence */
  int32_t k_bits;
  int32_t v_bits;
  int32_t sinkhorn_passes;  /* alternating row/column sweeps, rows first */
  int32_t flags;            /* KVQ_FLAG_* */
  /* Sign flips of the 128-point randomized Walsh-Hadamard transform used for
   * 128-wide heads: entries 0..127 are applied before the transform, 128..255
   * after; bit b of word w set means entry 64*w+b is -1.  Ignored otherwise. */
  uint64_t rot_signs[4];
  int32_t stage_fmt;        /* KVQ_STAGE_TQ6 (0, the default) or KVQ_STAGE_F16 */
  int32_t reserved;         /* must be 0 */
} kvq_config;

typedef struct kvq_cache kvq_cache;

/* Device bytes the arena of a cache with this configuration needs.
 * device_bytes: host out.  Errors: KVQ_ERR_INVALID. */
kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* device_bytes);

/* Create a cache over a caller-owned device arena of at least
 * kvq_cache_bytes() bytes (256-byte aligned).  The arena is not cleared:
 * only regions written by kvq_append / kvq_seal / kvq_import are ever read.
 * With KVQ_FLAG_PLAN_ONLY, arena may be NULL and the cache keeps only the
 * host metadata (appends and seals update counts; no kernel runs, decode and
 * export return KVQ_ERR_UNSUPPORTED).  out: host out, owned by the caller
 * until kvq_cache_destroy.  Errors: KVQ_ERR_INVALID, KVQ_ERR_CAPACITY. */
kvq_status kvq_cache_create(const kvq_config* cfg, void* device_arena, size_t arena_bytes, kvq_cache** out);

/* Free the host metadata.  Does not free the arena or wait for the device. */
kvq_status kvq_cache_destroy(kvq_cache* cache);

/* Append n_tok tokens to each listed sequence of one layer (SJ-KVaRN 2.1,
 * items 1-2).  Position p < 128 is copied to the fp16 sink unchanged; every
 * later position is rotated (section 2.2; 128-wide heads: KV cache math) and
 * written to the ring slot (p - 128) mod capacity as tq6_0 blocks (98 bytes
 * per 128 values: an fp16 scale d = fp16(amax/31) and 128 six-bit codes
 * q + 32, q = clamp(rne(x / d), -31, 31)), or, with f16 staging, copied to
 * that slot unchanged (original domain, like the sink).
 * seq_ids: host [n_seqs], distinct, in [0, max_seqs).
 * k, v: device fp16 [n_seqs][n_tok][n_kv_heads][head_dim], contiguous.
 * Never seals: if the ring cannot take the tokens it returns
 * KVQ_ERR_RING_FULL (call kvq_seal first).  Errors: KVQ_ERR_INVALID,
 * KVQ_ERR_CAPACITY (beyond max_ctx), KVQ_ERR_RING_FULL, KVQ_ERR_DEVICE. */
kvq_status kvq_append(kvq_cache* cache, int32_t layer, const int32_t* seq_ids, int32_t n_seqs,
                      const void* k, const void* v, int32_t n_tok, void* stream);

/* Seal eligible groups (SJ-KVaRN 2.1 item 4 and 4.3) of one layer, or of
 * every layer when layer == -1, for every sequence.  For each sequence and
 * layer with ring length n: with KVQ_SEAL_IF_FULL nothing happens unless
 * n >= tail_max; then (both modes) the oldest floor((n - tail_min)/128)
 * groups are sealed: each 128-token x 256-channel tile (128-channel for
 * 128-wide heads) of K and of V is read back from the ring (f16 staging: the
 * fp16 rows rotated, exactly, rounded once to fp32), balanced by
 * sinkhorn_passes alternating row/column log-domain passes (section 2.2),
 * divided by its fp16 column scales C, and each row rounded to k_bits / v_bits
 * with its own fp16 scale S and zero point Z.
 * groups_sealed: host out (may be NULL), number of 128-token groups sealed
 * summed over sequences and layers.  Errors: KVQ_ERR_INVALID, KVQ_ERR_DEVICE. */
kvq_status kvq_seal(kvq_cache* cache, int32_t layer, int32_t mode, void* stream, int32_t* groups_sealed);

/* Device workspace kvq_attn_decode and kvq_decode_step need for a call on n_seqs sequences
 * whose contexts are at most max_ctx.  bytes: host out. */
kvq_status kvq_workspace_bytes(const kvq_cache* cache, int32_t n_seqs, size_t* bytes);

/* Decode attention of one query per sequence over every cached token of one
 * layer: the sink, the ring (exact tail) and the sealed body, merged under one
 * softmax (SJ-KVaRN 2.1; KV Cache Precision Tail, section 2).  The query is
 * rotated once and the ring and body are read in the rotated domain; the
 * output is rotated back once (KV cache math, fused rotated-domain kernel).
 * Query head h uses KV head h / (n_q_heads / n_kv_heads).
 * q: device fp16 [n_seqs][n_q_heads][head_dim].  out: device
 * [n_seqs][n_q_heads][head_dim], fp32 or fp16 per out_dtype.  scale
 * multiplies q.k.  workspace: device, ws_bytes >= kvq_workspace_bytes(n_seqs).
 * Every listed sequence must hold at least one token.  Errors:
 * KVQ_ERR_INVALID, KVQ_ERR_CAPACITY (workspace too small), KVQ_ERR_DEVICE. */
kvq_status kvq_attn_decode(kvq_cache* cache, int32_t layer, const int32_t* seq_ids, int32_t n_seqs,
                           const void* q, void* out, int32_t out_dtype, float scale,
                           void* workspace, size_t ws_bytes, void* stream);

/* kvq_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and kernels, with the split-K partials held in a
 * device array the library owns instead of a caller workspace: 8 MiB
 * (KVQ_NOALLOC_SCRATCH_BYTES) per GPU, allocated with the code object (no
 * hipMalloc, hipFree or other allocating call) and held until the process
 * ends.  Every call on a GPU shares that GPU's array and leaves its contents
 * behind; calls that overlap on one GPU (several streams, or threads sharing
 * a device) race on it and must be ordered by the caller.
 * Arguments as kvq_attn_decode without workspace and ws_bytes.  Errors: those
 * of kvq_attn_decode; KVQ_ERR_CAPACITY when the call's partials exceed the
 * array, in which case nothing is enqueued.  The partials take n_seqs x
 * n_q_heads x (chunks per sequence) x (head_dim + 4) x 4 bytes: ~3.2 MB for
 * one 110,592-token sequence or 16 of 65,536 tokens (4 x 256 KV heads, 24
 * query heads, matrix-core plan), ~4.2 MB at 512-wide heads; many sequences
 * with short bodies, or the vector-ALU path (one partial per record), can
 * need more. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
kvq_status kvq_attn_decode_noalloc(kvq_cache* cache, int32_t layer, const int32_t* seq_ids, int32_t n_seqs,
                                   const void* q, void* out, int32_t out_dtype, float scale, void* stream);

/* Block attention of one layer, for prefill chunks and speculative verify
 * blocks: the queries of the newest n_q cached tokens of each listed sequence
 * (appended with kvq_append first), query t of the block belonging to the
 * token at position n_tok - n_q + t and seeing every cached token at or before
 * that position, whichever region holds it: sink, ring or sealed body (HAL
 * #582 section 3b measures prefill over the same quantised caches; SJ-KVaRN
 * 2.1 and KV Cache Precision Tail section 2: all regions under one softmax).
 * The same rotated-domain arithmetic as kvq_attn_decode, on the matrix cores
 * with up to 64 query rows (token, head) per product.
 * q: device fp16 [n_seqs][n_q][n_q_heads][head_dim].  out: device
 * [n_seqs][n_q][n_q_heads][head_dim], fp32 or fp16 per out_dtype.  scale
 * multiplies q.k.  1 <= n_q <= 4096 and every listed sequence holds at least
 * n_q tokens.  workspace: device, ws_bytes >= kvq_prefill_workspace_bytes(
 * n_seqs, n_q).  Every body width is supported at head_dim 256; at 128 and
 * 512 the 4/4 and 8/4 bodies.  Errors: KVQ_ERR_INVALID, KVQ_ERR_CAPACITY
 * (workspace too small), KVQ_ERR_UNSUPPORTED (2- or 3-bit bodies at head_dim
 * 128 or 512), KVQ_ERR_DEVICE. */
kvq_status kvq_prefill_workspace_bytes(const kvq_cache* cache, int32_t n_seqs, int32_t n_q, size_t* bytes);
kvq_status kvq_attn_prefill(kvq_cache* cache, int32_t layer, const int32_t* seq_ids, int32_t n_seqs, int32_t n_q,
                            const void* q, void* out, int32_t out_dtype, float scale, void* workspace,
                            size_t ws_bytes, void* stream);

/* One decode step of one layer: append one token per listed sequence, seal
 * what a KVQ_SEAL_IF_FULL seal of the layer would seal, then decode
 * attention of q over every cached token including the new one (SJ-KVaRN
 * 2.1: a decode pass reads sink, ring and body; the token just written is part
 * of the tail).  The result is that of kvq_append (n_tok = 1), kvq_seal(layer,
 * KVQ_SEAL_IF_FULL) and kvq_attn_decode in turn.  When the matrix-core path
 * runs, every new token lands in the ring and nothing is due for sealing in
 * the layer, it is one decode launch (plus the merge): the new token is
 * encoded into its ring slot by the same launch and enters the softmax as
 * its own split-K partial, with the decoded tq6_0 values the ring holds.
 * k, v: device fp16 [n_seqs][n_kv_heads][head_dim]; q, out, out_dtype, scale,
 * workspace, ws_bytes as kvq_attn_decode.  groups_sealed: host out (may be
 * NULL).  Errors: those of the three calls; on a fused launch, argument and
 * capacity errors leave the cache unchanged. */
kvq_status kvq_decode_step(kvq_cache* cache, int32_t layer, const int32_t* seq_ids, int32_t n_seqs,
                           const void* k, const void* v, const void* q, void* out, int32_t out_dtype,
                           float scale, void* workspace, size_t ws_bytes, void* stream,
                           int32_t* groups_sealed);

/* Select the kernel that scans sealed records: KVQ_PATH_AUTO (the default)
 * and KVQ_PATH_MFMA take the matrix cores (head_dim 128, 256 or 512 with
 * 4- or 8-bit K and 4-bit V; the 2- and 3-bit bodies at head_dim 256; AUTO
 * takes the vector-ALU scan for the 2- and 3-bit bodies of other widths,
 * MFMA refuses them with KVQ_ERR_UNSUPPORTED), KVQ_PATH_VALU the vector-ALU
 * reference scan (kept for A/B checks).  Errors: KVQ_ERR_INVALID. */
kvq_status kvq_set_decode_path(kvq_cache* cache, int32_t path);

/* Host-side counts of one (sequence, layer): tokens cached, sealed records,
 * ring length.  Any out pointer may be NULL. */
kvq_status kvq_seq_info(const kvq_cache* cache, int32_t seq, int32_t layer, int64_t* n_tok,
                        int64_t* n_records, int32_t* ring_len);

/* Drop every token of one sequence (all layers); its slots are reused. */
kvq_status kvq_seq_reset(kvq_cache* cache, int32_t seq);

/* Roll one sequence back to n_tok tokens on one layer (or all when layer ==
 * -1).  Only unsealed tokens can be removed: a target below the sealed
 * boundary 128 + 128 * n_records (when n_records > 0) returns KVQ_ERR_SEALED
 * (SJ-KVaRN section 10: removing tokens older than the seal boundary requires
 * reprocessing).  Growing is not allowed (KVQ_ERR_INVALID). */
kvq_status kvq_seq_truncate(kvq_cache* cache, int32_t seq, int32_t layer, int64_t n_tok);

/* Whole-sequence save and restore (the pages list save/restore and rollback
 * among the cache's operations: SJ-KVaRN section 10).  A saved sequence is
 * one host blob: a header (format version and the cache's layout and encoding
 * fingerprint: layers, KV heads, head_dim, ring capacity, bit widths,
 * balancing passes, rotation signs), the per-layer token and record counts,
 * then the sequence's sink, ring and sealed records as laid out in the arena.
 * Restoring a snapshot rolls a sequence back past its seal boundary, which
 * kvq_seq_truncate cannot do.
 * kvq_seq_save_bytes: host out, the blob size for the sequence as it is now.
 * kvq_seq_save: host_dst of exactly that many bytes; reads the device in
 * stream order and synchronises `stream` before returning.
 * kvq_seq_restore: host_src a blob from kvq_seq_save of a cache with the same
 * fingerprint (any max_seqs, max_ctx >= the saved counts); replaces slot seq
 * (any other slot, or the one saved) and synchronises `stream`.
 * Errors: KVQ_ERR_INVALID (range, size, or a blob that is not a saved
 * sequence of a matching cache; nothing is changed), KVQ_ERR_UNSUPPORTED
 * (plan-only cache), KVQ_ERR_DEVICE. */
kvq_status kvq_seq_save_bytes(const kvq_cache* cache, int32_t seq, size_t* bytes);
kvq_status kvq_seq_save(const kvq_cache* cache, int32_t seq, void* host_dst, size_t bytes, void* stream);
kvq_status kvq_seq_restore(kvq_cache* cache, int32_t seq, const void* host_src, size_t bytes, void* stream);

/* Copy canonical bytes of one cache unit to the host, synchronising `stream`:
 *   KVQ_REGION_SINK, index = token (< 128): [K fp16 x head_dim][V fp16 x head_dim];
 *   KVQ_REGION_RING, index = ring slot: for K then V, head_dim/128 tq6_0
 *     blocks of 98 bytes, each [fp16 d][96-byte LSB-first 6-bit stream]
 *     (f16 staging: [K fp16 x head_dim][V fp16 x head_dim], as the sink);
 *   KVQ_REGION_BODY, index = record: the record bytes, per 256-channel
 *     sub-tile (128 for 128-wide heads) [K codes 128 tokens x sub, row-major]
 *     [V codes sub channels x 128 tokens, channel-major] [K: C[sub] S[128]
 *     Z[128] fp16][V: the same]; each row of codes an LSB-first stream of
 *     k_bits (v_bits) values, value i in bits b i .. b i + b - 1 (4 bits: the
 *     even element in the low nibble; 8 bits: one byte each).
 * bytes must equal the unit's size (kvq_unit_bytes).  Errors:
 * KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED (plan-only cache), KVQ_ERR_DEVICE. */
kvq_status kvq_export(const kvq_cache* cache, int32_t seq, int32_t layer, int32_t kv_head, int32_t region,
                      int64_t index, void* host_dst, size_t bytes, void* stream);

/* The inverse of kvq_export: write canonical bytes into one unit (a hook for
 * tests that place reference-built records; counts are not changed). */
kvq_status kvq_import(kvq_cache* cache, int32_t seq, int32_t layer, int32_t kv_head, int32_t region,
                      int64_t index, const void* host_src, size_t bytes, void* stream);

/* Size in bytes of one exported unit of a region.  bytes: host out. */
kvq_status kvq_unit_bytes(const kvq_cache* cache, int32_t region, size_t* bytes);

/* Profiling hook.  kvq_profile_start(cache, max_calls) allocates a small
 * device buffer (2 timestamps per call) on the current device; each of the
 * following kvq_attn_decode (and kvq_decode_step) calls, up to max_calls of
 * them, stamps, with the device wall clock, the start of the first workgroup
 * and the end of the last workgroup of its main decode kernel: the fused
 * sink/ring/body scan on the matrix-core path, the vector-ALU scan otherwise
 * (the merge is not included); a kvq_attn_prefill call whose sequences hold
 * sealed records stamps its record launch the same way.  The stamps cost two atomics per workgroup and add no launch or
 * synchronisation to the stream.  kvq_profile_stop waits for the device,
 * writes the kernel durations in microseconds to us[0 .. *n_calls - 1] (us
 * may be NULL; otherwise it must hold max_calls floats), and frees the
 * buffer.  Starting again discards an unfinished profile.  Not for use under
 * graph capture.  Errors: KVQ_ERR_INVALID (bad arguments, stop without
 * start), KVQ_ERR_UNSUPPORTED (plan-only cache), KVQ_ERR_DEVICE. */
kvq_status kvq_profile_start(kvq_cache* cache, int32_t max_calls);
kvq_status kvq_profile_stop(kvq_cache* cache, float* us, int32_t* n_calls);

/* Measurement utility, not part of the method: one streaming read of `bytes`
 * bytes of the device buffer src (16-byte aligned, bytes a positive multiple
 * of 16) by coalesced 16-byte loads from every compute unit, enqueued on
 * stream (non-temporal loads, eight in flight per thread, 16,384 workgroups).
 * Timed over a buffer much larger than the 256 MB Infinity Cache it
 * gives the device's achievable HBM read rate, the ceiling next to which the
 * decode's bytes per second can be read.  out: device, at least
 * KVQ_READ_PROBE_OUT_BYTES bytes; receives one XOR checksum word per wave (it
 * keeps the loads live; the XOR of all its words is the XOR of the buffer's
 * 32-bit words).  Errors: KVQ_ERR_INVALID, KVQ_ERR_DEVICE. */
#define KVQ_READ_PROBE_OUT_BYTES ((size_t)262144)
kvq_status kvq_read_probe(const void* src, size_t bytes, void* out, void* stream);

/* TBQ4 comparator format (KV cache math: "rotate first", the fused
 * rotated-domain decode, and the format table).  A block holds 128 values:
 * y = R x with R the randomized Walsh-Hadamard transform (flip signs s1,
 * Walsh-Hadamard transform in natural order, multiply by 1/sqrt(128), flip
 * signs s2), norm = fp16(|y|), and per value the 4-bit index of the nearest
 * of 16 centroids (the Lloyd-Max quantiser of N(0, 1/128); ties go to the
 * lower index).  Bytes: [fp16 norm, little-endian][64 bytes of indices, value
 * 2j in the low nibble of byte j, 2j+1 in the high], 66 bytes per block.
 * signs: host, four words in the layout of kvq_config.rot_signs.
 *
 * kvq_tbq4_tables: host only, no device needed.  centroids (16 floats,
 * ascending) and boundaries (15 floats, the midpoints) are host outputs;
 * either may be NULL, not both.
 * kvq_tbq4_encode: x device fp16 [n][128]; blocks device [n][66].
 * kvq_tbq4_decode: blocks device [n][66]; out device fp32 [n][128], the
 * original domain (R^T of centroid x norm).
 * kvq_tbq4_attn_decode: one decode step over a TBQ4 cache, the query rotated
 * once, keys and values read as centroid x norm, every split-K partial
 * rotated back once, then merged under one softmax.  q device fp16
 * [n_seqs][n_q_heads][head_dim] (query head i reads KV head i / g, g =
 * n_q_heads / n_kv_heads <= 16); k_blocks, v_blocks device
 * [n_seqs][n_kv_heads][cap][head_dim / 128][66] (head_dim 128 or 256; each
 * 128-value block is its own TBQ4 block); seq_len host, n_seqs tokens counts
 * in 1 .. cap; out device [n_seqs][n_q_heads][head_dim] fp32 or fp16
 * (out_dtype); softmax(scale q.k).  workspace device, ws_bytes >=
 * kvq_tbq4_workspace_bytes(n_seqs, ..., max_len) for any max_len >= the
 * longest seq_len.  All work is queued on `stream`; nothing waits.
 * Errors: KVQ_ERR_INVALID (range or NULL), KVQ_ERR_UNSUPPORTED (head_dim),
 * KVQ_ERR_CAPACITY (workspace), KVQ_ERR_DEVICE. */
kvq_status kvq_tbq4_tables(float* centroids, float* boundaries);

/* tq5_0 and tq6_0 comparator blocks (SJ-KVaRN section 6: the rotated 5-bit
 * format, 82 bytes per 128 values; the 6-bit one, 98 bytes, is the staging
 * format's quantiser).  Per 128-value block: y = R x (the TBQ4 rotation
 * above, exact and rounded once to fp32), d = fp16(max|y| / L) with
 * L = 2^(bits-1) - 1, q = clamp(rne(y * fp32(1 / d)), -L, L), codes
 * u = q + 2^(bits-1) (all 2^(bits-1) when d = 0).  Bytes: [fp16 d,
 * little-endian][16 * bits bytes: LSB-first stream, value k in bits
 * bits*k .. bits*k + bits - 1].  bits: 5 or 6 (else KVQ_ERR_UNSUPPORTED).
 * kvq_tq_encode: x device fp16 [n][128]; blocks device [n][2 + 16 bits].
 * kvq_tq_decode: out device fp32 [n][128], R^T (d (u - 2^(bits-1))).
 * signs: host, as for TBQ4.  Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED,
 * KVQ_ERR_DEVICE. */
kvq_status kvq_tq_encode(const void* x, int64_t n, int32_t bits, const uint64_t* signs, void* blocks, void* stream);
kvq_status kvq_tq_decode(const void* blocks, int64_t n, int32_t bits, const uint64_t* signs, float* out,
                         void* stream);
kvq_status kvq_tbq4_encode(const void* x, int64_t n, const uint64_t* signs, void* blocks, void* stream);
kvq_status kvq_tbq4_decode(const void* blocks, int64_t n, const uint64_t* signs, float* out, void* stream);
kvq_status kvq_tbq4_workspace_bytes(int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int64_t max_len, size_t* bytes);
kvq_status kvq_tbq4_attn_decode(const void* q, const void* k_blocks, const void* v_blocks, int32_t n_seqs,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int64_t cap,
                                const int64_t* seq_len, const uint64_t* signs, float scale, void* out,
                                int32_t out_dtype, void* workspace, size_t ws_bytes, void* stream);

const char* kvq_status_string(kvq_status status);
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
