// Host runtime behind include/kvq.h: configuration checks, arena carving, the
// per-(sequence, layer) counts, the journaled adaptive seal rule, the split-K
// work plan, and kernel launches on the caller's stream.  All state needed to
// size a launch lives on the host, so no call waits for the device except
// kvq_export / kvq_import.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_layout.h"

namespace kvq {
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_read_probe(const void* src, int64_t bytes, void* out, hipStream_t stream);
hipError_t launch_seal(const SealArgs& a, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs& a, int grid_x, hipStream_t stream);
hipError_t launch_decode_main(const DecodeArgs& a, int n_items, hipStream_t stream);
hipError_t launch_decode_ring(const DecodeArgs& a, int n_items, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_prefill_body(const PrefillArgs& a, int nt, hipStream_t stream);
hipError_t launch_prefill_ring(const PrefillArgs& a, int nt, hipStream_t stream);
int prefill_row_tiles(int D, int rows, bool body);
int prefill_lds_bytes(int D, int kb, int nt, bool body);
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_tbq4_encode(const Tbq4CodecArgs& a, hipStream_t stream);
hipError_t launch_tbq4_decode(const Tbq4CodecArgs& a, hipStream_t stream);
hipError_t launch_tbq4_attn(const Tbq4AttnArgs& a, int grid_x, hipStream_t stream);
hipError_t launch_tq_codec(const Tbq4CodecArgs& a, int bits, bool encode, hipStream_t stream);
}  // namespace kvq

using namespace kvq;
static_assert(kNoAllocScratchBytes == KVQ_NOALLOC_SCRATCH_BYTES, "scratch size as the header states it");
static_assert((size_t)kReadProbeBlocks * 4 * 4 == KVQ_READ_PROBE_OUT_BYTES, "read probe output as the header states it");

struct kvq_cache {
  kvq_config cfg;
  Layout y;
  uint8_t* arena;
  bool plan_only;
  int32_t path;
  int32_t n_cu;
  uint32_t signs[8];
  unsigned long long* prof_ts = nullptr;  // profiling: {start, end} wall-clock stamps per decode call
  int32_t prof_n = 0, prof_used = 0;
  std::vector<int64_t> n_tok;  // [S * L]
  std::vector<int64_t> n_rec;  // [S * L]
  int64_t& tok(int s, int l) { return n_tok[(size_t)s * y.L + l]; }
  int64_t& rec(int s, int l) { return n_rec[(size_t)s * y.L + l]; }
  int64_t tok(int s, int l) const { return n_tok[(size_t)s * y.L + l]; }
  int64_t rec(int s, int l) const { return n_rec[(size_t)s * y.L + l]; }
  int64_t ring_len(int s, int l) const { return std::max<int64_t>(0, tok(s, l) - kSink - kGroup * rec(s, l)); }
};

static thread_local std::string g_err;

static kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

static kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

static kvq_status check_config(const kvq_config* c) {
  if (!c) return fail(KVQ_ERR_INVALID, "config is NULL");
  if (c->n_layers < 1 || c->n_kv_heads < 1 || c->max_seqs < 1)
    return fail(KVQ_ERR_INVALID, "n_layers, n_kv_heads and max_seqs must be >= 1");
  if (c->head_dim != 128 && c->head_dim != 256 && c->head_dim != 512)
    return fail(KVQ_ERR_INVALID, "head_dim must be 128, 256 or 512 (got %d)", c->head_dim);
  if (c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads != 0 ||
      c->n_q_heads / c->n_kv_heads > kMaxGroup)
    return fail(KVQ_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads, at most %d per KV head", kMaxGroup);
  if (c->tail_min < kGroup || c->tail_min % kGroup != 0 || c->tail_max < c->tail_min)
    return fail(KVQ_ERR_INVALID, "need tail_min a positive multiple of 128 and tail_min <= tail_max");
  if (c->margin < 0) return fail(KVQ_ERR_INVALID, "margin must be >= 0");
  if (c->max_ctx < 1 || c->max_ctx > ((int64_t)1 << 31) - kGroup)
    return fail(KVQ_ERR_INVALID, "max_ctx out of range");
  if ((c->k_bits != 2 && c->k_bits != 3 && c->k_bits != 4 && c->k_bits != 8) ||
      (c->v_bits != 2 && c->v_bits != 3 && c->v_bits != 4) || (c->v_bits == 4) != (c->k_bits >= 4))
    return fail(KVQ_ERR_INVALID, "supported bodies: k_bits 4 or 8 with v_bits 4; k_bits 2 or 3 with v_bits 2 or 3");
  if (c->sinkhorn_passes < 0 || c->sinkhorn_passes > 64)
    return fail(KVQ_ERR_INVALID, "sinkhorn_passes must be in [0, 64]");
  if ((int64_t)c->tail_max + c->margin > (1 << 28)) return fail(KVQ_ERR_INVALID, "ring too large");
  if (c->flags & ~KVQ_FLAG_PLAN_ONLY) return fail(KVQ_ERR_INVALID, "unknown flags");
  if ((c->stage_fmt != KVQ_STAGE_TQ6 && c->stage_fmt != KVQ_STAGE_F16) || c->reserved != 0)
    return fail(KVQ_ERR_INVALID, "stage_fmt must be KVQ_STAGE_TQ6 or KVQ_STAGE_F16 (reserved 0)");
  return KVQ_OK;
}

static Layout make_layout(const kvq_config& c) {
  Layout y{};
  y.S = c.max_seqs;
  y.L = c.n_layers;
  y.H = c.n_kv_heads;
  y.D = c.head_dim;
  y.NB = c.head_dim / kQBlock;
  y.cap = (int32_t)round_up((int64_t)c.tail_max + c.margin, kGroup);
  y.sub = c.head_dim == 128 ? 128 : 256;
  y.nsub = c.head_dim / y.sub;
  y.kbits = c.k_bits;
  y.vbits = c.v_bits;
  y.max_rec = (int32_t)std::max<int64_t>(0, (c.max_ctx - kSink) / kGroup);
  y.f16ring = c.stage_fmt == KVQ_STAGE_F16;
  y.kcode_bytes = (int64_t)kGroup * y.sub * y.kbits / 8;
  y.vcode_bytes = (int64_t)y.sub * kGroup * y.vbits / 8;
  y.sub_bytes = y.kcode_bytes + y.vcode_bytes + 4 * (y.sub + 2 * kGroup);
  y.rec_bytes = y.nsub * y.sub_bytes;
  const int64_t slh = (int64_t)y.S * y.L * y.H;
  int64_t off = 0;
  y.off_sink = off;
  off = round_up(off + slh * 2 * kSink * y.D * 2, 256);
  y.off_rcode = off;
  off = round_up(off + slh * 2 * y.cap * (int64_t)ring_row_bytes(y), 256);
  y.off_rscale = off;  // f16 staging has no block scales
  off = round_up(off + (y.f16ring ? 0 : slh * 2 * y.cap * (int64_t)y.NB * 2), 256);
  y.off_body = off;
  off = round_up(off + slh * y.max_rec * y.rec_bytes, 256);
  y.total = off;
  return y;
}

// Split-K plan.  Vector-ALU path: ring chunks of a multiple of 128 tokens and
// body chunks of a fixed number of records, sized so that a sequence never has
// more than kMaxChunks partials.
static int ring_chunk_tokens(const Layout& y) {
  return kGroup * (int)std::max<int64_t>(1, (y.cap / kGroup + 1023) / 1024);
}
static int valu_rec_per_chunk(const Layout& y) { return std::max(1, (y.max_rec + 2999) / 3000); }
static int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}
// matrix-core body scan (fused with the sink and ring): every shape the cache
// accepts (head_dim 128, 256 or 512; 4- or 8-bit K; 4-bit V)
static bool mfma_supported(const Layout& y) {
  if (y.vbits != 4)  // low-bit bodies: 256-wide heads (other widths take the vector-ALU scan)
    return y.D == 256 && (y.kbits == 2 || y.kbits == 3) && (y.vbits == 2 || y.vbits == 3);
  return (y.kbits == 4 || y.kbits == 8) && (y.D == 128 || y.D == 256 || y.D == 512);
}
// matrix-core sink and ring scan on its own: head_dim 128 or 256
static bool staged_supported(const Layout& y) { return y.D == 128 || y.D == 256; }
static constexpr int kRingStep = 64;         // tokens per step of the matrix-core sink/ring scan
static constexpr int kBlockStepTokens = 64;  // tokens per step of the block-attention sink/ring scan
static constexpr int kStagedRingChunk = 256; // ring tokens per chunk next to a vector-ALU body scan
// resident workgroups per CU of the fused kernel (512-wide heads: one, for the LDS of their sink/ring scan)
static int body_wg_per_cu(const Layout& y) { return y.D == 512 ? 1 : 2; }

// Matrix-core plan.  Work in units of one record (about one 64-token ring
// step; the sink is two).  All work items run in one round, two workgroups per
// compute unit (one for 512-wide heads); the first workgroup on a unit (grid
// index below the unit count) scans 1.4 times as fast as the second (the
// kernel gives it that much more of the records).  T = work / capacity is the time of the round in
// second-workgroup records; ring chunks take floor(T) steps (ring items come
// last in the grid, second on their unit), the remaining slots split the
// body records (body items are issued first).
struct MfmaPlan {
  int ring_chunk;
  int body_slots;      // workgroups left for body chunks
  double body_total;   // records of all the launch's (sequence, head) pairs
};
static MfmaPlan mfma_plan(const kvq_cache* c, const std::vector<int64_t>& n_rec, const std::vector<int64_t>& ring,
                          int reserved) {
  const int H = c->y.H;
  double body = 0, other = 0;
  for (size_t i = 0; i < n_rec.size(); ++i) {
    body += (double)H * n_rec[i];
    other += (double)H * ((ring[i] + kRingStep - 1) / kRingStep + 2);
  }
  // `reserved` workgroups (the append items of a fused step) are short and
  // leave their slots idle once done
  const int n_cu = c->n_cu ? c->n_cu : 256;
  const int slots = std::max(1, body_wg_per_cu(c->y) * n_cu - reserved);
  const double capacity = std::max(1.0, slots + 0.4 * std::min(n_cu, slots));
  const double per = std::max(1.0, (body + other) / capacity);
  MfmaPlan p;
  p.ring_chunk = kRingStep * std::max(1, (int)std::floor(per));
  int64_t ring_items = 0;
  for (size_t i = 0; i < ring.size(); ++i) ring_items += (int64_t)H * (1 + (ring[i] + p.ring_chunk - 1) / p.ring_chunk);
  p.body_slots = (int)std::max<int64_t>(H, slots - ring_items);
  p.body_total = body;
  return p;
}

static DecodeSeq plan_seq(const kvq_cache* c, int s, int layer, int rc, int n_body_chunks) {
  DecodeSeq d{};
  d.slot = s;
  const int64_t nt = c->tok(s, layer);
  d.n_sink = (int32_t)std::min<int64_t>(nt, kSink);
  d.n_rec = (int32_t)c->rec(s, layer);
  d.ring_len = (int32_t)c->ring_len(s, layer);
  d.ring0 = (int32_t)(((int64_t)kGroup * d.n_rec) % c->y.cap);
  d.n_ring_chunks = (d.ring_len + rc - 1) / rc;
  d.n_body_chunks = n_body_chunks;
  d.n_chunks = 1 + d.n_ring_chunks + d.n_body_chunks;
  return d;
}

static void fill_signs(const kvq_config& c, uint32_t* out) {
  for (int w = 0; w < 4; ++w) {
    out[2 * w] = (uint32_t)(c.rot_signs[w] & 0xFFFFFFFFu);
    out[2 * w + 1] = (uint32_t)(c.rot_signs[w] >> 32);
  }
}

extern "C" {

kvq_status kvq_read_probe(const void* src, size_t bytes, void* out, void* stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    return fail(KVQ_ERR_INVALID, "read probe: src and out non-NULL, src 16-byte aligned, bytes a positive multiple of 16");
  const hipError_t e = launch_read_probe(src, (int64_t)bytes, out, (hipStream_t)stream);
  return e == hipSuccess ? KVQ_OK : hip_fail(e, "read probe launch");
}

const char* kvq_status_string(kvq_status st) {
  switch (st) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_CAPACITY: return "capacity exceeded";
    case KVQ_ERR_RING_FULL: return "staging ring full";
    case KVQ_ERR_SEALED: return "sealed records cannot be rewritten";
    case KVQ_ERR_DEVICE: return "device error";
    case KVQ_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* kvq_last_error(void) { return g_err.c_str(); }

kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* device_bytes) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!device_bytes) return fail(KVQ_ERR_INVALID, "device_bytes is NULL");
  *device_bytes = (cfg->flags & KVQ_FLAG_PLAN_ONLY) ? 0 : (size_t)make_layout(*cfg).total;
  return KVQ_OK;
}

kvq_status kvq_cache_create(const kvq_config* cfg, void* device_arena, size_t arena_bytes, kvq_cache** out) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_ERR_INVALID, "out is NULL");
  const bool plan_only = (cfg->flags & KVQ_FLAG_PLAN_ONLY) != 0;
  Layout y = make_layout(*cfg);
  if (!plan_only) {
    if (!device_arena) return fail(KVQ_ERR_INVALID, "device_arena is NULL");
    if ((uintptr_t)device_arena % 256 != 0) return fail(KVQ_ERR_INVALID, "device_arena must be 256-byte aligned");
    if (arena_bytes < (size_t)y.total)
      return fail(KVQ_ERR_CAPACITY, "arena has %zu bytes, needs %lld", arena_bytes, (long long)y.total);
  }
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return fail(KVQ_ERR_CAPACITY, "out of host memory");
  c->cfg = *cfg;
  c->y = y;
  c->arena = plan_only ? nullptr : (uint8_t*)device_arena;
  c->plan_only = plan_only;
  c->path = KVQ_PATH_AUTO;
  c->n_cu = plan_only ? 0 : device_cu_count();  // sizes the matrix-core body chunks
  fill_signs(*cfg, c->signs);
  c->n_tok.assign((size_t)y.S * y.L, 0);
  c->n_rec.assign((size_t)y.S * y.L, 0);
  *out = c;
  return KVQ_OK;
}

static void profile_clear(kvq_cache* c);

kvq_status kvq_cache_destroy(kvq_cache* c) {
  if (c) profile_clear(c);
  delete c;
  return KVQ_OK;
}

static kvq_status check_seqs(const kvq_cache* c, const int32_t* ids, int32_t n) {
  if (n < 0) return fail(KVQ_ERR_INVALID, "n_seqs < 0");
  if (n > 0 && !ids) return fail(KVQ_ERR_INVALID, "seq_ids is NULL");
  std::vector<char> seen((size_t)c->y.S, 0);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= c->y.S) return fail(KVQ_ERR_INVALID, "seq id %d out of range", ids[i]);
    if (seen[ids[i]]) return fail(KVQ_ERR_INVALID, "seq id %d listed twice", ids[i]);
    seen[ids[i]] = 1;
  }
  return KVQ_OK;
}

kvq_status kvq_append(kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs, const void* k,
                      const void* v, int32_t n_tok, void* stream) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (layer < 0 || layer >= c->y.L) return fail(KVQ_ERR_INVALID, "layer %d out of range", layer);
  if (n_tok < 0) return fail(KVQ_ERR_INVALID, "n_tok < 0");
  kvq_status st = check_seqs(c, seq_ids, n_seqs);
  if (st != KVQ_OK) return st;
  if (n_seqs == 0 || n_tok == 0) return KVQ_OK;
  if (!c->plan_only && (!k || !v)) return fail(KVQ_ERR_INVALID, "k or v is NULL");
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    if (c->tok(s, layer) + n_tok > c->cfg.max_ctx)
      return fail(KVQ_ERR_CAPACITY, "sequence %d would exceed max_ctx %lld", s, (long long)c->cfg.max_ctx);
    const int64_t ring_after = std::max<int64_t>(0, c->tok(s, layer) + n_tok - kSink - kGroup * c->rec(s, layer));
    if (ring_after > c->y.cap)
      return fail(KVQ_ERR_RING_FULL, "sequence %d: ring would hold %lld of %d slots; seal first", s,
                  (long long)ring_after, c->y.cap);
  }
  if (!c->plan_only) {
    const int64_t per_seq = (int64_t)n_tok * c->y.H * c->y.D;
    for (int b0 = 0; b0 < n_seqs; b0 += kMaxLaunchSeqs) {
      AppendArgs a{};
      a.k = (const uint16_t*)k + b0 * per_seq;
      a.v = (const uint16_t*)v + b0 * per_seq;
      a.arena = c->arena;
      a.y = c->y;
      a.layer = layer;
      a.n_tok = n_tok;
      a.n_seqs = std::min(kMaxLaunchSeqs, n_seqs - b0);
      std::memcpy(a.signs, c->signs, sizeof a.signs);
      for (int b = 0; b < a.n_seqs; ++b) {
        a.slot[b] = seq_ids[b0 + b];
        a.pos0[b] = c->tok(seq_ids[b0 + b], layer);
      }
      hipError_t e = launch_append(a, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "append launch");
    }
  }
  for (int i = 0; i < n_seqs; ++i) c->tok(seq_ids[i], layer) += n_tok;
  return KVQ_OK;
}

static int64_t groups_to_seal(int64_t ring_len, const kvq_config& cfg, int mode) {
  if (mode == KVQ_SEAL_IF_FULL && ring_len < cfg.tail_max) return 0;
  return std::max<int64_t>(0, (ring_len - cfg.tail_min) / kGroup);
}

kvq_status kvq_seal(kvq_cache* c, int32_t layer, int32_t mode, void* stream, int32_t* groups_sealed) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (layer < -1 || layer >= c->y.L) return fail(KVQ_ERR_INVALID, "layer %d out of range", layer);
  if (mode != KVQ_SEAL_IF_FULL && mode != KVQ_SEAL_TO_MIN) return fail(KVQ_ERR_INVALID, "bad seal mode %d", mode);
  int64_t total = 0;
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->y.L : layer + 1;
  // every (sequence, layer) with groups due, all layers in the same launches:
  // the tiles are independent, and one wide launch keeps the whole GPU busy
  std::vector<SealTask> tasks;
  for (int l = l0; l < l1; ++l) {
    for (int s = 0; s < c->y.S; ++s) {
      const int64_t g = groups_to_seal(c->ring_len(s, l), c->cfg, mode);
      if (g <= 0) continue;
      SealTask t{};
      t.slot = s;
      t.layer = l;
      t.rec0 = (int32_t)c->rec(s, l);
      t.n_groups = (int32_t)g;
      tasks.push_back(t);
    }
  }
  for (size_t t0 = 0; t0 < tasks.size(); t0 += kMaxSealTasks) {
    SealArgs a{};
    a.arena = c->arena;
    a.y = c->y;
    a.passes = c->cfg.sinkhorn_passes;
    std::memcpy(a.signs, c->signs, sizeof a.signs);
    a.n_tasks = (int32_t)std::min<size_t>(kMaxSealTasks, tasks.size() - t0);
    int32_t first = 0;
    for (int i = 0; i < a.n_tasks; ++i) {
      a.task[i] = tasks[t0 + i];
      a.task[i].first = first;
      first += a.task[i].n_groups;
    }
    a.total_groups = first;
    if (!c->plan_only) {
      hipError_t e = launch_seal(a, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "seal launch");
    }
    for (int i = 0; i < a.n_tasks; ++i) {
      c->rec(a.task[i].slot, a.task[i].layer) += a.task[i].n_groups;
      total += a.task[i].n_groups;
    }
  }
  if (groups_sealed) *groups_sealed = (int32_t)total;
  return KVQ_OK;
}

static int max_chunks_bound(const kvq_cache* c) {
  // the most chunks any path makes: ring chunks of at least 64 tokens; body
  // chunks of the vector-ALU path, or of the matrix-core path, whose records
  // per chunk grow with the record total so that a sequence gets at most
  // 2 n_cu / H + 1 of them
  const int rc = std::min(ring_chunk_tokens(c->y), kRingStep);
  const int rpc = valu_rec_per_chunk(c->y);
  int body = (c->y.max_rec + rpc - 1) / rpc;
  if (mfma_supported(c->y)) {
    const int n_cu = c->n_cu ? c->n_cu : 256;
    body = std::max(body, std::min(c->y.max_rec, (body_wg_per_cu(c->y) * n_cu + c->y.H - 1) / c->y.H + 1));
  }
  return 1 + (c->y.cap + rc - 1) / rc + body + 1;  // + the new token of a fused decode step
}

kvq_status kvq_workspace_bytes(const kvq_cache* c, int32_t n_seqs, size_t* bytes) {
  if (!c || !bytes || n_seqs < 0) return fail(KVQ_ERR_INVALID, "bad arguments");
  *bytes = (size_t)n_seqs * c->cfg.n_q_heads * max_chunks_bound(c) * part_stride(c->y.D) * sizeof(float);
  return KVQ_OK;
}

kvq_status kvq_set_decode_path(kvq_cache* c, int32_t path) {
  if (!c || path < KVQ_PATH_AUTO || path > KVQ_PATH_MFMA) return fail(KVQ_ERR_INVALID, "bad decode path");
  c->path = path;
  return KVQ_OK;
}

static kvq_status check_decode_args(const kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs,
                                    const void* q, void* out, int32_t out_dtype, void* workspace) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (c->plan_only) return fail(KVQ_ERR_UNSUPPORTED, "decode on a plan-only cache");
  if (layer < 0 || layer >= c->y.L) return fail(KVQ_ERR_INVALID, "layer %d out of range", layer);
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_F16) return fail(KVQ_ERR_INVALID, "bad out_dtype");
  kvq_status st = check_seqs(c, seq_ids, n_seqs);
  if (st != KVQ_OK) return st;
  if (n_seqs > 0 && (!q || !out || !workspace)) return fail(KVQ_ERR_INVALID, "q, out and workspace must be non-NULL");
  return KVQ_OK;
}

// Decode launches.  With k_new/v_new (fused decode step, matrix-core path
// only) the caller has checked that every sequence's new token goes to the
// ring and that no seal is due; the token is written and counted here.
static kvq_status decode_impl(kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs, const void* q,
                              void* out, int32_t out_dtype, float scale, void* workspace, size_t ws_bytes,
                              void* stream, const void* k_new, const void* v_new, bool noalloc = false) {
  const bool fused = k_new != nullptr;
  const bool use_mfma = c->path != KVQ_PATH_VALU && mfma_supported(c->y);
  const bool staged = c->path != KVQ_PATH_VALU && staged_supported(c->y);
  if (c->path == KVQ_PATH_MFMA && !use_mfma)
    return fail(KVQ_ERR_UNSUPPORTED, "matrix-core body scan: 4/4 or 8/4 at head_dim 128, 256, 512; 2- or 3-bit "
                                     "bodies at head_dim 256");
  std::vector<int64_t> n_rec(n_seqs), ring(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    if (c->tok(seq_ids[i], layer) < 1) return fail(KVQ_ERR_INVALID, "sequence %d holds no tokens", seq_ids[i]);
    n_rec[i] = c->rec(seq_ids[i], layer);
    ring[i] = c->ring_len(seq_ids[i], layer);
  }
  int rc;
  MfmaPlan mp{};
  if (use_mfma) {
    mp = mfma_plan(c, n_rec, ring, fused ? std::min(n_seqs, kMaxLaunchSeqs) * c->y.H : 0);
    rc = mp.ring_chunk;
  } else {
    rc = staged ? kStagedRingChunk : ring_chunk_tokens(c->y);
  }
  const int valu_rpc = valu_rec_per_chunk(c->y);
  std::vector<DecodeSeq> plan(n_seqs);
  int max_chunks = 1;
  for (int i = 0; i < n_seqs; ++i) {
    int nb;
    if (use_mfma)  // this sequence's share of the body slots, whole per KV head
      nb = n_rec[i] == 0 ? 0
                         : (int)std::min<int64_t>(n_rec[i], std::max<int64_t>(1, (int64_t)std::floor(
                               (double)n_rec[i] * c->y.H * mp.body_slots / std::max(1.0, mp.body_total) / c->y.H)));
    else
      nb = (int)((n_rec[i] + valu_rpc - 1) / valu_rpc);
    plan[i] = plan_seq(c, seq_ids[i], layer, rc, nb);
    if (fused) {
      plan[i].app_slot = (int32_t)((plan[i].ring0 + plan[i].ring_len) % c->y.cap);
      plan[i].app_chunk = plan[i].n_chunks++;
    }
    max_chunks = std::max(max_chunks, plan[i].n_chunks);
  }
  if (max_chunks > kMaxChunks) return fail(KVQ_ERR_CAPACITY, "too many split-K chunks");
  const int Hq = c->cfg.n_q_heads, D = c->y.D;
  const size_t need = (size_t)n_seqs * Hq * max_chunks * part_stride(D) * sizeof(float);
  if (ws_bytes < need)
    return noalloc ? fail(KVQ_ERR_CAPACITY,
                          "the allocation-free decode holds %zu bytes of split-K partials per GPU; this call needs "
                          "%zu (fewer sequences per call, or kvq_attn_decode with a workspace)", ws_bytes, need)
                   : fail(KVQ_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  const size_t out_elem = out_dtype == KVQ_OUT_F16 ? 2 : 4;
  for (int b0 = 0; b0 < n_seqs; b0 += kMaxLaunchSeqs) {
    DecodeArgs a{};
    a.arena = c->arena;
    a.y = c->y;
    a.n_seqs = std::min(kMaxLaunchSeqs, n_seqs - b0);
    a.q = (const uint16_t*)q + (int64_t)b0 * Hq * D;
    if (fused) {
      a.k_new = (const uint16_t*)k_new + (int64_t)b0 * c->y.H * D;
      a.v_new = (const uint16_t*)v_new + (int64_t)b0 * c->y.H * D;
    }
    a.part = (float*)workspace + (int64_t)b0 * Hq * max_chunks * part_stride(D);
    a.scale = scale;
    a.layer = layer;
    a.Hq = Hq;
    a.g = Hq / c->y.H;
    a.max_chunks = max_chunks;
    a.ring_chunk = rc;
    std::memcpy(a.signs, c->signs, sizeof a.signs);
    // regions left to the vector-ALU kernel: bit 0 sink, 1 ring, 2 body
    a.valu_regions = (staged ? 0 : 3) | (use_mfma ? 0 : 4);
    int grid_valu = 0, n_body_items = 0, n_ring_items = 0;
    for (int b = 0; b < a.n_seqs; ++b) {
      a.seq[b] = plan[b0 + b];
      n_body_items += c->y.H * a.seq[b].n_body_chunks;
      n_ring_items += c->y.H * (1 + a.seq[b].n_ring_chunks);
      grid_valu = std::max(grid_valu, (a.valu_regions & 4) ? a.seq[b].n_chunks : 1 + a.seq[b].n_ring_chunks);
    }
    hipError_t e = hipSuccess;
    if (b0 == 0 && c->prof_used < c->prof_n) a.prof_ts = c->prof_ts + 2 * c->prof_used++;
    if (use_mfma) {
      a.n_app_items = fused ? a.n_seqs * c->y.H : 0;
      a.n_body_items = n_body_items;
      a.n_old = c->n_cu ? c->n_cu : 256;
      e = launch_decode_main(a, a.n_app_items + n_body_items + n_ring_items, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "decode launch");
    } else {
      if (staged) {
        DecodeArgs r = a;
        r.prof_ts = nullptr;  // stamps belong to the main scan
        e = launch_decode_ring(r, n_ring_items, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "sink/ring decode launch");
      }
      e = launch_decode_valu(a, grid_valu, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "decode launch");
    }
    MergeArgs m{};
    m.part = a.part;
    m.out = (uint8_t*)out + (size_t)b0 * Hq * D * out_elem;
    m.D = D;
    m.Hq = Hq;
    m.n_seqs = a.n_seqs;
    m.max_chunks = max_chunks;
    m.out_f16 = out_dtype == KVQ_OUT_F16;
    m.n_rows = 1;
    for (int b = 0; b < a.n_seqs; ++b) m.n_chunks[b] = a.seq[b].n_chunks;
    e = launch_merge(m, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  if (fused)
    for (int i = 0; i < n_seqs; ++i) c->tok(seq_ids[i], layer) += 1;
  return KVQ_OK;
}

kvq_status kvq_attn_decode(kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs, const void* q,
                           void* out, int32_t out_dtype, float scale, void* workspace, size_t ws_bytes,
                           void* stream) {
  kvq_status st = check_decode_args(c, layer, seq_ids, n_seqs, q, out, out_dtype, workspace);
  if (st != KVQ_OK || n_seqs == 0) return st;
  return decode_impl(c, layer, seq_ids, n_seqs, q, out, out_dtype, scale, workspace, ws_bytes, stream, nullptr,
                     nullptr);
}

kvq_status kvq_attn_decode_noalloc(kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs,
                                   const void* q, void* out, int32_t out_dtype, float scale, void* stream) {
  void* scratch = nullptr;
  kvq_status st = check_decode_args(c, layer, seq_ids, n_seqs, q, out, out_dtype, (void*)&scratch);
  if (st != KVQ_OK || n_seqs == 0) return st;
  hipError_t e = noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return decode_impl(c, layer, seq_ids, n_seqs, q, out, out_dtype, scale, scratch, kNoAllocScratchBytes, stream,
                     nullptr, nullptr, true);
}

kvq_status kvq_decode_step(kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs, const void* k,
                           const void* v, const void* q, void* out, int32_t out_dtype, float scale,
                           void* workspace, size_t ws_bytes, void* stream, int32_t* groups_sealed) {
  kvq_status st = check_decode_args(c, layer, seq_ids, n_seqs, q, out, out_dtype, workspace);
  if (st != KVQ_OK) return st;
  if (groups_sealed) *groups_sealed = 0;
  if (n_seqs == 0) return KVQ_OK;
  if (!k || !v) return fail(KVQ_ERR_INVALID, "k or v is NULL");
  // one launch when the matrix-core path runs, every new token lands in the
  // ring and the seal-if-full that follows the append would seal nothing (in
  // any sequence of the layer); otherwise the three calls in turn
  bool fused = c->path != KVQ_PATH_VALU && mfma_supported(c->y);
  std::vector<char> listed((size_t)c->y.S, 0);
  for (int i = 0; fused && i < n_seqs; ++i) {
    const int s = seq_ids[i];
    listed[s] = 1;
    if (c->tok(s, layer) < kSink || c->tok(s, layer) + 1 > c->cfg.max_ctx ||
        c->ring_len(s, layer) + 1 > c->y.cap ||
        groups_to_seal(c->ring_len(s, layer) + 1, c->cfg, KVQ_SEAL_IF_FULL) > 0)
      fused = false;
  }
  for (int s = 0; fused && s < c->y.S; ++s)
    if (!listed[s] && groups_to_seal(c->ring_len(s, layer), c->cfg, KVQ_SEAL_IF_FULL) > 0) fused = false;
  if (!fused) {
    st = kvq_append(c, layer, seq_ids, n_seqs, k, v, 1, stream);
    if (st == KVQ_OK) st = kvq_seal(c, layer, KVQ_SEAL_IF_FULL, stream, groups_sealed);
    if (st == KVQ_OK) st = kvq_attn_decode(c, layer, seq_ids, n_seqs, q, out, out_dtype, scale, workspace, ws_bytes, stream);
    return st;
  }
  return decode_impl(c, layer, seq_ids, n_seqs, q, out, out_dtype, scale, workspace, ws_bytes, stream, k, v);
}

static void profile_clear(kvq_cache* c) {
  if (c->prof_ts) (void)hipFree(c->prof_ts);
  c->prof_ts = nullptr;
  c->prof_n = c->prof_used = 0;
}

// ---------------------------------------------------------------------------
// Block attention (prefill chunks, verify blocks).  Plan: rows n_q g per
// (sequence, KV head) in row blocks of 16 nt (the record and the sink/ring
// launches each have their own nt); every row gets the same chunks as the
// others of its sequence: the sink, then ring chunks, then record chunks.
// The two launches run one after the other, so each is sized to fill the
// device on its own: record chunks to about four workgroups per resident slot,
// ring chunks (multiples of one 64-token step) to one round of the slots for
// few row blocks and about two per slot otherwise, each at most
// kMaxBlockChunks per sequence.
static bool prefill_supported(const Layout& y) {
  if (y.vbits == 4) return y.kbits == 4 || y.kbits == 8;
  return y.D == 256;  // the 2- and 3-bit bodies: 256-wide heads (as their matrix-core decode)
}

struct BlockBudget {
  int nt, n_rb, nt_ring, n_rb_ring, body_chunks, ring_chunks;
};
static BlockBudget prefill_budget(const kvq_cache* c, int n_seqs, int n_q) {
  const int D = c->y.D, g = c->cfg.n_q_heads / c->y.H, rows = n_q * g;
  BlockBudget b;
  b.nt = prefill_row_tiles(D, rows, true);
  b.nt_ring = prefill_row_tiles(D, rows, false);
  b.n_rb = (rows + 16 * b.nt - 1) / (16 * b.nt);
  b.n_rb_ring = (rows + 16 * b.nt_ring - 1) / (16 * b.nt_ring);
  const int64_t n_cu = c->n_cu ? c->n_cu : 256;
  auto chunks = [&](int lds, int n_rb, int per_slot) {
    const int64_t slots = n_cu * std::max(1, (160 << 10) / std::max(1, lds));
    const int64_t pairs = std::max<int64_t>(1, (int64_t)std::max(1, n_seqs) * c->y.H * n_rb);
    return (int)std::min<int64_t>(kMaxBlockChunks, std::max<int64_t>(1, (per_slot * slots + pairs - 1) / pairs));
  };
  b.body_chunks = chunks(prefill_lds_bytes(D, c->y.kbits, b.nt, true), b.n_rb, 4);
  {
    // few row blocks (verify-sized blocks): the sink/ring launch in one round of
    // the resident slots, (1 + ring chunks) items per row block, so that no item
    // waits for a second round; many row blocks: ~2 items per slot (measured:
    // one round was 14 % faster for an 8-token block, 8 % slower for 512 tokens)
    const int lds = prefill_lds_bytes(D, c->y.kbits, b.nt_ring, false);
    const int64_t slots = n_cu * std::max(1, (160 << 10) / std::max(1, lds));
    const int64_t pairs = std::max<int64_t>(1, (int64_t)std::max(1, n_seqs) * c->y.H * b.n_rb_ring);
    const int64_t nr = 2 * pairs <= slots ? slots / pairs - 1 : (2 * slots + pairs - 1) / pairs;
    b.ring_chunks = (int)std::min<int64_t>(kMaxBlockChunks, std::max<int64_t>(1, nr));
  }
  return b;
}

kvq_status kvq_prefill_workspace_bytes(const kvq_cache* c, int32_t n_seqs, int32_t n_q, size_t* bytes) {
  if (!c || !bytes || n_seqs < 0 || n_q < 1 || n_q > kMaxBlock) return fail(KVQ_ERR_INVALID, "bad arguments");
  const BlockBudget bb = prefill_budget(c, n_seqs, n_q);
  *bytes = (size_t)n_seqs * n_q * c->cfg.n_q_heads * (1 + bb.ring_chunks + bb.body_chunks) * part_stride(c->y.D) *
           sizeof(float);
  return KVQ_OK;
}

kvq_status kvq_attn_prefill(kvq_cache* c, int32_t layer, const int32_t* seq_ids, int32_t n_seqs, int32_t n_q,
                            const void* q, void* out, int32_t out_dtype, float scale, void* workspace,
                            size_t ws_bytes, void* stream) {
  kvq_status st = check_decode_args(c, layer, seq_ids, n_seqs, q, out, out_dtype, workspace);
  if (st != KVQ_OK) return st;
  if (n_q < 1 || n_q > kMaxBlock) return fail(KVQ_ERR_INVALID, "n_q %d outside 1..%d", n_q, kMaxBlock);
  if (n_seqs == 0) return KVQ_OK;
  if (!prefill_supported(c->y))
    return fail(KVQ_ERR_UNSUPPORTED, "block attention over 2- and 3-bit bodies: head_dim 256 only");
  for (int i = 0; i < n_seqs; ++i)
    if (c->tok(seq_ids[i], layer) < n_q)
      return fail(KVQ_ERR_INVALID, "sequence %d holds %lld tokens, fewer than the block's %d", seq_ids[i],
                  (long long)c->tok(seq_ids[i], layer), n_q);
  const int H = c->y.H, Hq = c->cfg.n_q_heads, D = c->y.D, g = Hq / H;
  const BlockBudget bb = prefill_budget(c, n_seqs, n_q);
  const int nt = bb.nt, nt_ring = bb.nt_ring, n_rb = bb.n_rb, n_rb_ring = bb.n_rb_ring;
  std::vector<PrefillSeq> plan(n_seqs);
  int max_chunks = 1;
  for (int i = 0; i < n_seqs; ++i) {
    PrefillSeq& d = plan[i];
    d = PrefillSeq{};
    const int s = seq_ids[i];
    const int64_t nt_tok = c->tok(s, layer);
    d.slot = s;
    d.n_sink = (int32_t)std::min<int64_t>(nt_tok, kSink);
    d.n_rec = (int32_t)c->rec(s, layer);
    d.ring_len = (int32_t)c->ring_len(s, layer);
    d.ring0 = (int32_t)(((int64_t)kGroup * d.n_rec) % c->y.cap);
    d.p0 = (int32_t)(nt_tok - n_q);
    d.n_body_chunks = std::min(d.n_rec, bb.body_chunks);
    d.ring_chunk = kBlockStepTokens;
    d.n_ring_chunks = 0;
    if (d.ring_len > 0) {
      const int nr = std::min((d.ring_len + kBlockStepTokens - 1) / kBlockStepTokens, bb.ring_chunks);
      d.ring_chunk = (int32_t)round_up((d.ring_len + nr - 1) / nr, kBlockStepTokens);
      d.n_ring_chunks = (d.ring_len + d.ring_chunk - 1) / d.ring_chunk;
    }
    d.n_chunks = 1 + d.n_ring_chunks + d.n_body_chunks;
    max_chunks = std::max(max_chunks, d.n_chunks);
  }
  const size_t need = (size_t)n_seqs * n_q * Hq * max_chunks * part_stride(D) * sizeof(float);
  if (ws_bytes < need) return fail(KVQ_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  const size_t out_elem = out_dtype == KVQ_OUT_F16 ? 2 : 4;
  for (int b0 = 0; b0 < n_seqs; b0 += kMaxLaunchSeqs) {
    PrefillArgs a{};
    a.arena = c->arena;
    a.y = c->y;
    a.n_seqs = std::min(kMaxLaunchSeqs, n_seqs - b0);
    a.q = (const uint16_t*)q + (int64_t)b0 * n_q * Hq * D;
    a.part = (float*)workspace + (int64_t)b0 * n_q * Hq * max_chunks * part_stride(D);
    a.scale = scale;
    a.layer = layer;
    a.Hq = Hq;
    a.g = g;
    a.n_q = n_q;
    a.max_chunks = max_chunks;
    a.n_rb = n_rb;
    std::memcpy(a.signs, c->signs, sizeof a.signs);
    int body_items = 0, ring_items = 0;
    for (int b = 0; b < a.n_seqs; ++b) {
      a.seq[b] = plan[b0 + b];
      a.seq[b].body_item0 = body_items;
      a.seq[b].ring_item0 = ring_items;
      body_items += H * n_rb * a.seq[b].n_body_chunks;
      ring_items += H * n_rb_ring * (1 + a.seq[b].n_ring_chunks);
    }
    a.seq[a.n_seqs].body_item0 = body_items;
    a.seq[a.n_seqs].ring_item0 = ring_items;
    hipError_t e = hipSuccess;
    if (body_items > 0) {
      a.n_items = body_items;
      if (b0 == 0 && c->prof_used < c->prof_n) a.prof_ts = c->prof_ts + 2 * c->prof_used++;
      e = launch_prefill_body(a, nt, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "block attention body launch");
      a.prof_ts = nullptr;
    }
    a.n_items = ring_items;
    a.n_rb = n_rb_ring;
    e = launch_prefill_ring(a, nt_ring, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "block attention sink/ring launch");
    MergeArgs m{};
    m.part = a.part;
    m.out = (uint8_t*)out + (size_t)b0 * n_q * Hq * D * out_elem;
    m.D = D;
    m.Hq = Hq;
    m.n_seqs = a.n_seqs;
    m.max_chunks = max_chunks;
    m.out_f16 = out_dtype == KVQ_OUT_F16;
    m.n_rows = n_q;
    for (int b = 0; b < a.n_seqs; ++b) m.n_chunks[b] = a.seq[b].n_chunks;
    e = launch_merge(m, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return KVQ_OK;
}

kvq_status kvq_profile_start(kvq_cache* c, int32_t max_calls) {
  if (!c || max_calls < 1) return fail(KVQ_ERR_INVALID, "bad arguments");
  if (c->plan_only) return fail(KVQ_ERR_UNSUPPORTED, "profiling a plan-only cache");
  profile_clear(c);
  std::vector<unsigned long long> init((size_t)2 * max_calls);
  for (size_t i = 0; i < init.size(); i += 2) {
    init[i] = 0;      // start of workgroup 0
    init[i + 1] = 0;  // latest end: atomic max
  }
  hipError_t e = hipMalloc((void**)&c->prof_ts, init.size() * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMemcpy(c->prof_ts, init.data(), init.size() * sizeof(unsigned long long), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    profile_clear(c);
    return hip_fail(e, "profile buffer");
  }
  c->prof_n = max_calls;
  return KVQ_OK;
}

kvq_status kvq_profile_stop(kvq_cache* c, float* us, int32_t* n_calls) {
  if (!c || !n_calls) return fail(KVQ_ERR_INVALID, "bad arguments");
  if (!c->prof_ts) return fail(KVQ_ERR_INVALID, "no profile started");
  const int32_t n = c->prof_used;
  std::vector<unsigned long long> ts((size_t)2 * std::max(n, 1));
  int dev = 0, khz = 0;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess && n > 0)
    e = hipMemcpy(ts.data(), c->prof_ts, (size_t)2 * n * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  profile_clear(c);
  if (e != hipSuccess) return hip_fail(e, "profile read");
  if (khz <= 0) return fail(KVQ_ERR_DEVICE, "device reports no wall clock rate");
  for (int32_t i = 0; us && i < n; ++i)
    us[i] = ts[2 * i + 1] >= ts[2 * i] ? (float)((double)(ts[2 * i + 1] - ts[2 * i]) * 1000.0 / khz) : 0.0f;
  *n_calls = n;
  return KVQ_OK;
}

kvq_status kvq_seq_info(const kvq_cache* c, int32_t seq, int32_t layer, int64_t* n_tok, int64_t* n_records,
                        int32_t* ring_len) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (seq < 0 || seq >= c->y.S || layer < 0 || layer >= c->y.L) return fail(KVQ_ERR_INVALID, "seq/layer out of range");
  if (n_tok) *n_tok = c->tok(seq, layer);
  if (n_records) *n_records = c->rec(seq, layer);
  if (ring_len) *ring_len = (int32_t)c->ring_len(seq, layer);
  return KVQ_OK;
}

kvq_status kvq_seq_reset(kvq_cache* c, int32_t seq) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (seq < 0 || seq >= c->y.S) return fail(KVQ_ERR_INVALID, "seq out of range");
  for (int l = 0; l < c->y.L; ++l) {
    c->tok(seq, l) = 0;
    c->rec(seq, l) = 0;
  }
  return KVQ_OK;
}

kvq_status kvq_seq_truncate(kvq_cache* c, int32_t seq, int32_t layer, int64_t n_tok) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (seq < 0 || seq >= c->y.S || layer < -1 || layer >= c->y.L) return fail(KVQ_ERR_INVALID, "seq/layer out of range");
  if (n_tok < 0) return fail(KVQ_ERR_INVALID, "n_tok < 0");
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->y.L : layer + 1;
  for (int l = l0; l < l1; ++l) {
    if (n_tok > c->tok(seq, l)) return fail(KVQ_ERR_INVALID, "truncate cannot grow a sequence");
    if (c->rec(seq, l) > 0 && n_tok < kSink + kGroup * c->rec(seq, l))
      return fail(KVQ_ERR_SEALED, "target %lld is below the sealed boundary %lld", (long long)n_tok,
                  (long long)(kSink + kGroup * c->rec(seq, l)));
  }
  for (int l = l0; l < l1; ++l) c->tok(seq, l) = n_tok;
  return KVQ_OK;
}

// ---------------------------------------------------------------------------
// Whole-sequence save / restore.  A sequence's state is its per-layer counts
// and four spans of the arena (the sequence is the outermost index of every
// region): the sink, the ring codes and the ring scales whole, and the sealed
// records of each (layer, KV head), which are contiguous from record 0.
namespace {
constexpr uint32_t kSaveMagic = 0x5351564Bu;  // "KVQS"
constexpr uint32_t kSaveVersion = 2;
struct SaveHeader {
  uint32_t magic, version;
  // layout fingerprint: a blob restores only into a cache that lays the same
  // bytes out the same way and encodes further tokens the same way
  int32_t L, H, D, NB, cap, kbits, vbits, sinkhorn_passes, stage_fmt, pad;
  int64_t rec_bytes;
  uint64_t rot_signs[4];
};
struct SeqSpans {
  int64_t sink_off, sink_n, rcode_off, rcode_n, rscale_off, rscale_n;
};
SeqSpans seq_spans(const Layout& y, int s) {
  SeqSpans p;
  p.sink_n = (int64_t)y.L * y.H * 2 * kSink * y.D * 2;
  p.sink_off = y.off_sink + (int64_t)s * p.sink_n;
  p.rcode_n = (int64_t)y.L * y.H * 2 * y.cap * ring_row_bytes(y);
  p.rcode_off = y.off_rcode + (int64_t)s * p.rcode_n;
  p.rscale_n = y.f16ring ? 0 : (int64_t)y.L * y.H * 2 * y.cap * y.NB * 2;
  p.rscale_off = y.off_rscale + (int64_t)s * p.rscale_n;
  return p;
}
SaveHeader save_header(const kvq_cache* c) {
  SaveHeader hd{};
  hd.magic = kSaveMagic;
  hd.version = kSaveVersion;
  hd.L = c->y.L;
  hd.H = c->y.H;
  hd.D = c->y.D;
  hd.NB = c->y.NB;
  hd.cap = c->y.cap;
  hd.kbits = c->y.kbits;
  hd.vbits = c->y.vbits;
  hd.sinkhorn_passes = c->cfg.sinkhorn_passes;
  hd.stage_fmt = c->cfg.stage_fmt;
  hd.rec_bytes = c->y.rec_bytes;
  for (int i = 0; i < 4; ++i) hd.rot_signs[i] = c->cfg.rot_signs[i];
  return hd;
}
size_t save_bytes(const kvq_cache* c, const int64_t* n_rec) {
  const SeqSpans p = seq_spans(c->y, 0);
  size_t n = sizeof(SaveHeader) + (size_t)2 * c->y.L * sizeof(int64_t) + p.sink_n + p.rcode_n + p.rscale_n;
  for (int l = 0; l < c->y.L; ++l) n += (size_t)c->y.H * n_rec[l] * c->y.rec_bytes;
  return n;
}
}  // namespace

kvq_status kvq_seq_save_bytes(const kvq_cache* c, int32_t seq, size_t* bytes) {
  if (!c || !bytes) return fail(KVQ_ERR_INVALID, "bad arguments");
  if (seq < 0 || seq >= c->y.S) return fail(KVQ_ERR_INVALID, "seq out of range");
  std::vector<int64_t> nr(c->y.L);
  for (int l = 0; l < c->y.L; ++l) nr[l] = c->rec(seq, l);
  *bytes = save_bytes(c, nr.data());
  return KVQ_OK;
}

kvq_status kvq_seq_save(const kvq_cache* c, int32_t seq, void* host_dst, size_t bytes, void* stream) {
  if (!c || !host_dst) return fail(KVQ_ERR_INVALID, "bad arguments");
  if (c->plan_only) return fail(KVQ_ERR_UNSUPPORTED, "no device arena");
  size_t need = 0;
  kvq_status st = kvq_seq_save_bytes(c, seq, &need);
  if (st != KVQ_OK) return st;
  if (bytes != need) return fail(KVQ_ERR_INVALID, "save needs %zu bytes, got %zu", need, bytes);
  const Layout& y = c->y;
  uint8_t* out = (uint8_t*)host_dst;
  const SaveHeader hd = save_header(c);
  std::memcpy(out, &hd, sizeof hd);
  size_t o = sizeof hd;
  for (int l = 0; l < y.L; ++l, o += sizeof(int64_t)) std::memcpy(out + o, &c->n_tok[(size_t)seq * y.L + l], sizeof(int64_t));
  for (int l = 0; l < y.L; ++l, o += sizeof(int64_t)) std::memcpy(out + o, &c->n_rec[(size_t)seq * y.L + l], sizeof(int64_t));
  const SeqSpans p = seq_spans(y, seq);
  hipStream_t sm = (hipStream_t)stream;
  const int64_t spans[3][2] = {{p.sink_off, p.sink_n}, {p.rcode_off, p.rcode_n}, {p.rscale_off, p.rscale_n}};
  for (const auto& sp : spans) {
    if (sp[1] == 0) continue;
    hipError_t e = hipMemcpyAsync(out + o, c->arena + sp[0], (size_t)sp[1], hipMemcpyDeviceToHost, sm);
    if (e != hipSuccess) return hip_fail(e, "save copy");
    o += (size_t)sp[1];
  }
  for (int l = 0; l < y.L; ++l)
    for (int h = 0; h < y.H; ++h) {
      const size_t n = (size_t)c->rec(seq, l) * y.rec_bytes;
      if (n == 0) continue;
      hipError_t e = hipMemcpyAsync(out + o, c->arena + rec_off(y, seq, l, h, 0), n, hipMemcpyDeviceToHost, sm);
      if (e != hipSuccess) return hip_fail(e, "save copy");
      o += n;
    }
  hipError_t e = hipStreamSynchronize(sm);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  return KVQ_OK;
}

kvq_status kvq_seq_restore(kvq_cache* c, int32_t seq, const void* host_src, size_t bytes, void* stream) {
  if (!c || !host_src) return fail(KVQ_ERR_INVALID, "bad arguments");
  if (c->plan_only) return fail(KVQ_ERR_UNSUPPORTED, "no device arena");
  if (seq < 0 || seq >= c->y.S) return fail(KVQ_ERR_INVALID, "seq out of range");
  const Layout& y = c->y;
  const uint8_t* in = (const uint8_t*)host_src;
  const size_t head = sizeof(SaveHeader) + (size_t)2 * y.L * sizeof(int64_t);
  if (bytes < head) return fail(KVQ_ERR_INVALID, "blob of %zu bytes is shorter than its header", bytes);
  SaveHeader hd;
  std::memcpy(&hd, in, sizeof hd);
  const SaveHeader want = save_header(c);
  if (hd.magic != kSaveMagic || hd.version != kSaveVersion)
    return fail(KVQ_ERR_INVALID, "not a saved sequence (magic or version)");
  if (std::memcmp(&hd, &want, sizeof hd) != 0)
    return fail(KVQ_ERR_INVALID, "saved sequence is from a cache with another layout or encoding");
  std::vector<int64_t> nt(y.L), nr(y.L);
  std::memcpy(nt.data(), in + sizeof hd, (size_t)y.L * sizeof(int64_t));
  std::memcpy(nr.data(), in + sizeof hd + (size_t)y.L * sizeof(int64_t), (size_t)y.L * sizeof(int64_t));
  for (int l = 0; l < y.L; ++l) {
    if (nt[l] < 0 || nt[l] > c->cfg.max_ctx || nr[l] < 0 || nr[l] > y.max_rec ||
        (nt[l] > kSink && (nr[l] > (nt[l] - kSink) / kGroup || nt[l] - kSink - kGroup * nr[l] > y.cap)) ||
        (nt[l] <= kSink && nr[l] != 0))
      return fail(KVQ_ERR_INVALID, "saved counts of layer %d are inconsistent", l);
  }
  if (bytes != save_bytes(c, nr.data())) return fail(KVQ_ERR_INVALID, "blob has %zu bytes, its counts need %zu", bytes,
                                                     save_bytes(c, nr.data()));
  size_t o = head;
  const SeqSpans p = seq_spans(y, seq);
  hipStream_t sm = (hipStream_t)stream;
  const int64_t spans[3][2] = {{p.sink_off, p.sink_n}, {p.rcode_off, p.rcode_n}, {p.rscale_off, p.rscale_n}};
  for (const auto& sp : spans) {
    if (sp[1] == 0) continue;
    hipError_t e = hipMemcpyAsync(c->arena + sp[0], in + o, (size_t)sp[1], hipMemcpyHostToDevice, sm);
    if (e != hipSuccess) return hip_fail(e, "restore copy");
    o += (size_t)sp[1];
  }
  for (int l = 0; l < y.L; ++l)
    for (int h = 0; h < y.H; ++h) {
      const size_t n = (size_t)nr[l] * y.rec_bytes;
      if (n == 0) continue;
      hipError_t e = hipMemcpyAsync(c->arena + rec_off(y, seq, l, h, 0), in + o, n, hipMemcpyHostToDevice, sm);
      if (e != hipSuccess) return hip_fail(e, "restore copy");
      o += n;
    }
  hipError_t e = hipStreamSynchronize(sm);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  for (int l = 0; l < y.L; ++l) {
    c->tok(seq, l) = nt[l];
    c->rec(seq, l) = nr[l];
  }
  return KVQ_OK;
}

kvq_status kvq_unit_bytes(const kvq_cache* c, int32_t region, size_t* bytes) {
  if (!c || !bytes) return fail(KVQ_ERR_INVALID, "bad arguments");
  switch (region) {
    case KVQ_REGION_SINK: *bytes = (size_t)2 * c->y.D * 2; return KVQ_OK;
    case KVQ_REGION_RING: *bytes = c->y.f16ring ? (size_t)2 * c->y.D * 2 : (size_t)2 * c->y.NB * (2 + kQBytes); return KVQ_OK;
    case KVQ_REGION_BODY: *bytes = (size_t)c->y.rec_bytes; return KVQ_OK;
  }
  return fail(KVQ_ERR_INVALID, "bad region %d", region);
}

static kvq_status check_unit(const kvq_cache* c, int32_t seq, int32_t layer, int32_t h, int32_t region, int64_t index,
                             const void* host, size_t bytes) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (c->plan_only) return fail(KVQ_ERR_UNSUPPORTED, "no device arena");
  if (seq < 0 || seq >= c->y.S || layer < 0 || layer >= c->y.L || h < 0 || h >= c->y.H)
    return fail(KVQ_ERR_INVALID, "seq/layer/head out of range");
  if (!host) return fail(KVQ_ERR_INVALID, "host buffer is NULL");
  size_t need = 0;
  kvq_status st = kvq_unit_bytes(c, region, &need);
  if (st != KVQ_OK) return st;
  if (bytes != need) return fail(KVQ_ERR_INVALID, "unit has %zu bytes, got %zu", need, bytes);
  const int64_t lim = region == KVQ_REGION_SINK ? kSink : region == KVQ_REGION_RING ? c->y.cap : c->y.max_rec;
  if (index < 0 || index >= lim) return fail(KVQ_ERR_INVALID, "index %lld out of range", (long long)index);
  return KVQ_OK;
}

static kvq_status copy_unit(const kvq_cache* c, int32_t seq, int32_t layer, int32_t h, int32_t region, int64_t index,
                            uint8_t* host, bool to_host, hipStream_t stream) {
  const Layout& y = c->y;
  struct Piece {
    int64_t dev_off;
    size_t host_off, n;
  };
  std::vector<Piece> pieces;
  if (region == KVQ_REGION_SINK) {
    for (int kv = 0; kv < 2; ++kv)
      pieces.push_back({y.off_sink + sink_elem(y, seq, layer, h, kv, (int)index) * 2, (size_t)kv * y.D * 2,
                        (size_t)y.D * 2});
  } else if (region == KVQ_REGION_RING && y.f16ring) {
    for (int kv = 0; kv < 2; ++kv)
      pieces.push_back({rcode_off(y, seq, layer, h, kv, (int)index), (size_t)kv * y.D * 2, (size_t)y.D * 2});
  } else if (region == KVQ_REGION_RING) {
    size_t ho = 0;
    for (int kv = 0; kv < 2; ++kv)
      for (int bl = 0; bl < y.NB; ++bl) {
        pieces.push_back({rscale_off(y, seq, layer, h, kv, (int)index) + 2 * bl, ho, 2});
        pieces.push_back({rcode_off(y, seq, layer, h, kv, (int)index) + (int64_t)kQBytes * bl, ho + 2, kQBytes});
        ho += 2 + kQBytes;
      }
  } else {
    pieces.push_back({rec_off(y, seq, layer, h, index), 0, (size_t)y.rec_bytes});
  }
  for (const Piece& p : pieces) {
    hipError_t e = to_host ? hipMemcpyAsync(host + p.host_off, c->arena + p.dev_off, p.n, hipMemcpyDeviceToHost, stream)
                           : hipMemcpyAsync(c->arena + p.dev_off, host + p.host_off, p.n, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "copy");
  }
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  return KVQ_OK;
}

kvq_status kvq_export(const kvq_cache* c, int32_t seq, int32_t layer, int32_t h, int32_t region, int64_t index,
                      void* host_dst, size_t bytes, void* stream) {
  kvq_status st = check_unit(c, seq, layer, h, region, index, host_dst, bytes);
  if (st != KVQ_OK) return st;
  return copy_unit(c, seq, layer, h, region, index, (uint8_t*)host_dst, true, (hipStream_t)stream);
}

kvq_status kvq_import(kvq_cache* c, int32_t seq, int32_t layer, int32_t h, int32_t region, int64_t index,
                      const void* host_src, size_t bytes, void* stream) {
  kvq_status st = check_unit(c, seq, layer, h, region, index, host_src, bytes);
  if (st != KVQ_OK) return st;
  return copy_unit(c, seq, layer, h, region, index, (uint8_t*)host_src, false, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// TBQ4 comparator codec and its fused rotated-domain decode.

namespace {

struct Tbq4Tables {
  float cent[16], bnd[15];
};

// Lloyd-Max quantiser of N(0, 1/128) with 16 levels: alternate "each cell
// boundary is the midpoint of its two levels" and "each level is the mean of
// its cell" until the levels stop moving.  The quantiser is symmetric, so the
// iteration runs on the 8 positive levels of the unit Gaussian (the middle
// boundary is 0) and scales by 1/sqrt(128) at the end, in binary64.
const Tbq4Tables& tbq4_tables() {
  static const Tbq4Tables t = [] {
    const double inv_sqrt2pi = 0.39894228040143267794, inv_sqrt2 = 0.70710678118654752440;
    auto pdf = [&](double z) { return std::isinf(z) ? 0.0 : inv_sqrt2pi * std::exp(-0.5 * z * z); };
    double c[8];
    for (int k = 0; k < 8; ++k) c[k] = 0.375 * (k + 0.5);
    for (int it = 0; it < 200000; ++it) {
      double bd[9];
      bd[0] = 0.0;
      for (int k = 1; k < 8; ++k) bd[k] = 0.5 * (c[k - 1] + c[k]);
      bd[8] = INFINITY;
      double moved = 0.0;
      for (int k = 0; k < 8; ++k) {
        const double mass = 0.5 * (std::erfc(bd[k] * inv_sqrt2) - std::erfc(bd[k + 1] * inv_sqrt2));
        const double nc = (pdf(bd[k]) - pdf(bd[k + 1])) / mass;
        moved = std::max(moved, std::fabs(nc - c[k]));
        c[k] = nc;
      }
      if (moved <= 1e-15) break;
    }
    const double sigma = 1.0 / std::sqrt(128.0);
    double lv[16];
    for (int k = 0; k < 8; ++k) {
      lv[8 + k] = c[k] * sigma;
      lv[7 - k] = -c[k] * sigma;
    }
    Tbq4Tables r{};
    for (int k = 0; k < 16; ++k) r.cent[k] = (float)lv[k];
    for (int k = 0; k < 15; ++k) r.bnd[k] = (float)(0.5 * (lv[k] + lv[k + 1]));
    return r;
  }();
  return t;
}

void tbq4_signs(const uint64_t* s, uint32_t* out) {
  for (int w = 0; w < 4; ++w) {
    out[2 * w] = (uint32_t)(s[w] & 0xFFFFFFFFu);
    out[2 * w + 1] = (uint32_t)(s[w] >> 32);
  }
}

// Split-K chunking of a TBQ4 decode: about 4096 workgroups per launch, whole
// passes of 64 tokens.  The chunk count grows with max_len, so a workspace
// sized for a bound on the length fits every shorter batch.
int64_t tbq4_chunk_count(int32_t n_seqs, int32_t H, int64_t max_len) {
  const int64_t per_launch = std::min<int32_t>(n_seqs, kMaxLaunchSeqs) * (int64_t)H;
  const int64_t target = std::min<int64_t>(kMaxChunks, std::max<int64_t>(1, 4096 / std::max<int64_t>(1, per_launch)));
  return std::min<int64_t>((max_len + 63) / 64, target);
}

// Workspace: the rotated queries (fp32, 256-byte aligned span), then the
// split-K partial rows.
size_t tbq4_qr_bytes(int32_t n_seqs, int32_t Hq, int32_t D) {
  return (size_t)round_up((int64_t)n_seqs * Hq * D * (int64_t)sizeof(float), 256);
}

}  // namespace

extern "C" {

kvq_status kvq_tbq4_tables(float* centroids, float* boundaries) {
  if (!centroids && !boundaries) return fail(KVQ_ERR_INVALID, "no output");
  const Tbq4Tables& t = tbq4_tables();
  if (centroids) std::memcpy(centroids, t.cent, sizeof t.cent);
  if (boundaries) std::memcpy(boundaries, t.bnd, sizeof t.bnd);
  return KVQ_OK;
}

kvq_status kvq_tbq4_encode(const void* x, int64_t n, const uint64_t* signs, void* blocks, void* stream) {
  if (n < 0 || !signs || (n > 0 && (!x || !blocks))) return fail(KVQ_ERR_INVALID, "bad TBQ4 encode arguments");
  if (n == 0) return KVQ_OK;
  Tbq4CodecArgs a{};
  a.x = (const uint16_t*)x;
  a.blocks_out = (uint8_t*)blocks;
  a.n = n;
  const Tbq4Tables& t = tbq4_tables();
  std::memcpy(a.cent, t.cent, sizeof t.cent);
  std::memcpy(a.bnd, t.bnd, sizeof t.bnd);
  tbq4_signs(signs, a.signs);
  hipError_t e = launch_tbq4_encode(a, (hipStream_t)stream);
  return e == hipSuccess ? KVQ_OK : hip_fail(e, "TBQ4 encode launch");
}

kvq_status kvq_tbq4_decode(const void* blocks, int64_t n, const uint64_t* signs, float* out, void* stream) {
  if (n < 0 || !signs || (n > 0 && (!blocks || !out))) return fail(KVQ_ERR_INVALID, "bad TBQ4 decode arguments");
  if (n == 0) return KVQ_OK;
  Tbq4CodecArgs a{};
  a.blocks_in = (const uint8_t*)blocks;
  a.y = out;
  a.n = n;
  const Tbq4Tables& t = tbq4_tables();
  std::memcpy(a.cent, t.cent, sizeof t.cent);
  tbq4_signs(signs, a.signs);
  hipError_t e = launch_tbq4_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? KVQ_OK : hip_fail(e, "TBQ4 decode launch");
}

kvq_status kvq_tq_encode(const void* x, int64_t n, int32_t bits, const uint64_t* signs, void* blocks,
                          void* stream) {
  if (n < 0 || !signs || (n > 0 && (!x || !blocks))) return fail(KVQ_ERR_INVALID, "bad tq encode arguments");
  if (bits != 5 && bits != 6) return fail(KVQ_ERR_UNSUPPORTED, "tq blocks take 5 or 6 bits, not %d", bits);
  if (n == 0) return KVQ_OK;
  Tbq4CodecArgs a{};
  a.x = (const uint16_t*)x;
  a.blocks_out = (uint8_t*)blocks;
  a.n = n;
  tbq4_signs(signs, a.signs);
  hipError_t e = launch_tq_codec(a, bits, true, (hipStream_t)stream);
  return e == hipSuccess ? KVQ_OK : hip_fail(e, "tq encode launch");
}

kvq_status kvq_tq_decode(const void* blocks, int64_t n, int32_t bits, const uint64_t* signs, float* out,
                          void* stream) {
  if (n < 0 || !signs || (n > 0 && (!blocks || !out))) return fail(KVQ_ERR_INVALID, "bad tq decode arguments");
  if (bits != 5 && bits != 6) return fail(KVQ_ERR_UNSUPPORTED, "tq blocks take 5 or 6 bits, not %d", bits);
  if (n == 0) return KVQ_OK;
  Tbq4CodecArgs a{};
  a.blocks_in = (const uint8_t*)blocks;
  a.y = out;
  a.n = n;
  tbq4_signs(signs, a.signs);
  hipError_t e = launch_tq_codec(a, bits, false, (hipStream_t)stream);
  return e == hipSuccess ? KVQ_OK : hip_fail(e, "tq decode launch");
}

static kvq_status tbq4_check_shape(int32_t n_seqs, int32_t Hq, int32_t H, int32_t D) {
  if (n_seqs < 0) return fail(KVQ_ERR_INVALID, "n_seqs < 0");
  if (D != 128 && D != 256) return fail(KVQ_ERR_UNSUPPORTED, "TBQ4 decode takes head_dim 128 or 256, not %d", D);
  if (H < 1 || Hq < H || Hq % H != 0 || Hq / H > kMaxGroup)
    return fail(KVQ_ERR_INVALID, "n_q_heads must be 1 .. %d times n_kv_heads", kMaxGroup);
  return KVQ_OK;
}

kvq_status kvq_tbq4_workspace_bytes(int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int64_t max_len, size_t* bytes) {
  kvq_status st = tbq4_check_shape(n_seqs, n_q_heads, n_kv_heads, head_dim);
  if (st != KVQ_OK) return st;
  if (!bytes || max_len < 1) return fail(KVQ_ERR_INVALID, "bad TBQ4 workspace arguments");
  *bytes = tbq4_qr_bytes(n_seqs, n_q_heads, head_dim) +
           (size_t)n_seqs * n_q_heads * tbq4_chunk_count(n_seqs, n_kv_heads, max_len) * part_stride(head_dim) *
               sizeof(float);
  return KVQ_OK;
}

kvq_status kvq_tbq4_attn_decode(const void* q, const void* k_blocks, const void* v_blocks, int32_t n_seqs,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int64_t cap,
                                const int64_t* seq_len, const uint64_t* signs, float scale, void* out,
                                int32_t out_dtype, void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = tbq4_check_shape(n_seqs, n_q_heads, n_kv_heads, head_dim);
  if (st != KVQ_OK || n_seqs == 0) return st;
  if (!q || !k_blocks || !v_blocks || !seq_len || !signs || !out || !workspace || cap < 1)
    return fail(KVQ_ERR_INVALID, "bad TBQ4 decode arguments");
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_F16) return fail(KVQ_ERR_INVALID, "bad out_dtype");
  int64_t max_len = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (seq_len[i] < 1 || seq_len[i] > cap)
      return fail(KVQ_ERR_INVALID, "seq_len[%d] = %lld is outside 1 .. cap", i, (long long)seq_len[i]);
    max_len = std::max(max_len, seq_len[i]);
  }
  const int32_t H = n_kv_heads, Hq = n_q_heads, D = head_dim, NB = D / 128;
  const int64_t nc = tbq4_chunk_count(n_seqs, H, max_len);
  const int64_t chunk = round_up((max_len + nc - 1) / nc, 64);
  const int64_t max_chunks = (max_len + chunk - 1) / chunk;
  if (chunk > 0x7FFFFFFF) return fail(KVQ_ERR_CAPACITY, "sequence too long");
  const size_t qr_bytes = tbq4_qr_bytes(n_seqs, Hq, D);
  const size_t need = qr_bytes + (size_t)n_seqs * Hq * max_chunks * part_stride(D) * sizeof(float);
  if (ws_bytes < need) return fail(KVQ_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  const Tbq4Tables& t = tbq4_tables();
  float* qr_all = (float*)workspace;
  float* part_all = (float*)((uint8_t*)workspace + qr_bytes);
  const size_t out_elem = out_dtype == KVQ_OUT_F16 ? 2 : 4;
  const int64_t head_bytes = cap * NB * kTbqBytes;
  for (int b0 = 0; b0 < n_seqs; b0 += kMaxLaunchSeqs) {
    Tbq4AttnArgs a{};
    a.n_seqs = std::min(kMaxLaunchSeqs, n_seqs - b0);
    a.q = (const uint16_t*)q + (int64_t)b0 * Hq * D;
    a.kb = (const uint8_t*)k_blocks + (int64_t)b0 * H * head_bytes;
    a.vb = (const uint8_t*)v_blocks + (int64_t)b0 * H * head_bytes;
    a.qr = qr_all + (int64_t)b0 * Hq * D;
    a.part = part_all + (int64_t)b0 * Hq * max_chunks * part_stride(D);
    a.cap = cap;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.D = D;
    a.H = H;
    a.Hq = Hq;
    a.g = Hq / H;
    a.max_chunks = (int32_t)max_chunks;
    a.chunk = (int32_t)chunk;
    std::memcpy(a.cent, t.cent, sizeof t.cent);
    tbq4_signs(signs, a.signs);
    MergeArgs m{};
    int grid_x = 1;
    for (int b = 0; b < a.n_seqs; ++b) {
      a.len[b] = seq_len[b0 + b];
      m.n_chunks[b] = (int32_t)((a.len[b] + chunk - 1) / chunk);
      grid_x = std::max(grid_x, m.n_chunks[b]);
    }
    hipError_t e = launch_tbq4_attn(a, grid_x, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "TBQ4 decode launch");
    m.part = a.part;
    m.out = (uint8_t*)out + (size_t)b0 * Hq * D * out_elem;
    m.D = D;
    m.Hq = Hq;
    m.n_seqs = a.n_seqs;
    m.max_chunks = a.max_chunks;
    m.out_f16 = out_dtype == KVQ_OUT_F16;
    m.n_rows = 1;
    e = launch_merge(m, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return KVQ_OK;
}

}  // extern "C"
