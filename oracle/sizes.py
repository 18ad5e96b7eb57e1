"""Cache-size arithmetic the pages print (oracle; test infrastructure only).

* KV cache math, "Bytes per token":
  kv_bytes_per_token = 2 x n_attn_layers x n_kv_heads x head_dim x bytes_per_value.
* Block formats (SJ-KVaRN sections 6 and 7.2; KV cache math table): q8_0 34 B
  per 32 values, q5_1 24 B / 32, q4_0 18 B / 32, q5_0 5.5 bits, tq6_0 98 B /
  128, tq5_0 82 B / 128, turbo4 / TBQ4 66 B / 128, turbo3 50 B / 128.
* SJ-KVaRN section 3: body records carry 2,304 B of fp16 scales per record per
  KV head (+0.28125 bits per value); effective bits over the occupied cache
  [(N - 128 - t) body + t 6.125 + 128 (6.125 + 16)] / N.
* SJ-KVaRN section 7.2: allocated SJ-KVaRN bytes = body bytes per token x
  (context - 4,224) + 259 MiB for the sink, staging rows and full-size ring.
* GB means GiB (SJ-KVaRN section 1: "GB means 1,024 MiB").
"""
from __future__ import annotations

KIB, MIB, GIB = 1024, 1024 ** 2, 1024 ** 3

FORMAT_BITS = {
    "f16": 16.0,
    "bf16": 16.0,
    "q8_0": 34 * 8 / 32,
    "q5_1": 24 * 8 / 32,
    "q5_0": 22 * 8 / 32,
    "q4_0": 18 * 8 / 32,
    "tq6_0": 98 * 8 / 128,
    "tq5_0": 82 * 8 / 128,
    "turbo4": 66 * 8 / 128,
    "tbq4": 66 * 8 / 128,
    "turbo3": 50 * 8 / 128,
}

PAGE_SCALE_BYTES = 2304      # fp16 scales per record per KV head, as the pages count them
SINK = 128
RING_FIXED_BYTES = 259 * MIB
RULE_OFFSET_TOKENS = 4224


def kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bits_k, bits_v=None) -> float:
    """2 x layers x heads x dim x bytes, with K and V formats allowed to differ."""
    bits_v = bits_k if bits_v is None else bits_v
    return n_layers * n_kv_heads * head_dim * (bits_k + bits_v) / 8


def values_per_token(n_layers, n_kv_heads, head_dim) -> int:
    return 2 * n_layers * n_kv_heads * head_dim


def page_record_bytes(k_bits, v_bits, head_dim=256, scale_bytes=PAGE_SCALE_BYTES) -> int:
    """One 128-token record for one KV head with the pages' scale count."""
    return 128 * head_dim * (k_bits + v_bits) // 8 + scale_bytes


def body_bits_per_value(k_bits, v_bits, head_dim=256, scale_bytes=PAGE_SCALE_BYTES) -> float:
    return page_record_bytes(k_bits, v_bits, head_dim, scale_bytes) * 8 / (128 * 2 * head_dim)


def body_bytes_per_token(k_bits, v_bits, n_layers, n_kv_heads, head_dim=256, scale_bytes=PAGE_SCALE_BYTES) -> float:
    return page_record_bytes(k_bits, v_bits, head_dim, scale_bytes) * n_layers * n_kv_heads / 128


def effective_bits(n_tokens, tail, body_bits, stage_bits=98 * 8 / 128) -> float:
    return ((n_tokens - SINK - tail) * body_bits + tail * stage_bits + SINK * (stage_bits + 16)) / n_tokens


def allocated_bytes(body_bytes_per_tok, ctx) -> float:
    return body_bytes_per_tok * (ctx - RULE_OFFSET_TOKENS) + RING_FIXED_BYTES


def allocated_bits(total_bytes, ctx, n_layers, n_kv_heads, head_dim) -> float:
    return total_bytes * 8 / (ctx * values_per_token(n_layers, n_kv_heads, head_dim))


def format_bytes(fmt_k, ctx, n_values_per_token, fmt_v=None) -> float:
    fmt_v = fmt_k if fmt_v is None else fmt_v
    return ctx * n_values_per_token / 2 * (FORMAT_BITS[fmt_k] + FORMAT_BITS[fmt_v]) / 8
