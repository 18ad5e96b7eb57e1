"""Decode attention in float64 (oracle; test infrastructure only).

SJ-KVaRN, section 2.1: every token passes through up to four regions and the
attention kernel reads all of them in one pass.  KV Cache Precision Tail,
section 2: attention sees the whole valid context; the exact recent rows and
the quantised body are combined under one softmax.  SJ-KVaRN section 2.2:
queries are rotated like keys, so q.k is unchanged, and the output is rotated
back; KV cache math states the same identity, q.k = (Hq).(Hk).

The oracle takes the plain definition: dequantise every region back to the
original domain in float64 (R^T of the rotated payloads; the sink is already
original f16) and compute softmax(scale * q.k) . v over all cached tokens.
Readings: the sink is not rotated (it stays exact 16-bit, section 2.1 item 1);
decode has no mask; grouped-query attention maps query head h to KV head
h // (H_q / H_kv).
"""
from __future__ import annotations

import numpy as np


def attend(q, keys, values, scale: float) -> np.ndarray:
    """One query head over one KV head: q (D,), keys/values (n, D) float64 -> (D,)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(keys, np.float64)
    v = np.asarray(values, np.float64)
    s = scale * (k @ q)
    m = s.max()
    p = np.exp(s - m)
    return (p @ v) / p.sum()


def attend_gqa(q, keys_by_head, values_by_head, scale: float) -> np.ndarray:
    """q (H_q, D); keys_by_head/values_by_head: lists (one per KV head) of (n, D)."""
    q = np.asarray(q, np.float64)
    hq = q.shape[0]
    hkv = len(keys_by_head)
    g = hq // hkv
    out = np.zeros_like(q)
    for h in range(hq):
        out[h] = attend(q[h], keys_by_head[h // g], values_by_head[h // g], scale)
    return out


def merge_partials(parts):
    """Combine (m, l, acc) partial softmax states into one output acc / l.

    Each part: m = max score in the part, l = sum exp(s - m), acc = sum exp(s - m) v.
    Used by tests to state the split invariance the GPU relies on.
    """
    M = max(p[0] for p in parts)
    L = sum(np.exp(p[0] - M) * p[1] for p in parts)
    A = sum(np.exp(p[0] - M) * np.asarray(p[2], np.float64) for p in parts)
    return A / L


def partial(q, keys, values, scale: float):
    s = scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), p @ np.asarray(values, np.float64)


def attend_causal_gqa(q, keys_by_head, values_by_head, p0: int, scale: float) -> np.ndarray:
    """Block (prefill or verify) attention: q (n_q, H_q, D) holds the queries of
    the tokens at positions p0 .. p0 + n_q - 1, each of which is already among
    the cached tokens; query t sees tokens 0 .. p0 + t (the causal mask of a
    prefill chunk, HAL #582 section 3b; a speculative verify block is the same
    computation).  keys_by_head/values_by_head: (n, D) per KV head, n >= p0 + n_q.
    Returns (n_q, H_q, D) float64."""
    q = np.asarray(q, np.float64)
    n_q = q.shape[0]
    out = np.zeros_like(q)
    for t in range(n_q):
        n = p0 + t + 1
        out[t] = attend_gqa(q[t], [k[:n] for k in keys_by_head], [v[:n] for v in values_by_head], scale)
    return out
