"""Pins for the oracle's block attention (prefill chunks and verify blocks):
the newest n_q cached tokens' queries, each seeing every cached token up to its
own position (HAL #582 section 3b measures prefill over the same quantised
caches; a causal chunk is the plain reading)."""
import math

import numpy as np
import pytest

from oracle import attention, cache
from quantized_kv_cache_seal_amd import inputs


def _cache(D=128, H=2, Hq=6, tail_min=128, tail_max=256, max_ctx=2048, stage="tq6"):
    signs = inputs.rotation_signs(5) if D == 128 else None
    return cache.OracleCache(1, H, D, Hq, 1, max_ctx, tail_min, tail_max, 128, 4, 4, 4, signs, stage=stage)


def _fill(c, k, v, t0, t1, step=64):
    """Append tokens t0 .. t1 - 1 in steps, sealing when the ring is full."""
    for t in range(t0, t1, step):
        e = min(t1, t + step)
        assert c.append(0, [0], k[None, t:e], v[None, t:e]) == cache.OK
        c.seal(0, cache.SEAL_IF_FULL)


def _tokens(H, D, seed, t0, n):
    spec = inputs.KVSpec(1, H, D, seed, outliers=3, outlier_scale=10.0)
    return spec.tokens(0, "k", t0, n), spec.tokens(0, "v", t0, n)


@pytest.mark.parametrize("stage", ["tq6", "f16"])
def test_block_equals_decoding_token_by_token(stage):
    """Row t of the block equals the decode attention the same query gets right
    after its token is appended: a query sees exactly the tokens before it."""
    D, H, Hq, n_q = 128, 2, 6, 9
    p0 = 128 + 3 * 128 + 150
    k, v = _tokens(H, D, 3, 0, p0 + n_q)
    a, b = _cache(stage=stage), _cache(stage=stage)
    for c in (a, b):
        _fill(c, k, v, 0, p0)
        c.seal(0, cache.SEAL_TO_MIN)
    assert a.info(0, 0)[1] >= 3
    assert a.append(0, [0], k[None, p0:], v[None, p0:]) == cache.OK
    q = inputs.block_queries(9, 0, 0, 1, n_q, Hq, D)[0]
    got = a.attention_block(0, 0, q, 1 / math.sqrt(D))
    for t in range(n_q):
        assert b.append(0, [0], k[None, p0 + t:p0 + t + 1], v[None, p0 + t:p0 + t + 1]) == cache.OK
        assert np.array_equal(got[t], b.attention(0, 0, q[t], 1 / math.sqrt(D)))


def test_block_against_pure_python_brute_force():
    """Sink-only cache (the sink keeps the appended fp16 values): explicit loops
    over the visible tokens, query head h on KV head h // g."""
    D, H, Hq, n_tok, n_q = 128, 2, 4, 11, 5
    k, v = _tokens(H, D, 4, 0, n_tok)
    c = _cache(H=H, Hq=Hq)
    assert c.append(0, [0], k[None], v[None]) == cache.OK
    q = inputs.block_queries(4, 1, 0, 1, n_q, Hq, D)[0]
    got = c.attention_block(0, 0, q, 0.3)
    g = Hq // H
    for t in range(n_q):
        last = n_tok - n_q + t
        for h in range(Hq):
            qq = [float(x) for x in q[t, h]]
            s = [0.3 * sum(qq[j] * float(k[i, h // g, j]) for j in range(D)) for i in range(last + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            ref = [sum(w[i] * float(v[i, h // g, j]) for i in range(last + 1)) / tot for j in range(D)]
            assert np.allclose(got[t, h], ref, rtol=0, atol=1e-13)


def test_later_tokens_leave_earlier_rows_unchanged():
    """Rewriting the newest token's ring slot changes only the last row."""
    D, H, Hq, n_q = 128, 2, 6, 12
    n_tok = 128 + 2 * 128 + 200
    k, v = _tokens(H, D, 6, 0, n_tok)
    c = _cache()
    _fill(c, k, v, 0, n_tok - 200)
    c.seal(0, cache.SEAL_TO_MIN)
    assert c.append(0, [0], k[None, n_tok - 200:], v[None, n_tok - 200:]) == cache.OK
    q = inputs.block_queries(6, 0, 0, 1, n_q, Hq, D)[0]
    before = c.attention_block(0, 0, q, 0.2)
    n_rec = c.info(0, 0)[1]
    slot = (n_tok - 1 - 128) % c.cap
    other = _cache()
    kk, vv = _tokens(H, D, 99, 0, 1)
    assert other.append(0, [0], np.repeat(kk[None], 200, 1), np.repeat(vv[None], 200, 1)) == cache.OK
    for h in range(H):
        c.import_ring(0, 0, h, slot, other.export(0, 0, h, cache.REGION_RING, 150))
    assert c.info(0, 0)[1] == n_rec
    after = c.attention_block(0, 0, q, 0.2)
    assert np.array_equal(before[:-1], after[:-1])
    assert not np.allclose(before[-1], after[-1])


def test_block_reaching_into_sealed_records():
    """A block longer than the unsealed tail: rows whose tokens are sealed see the
    body's dequantised values, in order, exactly as the full decode of the
    newest token sees them."""
    D, H, Hq = 128, 2, 6
    n_tok = 128 + 4 * 128 + 140
    k, v = _tokens(H, D, 8, 0, n_tok)
    c = _cache()
    _fill(c, k, v, 0, n_tok)
    c.seal(0, cache.SEAL_TO_MIN)
    n_rec = c.info(0, 0)[1]
    n_q = n_tok - (128 + 128 * n_rec) + 130  # the block starts 130 tokens inside the body
    q = inputs.block_queries(8, 0, 0, 1, n_q, Hq, D)[0]
    got = c.attention_block(0, 0, q, 0.25)
    keys, vals = zip(*[c.head_kv(0, 0, h) for h in range(H)])
    for t in (0, 1, 129, 130, n_q - 1):
        n = n_tok - n_q + t + 1
        ref = attention.attend_gqa(q[t].astype(np.float64), [x[:n] for x in keys], [x[:n] for x in vals], 0.25)
        assert np.array_equal(got[t], ref)
    assert np.array_equal(got[-1], c.attention(0, 0, q[-1], 0.25))


def test_block_size_limits():
    c = _cache()
    k, v = _tokens(2, 128, 1, 0, 10)
    assert c.append(0, [0], k[None], v[None]) == cache.OK
    q = inputs.block_queries(1, 0, 0, 1, 11, 6, 128)[0]
    with pytest.raises(ValueError):
        c.attention_block(0, 0, q, 1.0)
    with pytest.raises(ValueError):
        c.attention_block(0, 0, q[:0], 1.0)
    full = c.attention_block(0, 0, q[:10], 1.0)  # the whole cache is the block
    assert np.array_equal(full[0, :3], attention.attend_gqa(
        q[0].astype(np.float64), [k[:1, 0].astype(np.float64), k[:1, 1].astype(np.float64)],
        [v[:1, 0].astype(np.float64), v[:1, 1].astype(np.float64)], 1.0)[:3])
