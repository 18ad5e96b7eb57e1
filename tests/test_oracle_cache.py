"""Pins for the oracle's four-region cache and the journaled adaptive seal rule
(SJ-KVaRN sections 2.1, 3, 4.3 and 10)."""
import math

import numpy as np
import pytest

from oracle import attention, cache, rotation, sizes, tq6
from quantized_kv_cache_seal_amd import configs, inputs


def test_seal_rule_counts():
    # tail grows to the maximum, then everything older than the newest tail_min is sealed
    assert cache.groups_to_seal(8191, 4096, 8192, cache.SEAL_IF_FULL) == 0
    assert cache.groups_to_seal(8192, 4096, 8192, cache.SEAL_IF_FULL) == 32
    assert cache.groups_to_seal(8200, 4096, 8192, cache.SEAL_IF_FULL) == 32
    assert cache.groups_to_seal(4223, 4096, 8192, cache.SEAL_TO_MIN) == 0
    assert cache.groups_to_seal(4224, 4096, 8192, cache.SEAL_TO_MIN) == 1
    assert cache.groups_to_seal(100, 4096, 8192, cache.SEAL_TO_MIN) == 0
    assert cache.ring_capacity(8192, 512) == 8704
    assert cache.ring_capacity(4352, 512) == 4864


def test_streaming_schedule_seals_every_4096_tokens():
    # one token per step (decode), seal check after every step
    n_rec, events, tail = 0, [], []
    for n_tok in range(1, 60_000):
        ring = max(0, n_tok - 128 - 128 * n_rec)
        g = cache.groups_to_seal(ring, 4096, 8192, cache.SEAL_IF_FULL)
        if g:
            events.append((n_tok, g))
            n_rec += g
        tail.append(max(0, n_tok - 128 - 128 * n_rec))
    gaps = np.diff([e[0] for e in events])
    assert np.all(gaps == 4096) and all(g == 32 for _, g in events)
    steady = np.array(tail[9000:])
    assert steady.min() == 4096 and steady.max() == 8191


def test_effective_bits_printed_formula_from_region_counts():
    # regions of a just-sealed cache at N = 110,592 and of one just before a seal
    body = sizes.body_bits_per_value(4, 4)
    assert body == 4.28125
    for tail, expect in ((4096, 4.3702), (8192, 4.4385)):
        n = 110_592
        n_body = n - 128 - tail
        bits = (n_body * body + tail * tq6.BITS_PER_VALUE + 128 * (tq6.BITS_PER_VALUE + 16)) / n
        assert abs(bits - sizes.effective_bits(n, tail, body)) < 1e-12
        assert round(bits, 4) == expect


def _tiny_cache(cfg, signs=None):
    return cache.OracleCache(cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads, cfg.n_seqs,
                             cfg.ctx, cfg.tail_min, cfg.tail_max, cfg.margin, cfg.k_bits, cfg.v_bits,
                             cfg.passes, signs)


def test_errors_leave_state_unchanged():
    cfg = configs.TINY
    c = _tiny_cache(cfg)
    spec = inputs.KVSpec(1, 1, 256, 1)
    k = spec.tokens(0, "k", 0, 1024)[None]
    v = spec.tokens(0, "v", 0, 1024)[None]
    assert c.append(0, [0], k, v) == cache.OK
    assert c.info(0, 0) == (1024, 0, 896)
    big = spec.tokens(0, "k", 0, 200)[None]
    assert c.append(0, [0], big, big) == cache.ERR_RING_FULL     # 896 + 200 > 1024 slots
    assert c.info(0, 0) == (1024, 0, 896)
    assert c.append(1, [0], big, big) == cache.ERR_INVALID
    assert c.append(0, [3], big, big) == cache.ERR_INVALID
    assert c.seal(0, cache.SEAL_IF_FULL) == 5                     # (896 - 256) // 128
    assert c.info(0, 0) == (1024, 5, 256)
    c2 = _tiny_cache(cfg.scaled(ctx=1100))
    assert c2.append(0, [0], k, v) == cache.OK
    assert c2.append(0, [0], big, big) == cache.ERR_CAPACITY


def test_tiny_end_to_end_regions_and_accuracy():
    cfg = configs.TINY
    c = _tiny_cache(cfg)
    spec = inputs.KVSpec(1, 1, 256, cfg.seed, outliers=cfg.outliers, outlier_scale=cfg.outlier_scale)
    k = spec.tokens(0, "k", 0, cfg.ctx)
    v = spec.tokens(0, "v", 0, cfg.ctx)
    for t0 in range(0, cfg.ctx, 512):
        assert c.append(0, [0], k[None, t0:t0 + 512], v[None, t0:t0 + 512]) == cache.OK
        c.seal(0, cache.SEAL_IF_FULL)
    c.seal(0, cache.SEAL_TO_MIN)
    n_tok, n_rec, ring = c.info(0, 0)
    assert (n_tok, n_rec, ring) == (2048, 13, 256)
    # sink bytes are the inputs; ring slots are the tq6 encoding of the rotated inputs
    assert c.export(0, 0, 0, cache.REGION_SINK, 5) == k[5, 0].tobytes() + v[5, 0].tobytes()
    t = 2000
    slot = (t - 128) % c.cap
    expect = tq6.encode_vector(rotation.rotate(k[t, 0], 256)) + tq6.encode_vector(rotation.rotate(v[t, 0], 256))
    assert c.export(0, 0, 0, cache.REGION_RING, slot) == expect
    # every token is back in token order and close to its input
    kk, vv = c.head_kv(0, 0, 0)
    assert kk.shape == (2048, 256)
    assert np.array_equal(kk[:128], k[:128, 0].astype(np.float64))
    rel_k = np.linalg.norm(kk - k[:, 0]) / np.linalg.norm(k[:, 0].astype(np.float64))
    rel_v = np.linalg.norm(vv - v[:, 0]) / np.linalg.norm(v[:, 0].astype(np.float64))
    assert rel_k < 0.12 and rel_v < 0.12
    ring_part = np.linalg.norm(kk[-256:] - k[-256:, 0]) / np.linalg.norm(k[-256:, 0].astype(np.float64))
    assert ring_part < 0.03          # 6-bit staging is much finer than the 4-bit body
    # SJ-KVaRN section 2.2: plain rounding fails on outlier channels, rotation and
    # balancing fix that.  Per-token 4-bit rounding of the raw keys does far worse.
    body = slice(128, 128 + 13 * 128)
    kb = k[body, 0].astype(np.float64)
    mn = kb.min(axis=1, keepdims=True)
    st = (kb.max(axis=1, keepdims=True) - mn) / 15
    naive = np.rint((kb - mn) / st) * st + mn
    ours = np.linalg.norm(kk[body] - kb)
    assert ours < 0.5 * np.linalg.norm(naive - kb)
    q = inputs.queries(cfg.seed, 0, 0, 1, 4, 256)[0]
    out = c.attention(0, 0, q, 1.0)
    assert out.shape == (4, 256) and np.all(np.isfinite(out))


def test_gqa_sink_only_cache():
    c = cache.OracleCache(1, 2, 128, 6, 1, 4096, 256, 512, signs=inputs.rotation_signs(1))
    spec = inputs.KVSpec(1, 2, 128, 4)
    k = spec.tokens(0, "k", 0, 100)
    v = spec.tokens(0, "v", 0, 100)
    assert c.append(0, [0], k[None], v[None]) == cache.OK
    q = inputs.queries(4, 0, 0, 1, 6, 128)[0]
    out = c.attention(0, 0, q, 1 / math.sqrt(128))
    for h in range(6):
        ref = attention.attend(q[h].astype(np.float64), k[:, h // 3].astype(np.float64),
                               v[:, h // 3].astype(np.float64), 1 / math.sqrt(128))
        assert np.array_equal(out[h], ref)


# ---------------------------------------------------------------------------
# Staging precision: the f16 ring (SJ-KVaRN section 4.1; KV Cache Precision
# Tail, section 2: KVarN's exact F16 tail).

def test_f16_staging_ring_size_printed():
    """The f16 ring costs 65,536 - 25,088 = 40,448 more bytes per slot than
    tq6_0 in the Qwen 27B-like shape; a ring of tail_max 8,192 + one 512-token
    micro-batch holds 8,704 slots: 0.33 GB more, the low end of the printed
    0.33 to 0.39 GB (the high end matches ~10,240 slots, 8,192 + 2,048)."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_numbers.json")))
    e = g["f16_staging_extra_gb_at_100k"]
    per_slot = sizes.kv_bytes_per_token(16, 4, 256, 16) - sizes.kv_bytes_per_token(16, 4, 256, tq6.BITS_PER_VALUE)
    assert per_slot == 40448
    extra = cache.ring_capacity(8192, 512) * per_slot / sizes.GIB
    assert round(extra, e["digits"]) == e["value"]
    assert round(cache.ring_capacity(8192, 2048) * per_slot / sizes.GIB, 2) == e["upper"]


def _f16_pair(D, signs):
    w = configs.TINY.scaled(head_dim=D, n_q_heads=4, ctx=1200, tail_min=256, tail_max=384)
    spec = inputs.KVSpec(1, 1, D, 5, outliers=3, outlier_scale=10.0)
    k = spec.tokens(0, "k", 0, w.ctx)[None]
    v = spec.tokens(0, "v", 0, w.ctx)[None]
    caches = []
    for stage in ("f16", "tq6"):
        c = cache.OracleCache(1, 1, D, 4, 1, w.ctx, w.tail_min, w.tail_max, w.margin, 4, 4, 8, signs, stage=stage)
        for t0 in range(0, w.ctx, 200):
            assert c.append(0, [0], k[:, t0:t0 + 200], v[:, t0:t0 + 200]) == cache.OK
            c.seal(0, cache.SEAL_IF_FULL)
        caches.append(c)
    return w, k[0], v[0], caches


@pytest.mark.parametrize("D", [256, 128])
def test_f16_staging_ring_holds_tokens_and_seals_their_rotation(D):
    """Ring slots hold the tokens bit for bit; each sealed record is the
    balancing and rounding of the group's tokens rotated exactly and rounded
    once to fp32 (written out here from the rotation, balancing and rounding
    functions); the seal schedule is the tq6 one."""
    from oracle import record
    signs = inputs.rotation_signs(3) if D == 128 else None
    w, k, v, (c16, c6) = _f16_pair(D, signs)
    assert c16.info(0, 0) == c6.info(0, 0)
    n_tok, n_rec, ring = c16.info(0, 0)
    assert n_rec > 0 and ring > 0
    for t in range(128 + 128 * n_rec, n_tok):
        slot = (t - 128) % c16.cap
        assert c16.export(0, 0, 0, cache.REGION_RING, slot) == k[t, 0].tobytes() + v[t, 0].tobytes()
    for r in range(n_rec):
        toks = slice(128 + 128 * r, 256 + 128 * r)
        want = []
        for x16 in (k[toks, 0], v[toks, 0]):
            xr = rotation.rotate(x16, D, signs)
            want.append(cache.encode_tile(xr[:, :record.sub_width(D)], 8, 4))
        got = record.parse_record(c16.export(0, 0, 0, cache.REGION_BODY, r), D, 4, 4)[0]
        for g_, w_ in zip(got, want):
            for n in ("codes", "C", "S", "Z"):
                assert np.array_equal(g_[n], w_[n]), (r, n)


def test_f16_staging_attention_is_exact_over_the_ring():
    """Attention over an f16-staged cache equals float64 attention over the
    sink and ring tokens as given plus the records dequantised and rotated
    back (brute force, written out here); against the tq6-staged cache of
    the same tokens it differs only by the staged ring's quantisation."""
    from oracle import record, rounding
    w, k, v, (c16, c6) = _f16_pair(256, None)
    n_tok, n_rec, ring = c16.info(0, 0)
    q = inputs.queries(5, 0, 0, 1, 4, 256)[0]
    keys = [k[:128, 0].astype(np.float64)]
    vals = [v[:128, 0].astype(np.float64)]
    for r in range(n_rec):
        kk, vv = record.parse_record(c16.export(0, 0, 0, cache.REGION_BODY, r), 256, 4, 4)[0]
        keys.append(rotation.inverse_exact(rounding.dequant(kk["codes"], kk["C"], kk["S"], kk["Z"]), 256))
        vals.append(rotation.inverse_exact(rounding.dequant(vv["codes"], vv["C"], vv["S"], vv["Z"]), 256))
    keys.append(k[128 + 128 * n_rec:n_tok, 0].astype(np.float64))
    vals.append(v[128 + 128 * n_rec:n_tok, 0].astype(np.float64))
    K, V = np.concatenate(keys), np.concatenate(vals)
    qf = q.astype(np.float64)
    want = []
    for h in range(4):
        s = K @ qf[h]
        p = np.exp(s - s.max())
        want.append(p @ V / p.sum())
    got = c16.attention(0, 0, q, 1.0)
    assert np.max(np.abs(got - np.array(want))) < 1e-12
    # the two stagings differ (the tq6 ring and the records sealed from it
    # carry its 6-bit rounding), by a small fraction of the N(0, 1) values
    other = c6.attention(0, 0, q, 1.0)
    assert 0 < np.max(np.abs(got - other)) < 0.1
