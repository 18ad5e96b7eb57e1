"""Parity at the full size of every workload bench.py times: the 16-layer,
4 x 256 KV, 24-query-head cache at 110,592 tokens (the default), the 512-wide
heads at 32,768, the 48-layer 8 x 128 K8/V4 cache at 262,144 and 16 sequences
x 65,536 (one launch over all 16), each built by the real path (chunked
append, seal-if-full, idle seal-back), then one kvq_decode_step per checked
layer over all the workload's sequences: the call and launch configuration
bench.py times.

The oracle cannot seal tens of thousands of tiles in seconds, so the checks
sample (the first and last sequence of a batch):
* every ring slot of the checked layers (4,097 tokens per KV head, the new one
  included) and sampled sink tokens: bit-exact with the oracle's own staging of
  the same inputs;
* sampled records: column scales within 1e-3 of the oracle's Sinkhorn, codes
  bit-exact given the GPU's scales (midpoint ties counted);
* the decode output of all 24 query heads against float64 attention over the
  same dequantised cache (the GPU's exported records, the oracle's sink and
  ring), max |o - ref| / rms(ref) <= 2e-3.
"""
import math
import sys
import time

import numpy as np
import pytest

from oracle import attention, cache as ocache, record, rotation, rounding, tq6
from quantized_kv_cache_seal_amd import configs, inputs, kvq, synthetic

from harness import ATTN_TOL, BOUNDARY_REL, SCALE_TOL

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

# workload -> KV layers checked
WORKLOADS = {
    "qwen27b": (configs.QWEN27B, (0, configs.QWEN27B.n_layers - 1)),
    "gemma31b": (configs.GEMMA31B, (configs.GEMMA31B.n_layers - 1,)),
    "qwen14b1m": (configs.QWEN14B1M, (configs.QWEN14B1M.n_layers - 1,)),
    "batched": (configs.BATCHED, (configs.BATCHED.n_layers - 1,)),
}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=list(WORKLOADS))
def full(request):
    import torch
    W, layers = WORKLOADS[request.param]
    t0 = time.time()
    _say(f"[fullsize] building {W.name}")
    cache = synthetic.build(W, ctx=W.ctx, max_ctx=W.ctx + 1)
    n_tok, n_rec, ring = cache.info(0, 0)
    _say(f"[fullsize] built in {time.time() - t0:.1f}s: {(n_tok, n_rec, ring)}")
    assert n_tok == W.ctx and 128 + 128 * n_rec + ring == W.ctx
    if W.name == configs.QWEN27B.name:
        assert (n_tok, n_rec, ring) == (110_592, 831, 4096)
    for s in range(W.n_seqs):
        assert cache.info(s, W.n_layers - 1) == (n_tok, n_rec, ring)
    yield cache, torch, W, layers
    del cache
    torch.cuda.empty_cache()


def _dequant_record(buf, W, side):
    """One record's K (side 0) or V (side 1) as float64 (128, D), rotated domain."""
    subs = record.parse_record(buf, W.head_dim, W.k_bits, W.v_bits)
    return np.concatenate([rounding.dequant(sb[side]["codes"], sb[side]["C"], sb[side]["S"], sb[side]["Z"])
                           for sb in subs], axis=1)


def _tokens(spec, layer, kv, t0, n):
    """The cache's own inputs: drawn by the same seeded generator on the device
    (as the build draws them; its float64 transcendental functions may round an
    ulp away from the host's), then copied to the host."""
    return spec.tokens(layer, kv, t0, n, backend="torch", device="cuda").cpu().numpy()


def _ring_tokens(spec, layer, t0, t1):
    return _tokens(spec, layer, "k", t0, t1 - t0), _tokens(spec, layer, "v", t0, t1 - t0)


def test_fullsize_decode_step(full):
    cache, torch, W, layers = full
    D, H, Hq, N = W.head_dim, W.n_kv_heads, W.n_q_heads, W.n_seqs
    sg = synthetic.signs(W)
    seqs = list(range(N))
    specs = [synthetic.spec_for(W, s) for s in seqs]
    cap = ocache.ring_capacity(W.tail_max, W.margin)
    ws = cache.workspace(N)
    for layer in layers:
        n_tok, n_rec, ring = cache.info(0, layer)
        knew = np.concatenate([_tokens(specs[s], layer, "k", n_tok, 1) for s in seqs])
        vnew = np.concatenate([_tokens(specs[s], layer, "v", n_tok, 1) for s in seqs])
        q = inputs.queries(W.seed, 0, layer, N, Hq, D)
        _say(f"[fullsize] {W.name} layer {layer}: decode_step over {N} sequence(s) at {n_tok} tokens")
        out, g = cache.decode_step(layer, seqs, torch.from_numpy(knew).cuda(), torch.from_numpy(vnew).cuda(),
                                   torch.from_numpy(q).cuda(), workspace=ws)
        got_all = out.cpu().numpy().astype(np.float64)
        assert g == 0
        for s in seqs:
            assert cache.info(s, layer) == (n_tok + 1, n_rec, ring + 1)
        t_ring = 128 + 128 * n_rec
        for s in sorted({0, N - 1}):
            spec = specs[s]
            k_sink, v_sink = _ring_tokens(spec, layer, 0, 128)
            k_ring, v_ring = _ring_tokens(spec, layer, t_ring, n_tok + 1)
            keys, vals = [], []
            n_ring_checked = 0
            for h in range(H):
                # sink: unchanged fp16, sampled bytes
                for t in (0, 63, 127):
                    assert cache.export(s, layer, h, kvq.REGION_SINK, t) == \
                        k_sink[t, h].tobytes() + v_sink[t, h].tobytes(), ("sink", s, layer, h, t)
                # ring: the oracle's staging of the same tokens, every slot
                xs = []
                for side, x16 in ((0, k_ring[:, h]), (1, v_ring[:, h])):
                    d, u = tq6.encode_blocks(rotation.rotate(x16, D, sg).reshape(-1, D // 128, 128))
                    xs.append((d, u))
                for i in range(n_tok + 1 - t_ring):
                    slot = (t_ring + i - 128) % cap
                    want = b"".join(tq6.block_bytes(xs[b2][0][i, b], xs[b2][1][i, b])
                                    for b2 in (0, 1) for b in range(D // 128))
                    assert cache.export(s, layer, h, kvq.REGION_RING, slot) == want, ("ring", s, layer, h, i)
                    n_ring_checked += 1
                kr = rotation.inverse_exact(tq6.decode_blocks(*xs[0]).reshape(-1, D), D, sg)
                vr = rotation.inverse_exact(tq6.decode_blocks(*xs[1]).reshape(-1, D), D, sg)
                # body: the GPU's own records, dequantised by the oracle
                bufs = [cache.export(s, layer, h, kvq.REGION_BODY, r) for r in range(n_rec)]
                kb = rotation.inverse_exact(np.concatenate([_dequant_record(b, W, 0) for b in bufs]), D, sg)
                vb = rotation.inverse_exact(np.concatenate([_dequant_record(b, W, 1) for b in bufs]), D, sg)
                keys.append(np.concatenate([k_sink[:, h].astype(np.float64), kb, kr]))
                vals.append(np.concatenate([v_sink[:, h].astype(np.float64), vb, vr]))
                assert keys[-1].shape == (n_tok + 1, D)
                _say(f"[fullsize]   sequence {s} head {h}: ring and records read")
            ref = attention.attend_gqa(q[s].astype(np.float64), keys, vals, 1.0)
            got = got_all[s]
            errs = np.max(np.abs(got - ref), axis=1) / np.sqrt(np.mean(ref ** 2, axis=1))
            _say(f"[fullsize] {W.name} layer {layer} sequence {s}: ring slots bit-exact {n_ring_checked}; "
                 f"decode err max {errs.max():.2e} over {Hq} query heads")
            assert errs.max() <= ATTN_TOL


def test_fullsize_sampled_records(full):
    cache, _, W, _ = full
    D = W.head_dim
    sg = synthetic.signs(W)
    sub = record.sub_width(D)
    layer = 0
    n_rec = cache.info(0, layer)[1]
    sample = sorted({0, n_rec // 2, n_rec - 1})
    ties = 0
    for s in sorted({0, W.n_seqs - 1}):
        spec = synthetic.spec_for(W, s)
        for h in range(W.n_kv_heads):
            for r in sample:
                subs = record.parse_record(cache.export(s, layer, h, kvq.REGION_BODY, r), D, W.k_bits, W.v_bits)
                for side, bits in ((0, W.k_bits), (1, W.v_bits)):
                    x16 = _tokens(spec, layer, "kv"[side], 128 + 128 * r, 128)[:, h]
                    d, u = tq6.encode_blocks(rotation.rotate(x16, D, sg).reshape(128, D // 128, 128))
                    xall = tq6.decode_blocks(d, u).reshape(128, D)
                    for i, sb in enumerate(subs):
                        x = np.ascontiguousarray(xall[:, sub * i:sub * (i + 1)])
                        g = sb[side]
                        want = ocache.encode_tile(x, W.passes, bits)
                        rel = np.abs(g["C"].astype(np.float64) / want["C"].astype(np.float64) - 1)
                        assert rel.max() <= SCALE_TOL, ("C", s, h, r, side, i, rel.max())
                        codes, S, Z = rounding.round_rows(x, g["C"], bits)
                        assert np.array_equal(S, g["S"]) and np.array_equal(Z, g["Z"]), ("SZ", s, h, r, side, i)
                        bad = codes != g["codes"]
                        if bad.any():
                            t = rounding.pre_round_values(x, g["C"], g["S"], g["Z"])
                            k = np.floor(t[bad])
                            assert (np.abs(t[bad] - (k + 0.5)) <= BOUNDARY_REL * np.abs(k + 0.5)).all(), \
                                ("codes", s, h, r, side, i)
                            ties += int(bad.sum())
    _say(f"[fullsize] {W.name}: sampled records {len(sample)} x {W.n_kv_heads} heads x K,V: scales within "
         f"{SCALE_TOL}, codes exact ({ties} midpoint ties)")
    assert math.isfinite(ties)


def _float_kv(cache, W, specs, layer, s, n_tok, n_rec):
    """Keys and values of every cached token of (s, layer) as float64 per KV
    head, in the original domain: the sink's and ring's inputs as the oracle
    stages them, the GPU's own records dequantised by the oracle."""
    D, H = W.head_dim, W.n_kv_heads
    sg = synthetic.signs(W)
    t_ring = 128 + 128 * n_rec
    k_sink, v_sink = _ring_tokens(specs[s], layer, 0, 128)
    k_ring, v_ring = _ring_tokens(specs[s], layer, t_ring, n_tok)
    keys, vals = [], []
    for h in range(H):
        rr = []
        for x16 in (k_ring[:, h], v_ring[:, h]):
            d, u = tq6.encode_blocks(rotation.rotate(x16, D, sg).reshape(-1, D // 128, 128))
            rr.append(rotation.inverse_exact(tq6.decode_blocks(d, u).reshape(-1, D), D, sg))
        bufs = [cache.export(s, layer, h, kvq.REGION_BODY, r) for r in range(n_rec)]
        kb = rotation.inverse_exact(np.concatenate([_dequant_record(b, W, 0) for b in bufs]), D, sg)
        vb = rotation.inverse_exact(np.concatenate([_dequant_record(b, W, 1) for b in bufs]), D, sg)
        keys.append(np.concatenate([k_sink[:, h].astype(np.float64), kb, rr[0]]))
        vals.append(np.concatenate([v_sink[:, h].astype(np.float64), vb, rr[1]]))
    return keys, vals


def test_fullsize_block_attention(full):
    """kvq_attn_prefill as bench.py times it at the headline shape: a 512-token
    prefill chunk and an 8-token verify block (the newest tokens) of the
    110,592-token cache, every query head of sampled rows (and every row of the
    verify block) against float64 causal attention over the same cache."""
    cache, torch, W, layers = full
    if W.name != configs.QWEN27B.name:
        pytest.skip("the block-attention leg is timed at the headline shape")
    D, Hq, N = W.head_dim, W.n_q_heads, W.n_seqs
    specs = [synthetic.spec_for(W, s) for s in range(N)]
    layer = layers[-1]
    n_tok, n_rec, ring = cache.info(0, layer)
    keys, vals = _float_kv(cache, W, specs, layer, 0, n_tok, n_rec)
    for n_q, rows in ((512, (0, 1, 127, 255, 256, 510, 511)), (8, tuple(range(8)))):
        q = inputs.block_queries(W.seed, 500 + layer, layer, N, n_q, Hq, D)
        _say(f"[fullsize] {W.name} layer {layer}: block attention n_q={n_q} at {n_tok} tokens")
        got = cache.attn_prefill(layer, list(range(N)), torch.from_numpy(q).cuda()).cpu().numpy().astype(np.float64)
        worst = 0.0
        for t in rows:
            n = n_tok - n_q + t + 1
            ref = attention.attend_gqa(q[0, t].astype(np.float64), [k[:n] for k in keys], [v[:n] for v in vals], 1.0)
            worst = max(worst, float(np.max(np.abs(got[0, t] - ref)) / math.sqrt(np.mean(ref ** 2))))
        _say(f"[fullsize] block attention n_q={n_q}: err max {worst:.2e} over rows {rows} x {Hq} heads")
        assert worst <= ATTN_TOL
