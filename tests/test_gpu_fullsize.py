"""Parity at the full size of the decode benchmark: the 16-layer, 4 x 256 KV,
24-query-head cache at 110,592 tokens, built by the real path (chunked append,
seal-if-full, idle seal-back), then one kvq_decode_step per checked layer, the
call and launch configuration bench.py times.

The oracle cannot seal 26,592 tiles in seconds, so the checks sample:
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

pytestmark = pytest.mark.gpu

W = configs.QWEN27B
LAYERS = (0, W.n_layers - 1)
SAMPLE_RECORDS = (0, 415, 830)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def full():
    import torch
    t0 = time.time()
    _say(f"[fullsize] building {W.name}")
    cache = synthetic.build(W, ctx=W.ctx, max_ctx=W.ctx + 1)
    _say(f"[fullsize] built in {time.time() - t0:.1f}s: {cache.info(0, 0)}")
    assert cache.info(0, 0) == (110_592, 831, 4096)
    yield cache, torch
    del cache
    torch.cuda.empty_cache()


def _tokens(spec, layer, kv, t0, n):
    """The cache's own inputs: drawn by the same seeded generator on the device
    (as the build draws them; its float64 transcendental functions may round an
    ulp away from the host's), then copied to the host."""
    return spec.tokens(layer, kv, t0, n, backend="torch", device="cuda").cpu().numpy()


def _ring_tokens(spec, layer, t0, t1):
    return _tokens(spec, layer, "k", t0, t1 - t0), _tokens(spec, layer, "v", t0, t1 - t0)


def test_fullsize_decode_step(full):
    cache, torch = full
    spec = synthetic.spec_for(W)
    D, H, Hq = W.head_dim, W.n_kv_heads, W.n_q_heads
    cap = ocache.ring_capacity(W.tail_max, W.margin)
    ws = cache.workspace(1)
    for layer in LAYERS:
        n_tok, n_rec, ring = cache.info(0, layer)
        knew = _tokens(spec, layer, "k", n_tok, 1)
        vnew = _tokens(spec, layer, "v", n_tok, 1)
        q = inputs.queries(W.seed, 0, layer, 1, Hq, D)
        _say(f"[fullsize] layer {layer}: decode_step at {n_tok} tokens")
        out, g = cache.decode_step(layer, [0], torch.from_numpy(knew).cuda(), torch.from_numpy(vnew).cuda(),
                                   torch.from_numpy(q).cuda(), workspace=ws)
        got = out.cpu().numpy()[0].astype(np.float64)
        assert g == 0 and cache.info(0, layer) == (n_tok + 1, n_rec, ring + 1)

        t_ring = 128 + 128 * n_rec
        k_sink, v_sink = _ring_tokens(spec, layer, 0, 128)
        k_ring, v_ring = _ring_tokens(spec, layer, t_ring, n_tok + 1)
        keys, vals = [], []
        n_ring_checked = 0
        for h in range(H):
            # sink: unchanged fp16, sampled bytes
            for t in (0, 63, 127):
                assert cache.export(0, layer, h, kvq.REGION_SINK, t) == \
                    k_sink[t, h].tobytes() + v_sink[t, h].tobytes(), ("sink", layer, h, t)
            # ring: the oracle's staging of the same tokens, every slot
            xs = []
            for side, x16 in ((0, k_ring[:, h]), (1, v_ring[:, h])):
                d, u = tq6.encode_blocks(rotation.rotate(x16, D).reshape(-1, D // 128, 128))
                xs.append((d, u))
            for i in range(n_tok + 1 - t_ring):
                slot = (t_ring + i - 128) % cap
                want = b"".join(tq6.block_bytes(xs[s][0][i, b], xs[s][1][i, b]) for s in (0, 1) for b in range(D // 128))
                assert cache.export(0, layer, h, kvq.REGION_RING, slot) == want, ("ring", layer, h, i)
                n_ring_checked += 1
            kr = [rotation.inverse_exact(tq6.decode_blocks(*xs[0]).reshape(-1, D), D)]
            vr = [rotation.inverse_exact(tq6.decode_blocks(*xs[1]).reshape(-1, D), D)]
            # body: the GPU's own records, dequantised by the oracle
            kb, vb = [], []
            for r in range(n_rec):
                subs = record.parse_record(cache.export(0, layer, h, kvq.REGION_BODY, r), D, W.k_bits, W.v_bits)
                kb.append(rounding.dequant(subs[0][0]["codes"], subs[0][0]["C"], subs[0][0]["S"], subs[0][0]["Z"]))
                vb.append(rounding.dequant(subs[0][1]["codes"], subs[0][1]["C"], subs[0][1]["S"], subs[0][1]["Z"]))
            kb = rotation.inverse_exact(np.concatenate(kb), D)
            vb = rotation.inverse_exact(np.concatenate(vb), D)
            keys.append(np.concatenate([k_sink[:, h].astype(np.float64), kb, kr[0]]))
            vals.append(np.concatenate([v_sink[:, h].astype(np.float64), vb, vr[0]]))
            assert keys[-1].shape == (n_tok + 1, D)
        ref = attention.attend_gqa(q[0].astype(np.float64), keys, vals, 1.0)
        errs = np.max(np.abs(got - ref), axis=1) / np.sqrt(np.mean(ref ** 2, axis=1))
        _say(f"[fullsize] layer {layer}: ring slots bit-exact {n_ring_checked}; decode err max {errs.max():.2e} "
             f"over {Hq} query heads")
        assert errs.max() <= ATTN_TOL


def test_fullsize_sampled_records(full):
    cache, _ = full
    spec = synthetic.spec_for(W)
    D = W.head_dim
    layer = 0
    ties = 0
    for h in range(W.n_kv_heads):
        for r in SAMPLE_RECORDS:
            subs = record.parse_record(cache.export(0, layer, h, kvq.REGION_BODY, r), D, W.k_bits, W.v_bits)
            for side, bits in ((0, W.k_bits), (1, W.v_bits)):
                x16 = _tokens(spec, layer, "kv"[side], 128 + 128 * r, 128)[:, h]
                d, u = tq6.encode_blocks(rotation.rotate(x16, D).reshape(128, D // 128, 128))
                x = tq6.decode_blocks(d, u).reshape(128, D)
                g = subs[0][side]
                want = ocache.encode_tile(x, W.passes, bits)
                rel = np.abs(g["C"].astype(np.float64) / want["C"].astype(np.float64) - 1)
                assert rel.max() <= SCALE_TOL, ("C", h, r, side, rel.max())
                codes, S, Z = rounding.round_rows(x, g["C"], bits)
                assert np.array_equal(S, g["S"]) and np.array_equal(Z, g["Z"]), ("SZ", h, r, side)
                bad = codes != g["codes"]
                if bad.any():
                    t = rounding.pre_round_values(x, g["C"], g["S"], g["Z"])
                    k = np.floor(t[bad])
                    assert (np.abs(t[bad] - (k + 0.5)) <= BOUNDARY_REL * np.abs(k + 0.5)).all(), ("codes", h, r, side)
                    ties += int(bad.sum())
    _say(f"[fullsize] sampled records {len(SAMPLE_RECORDS)} x {W.n_kv_heads} heads x K,V: scales within "
         f"{SCALE_TOL}, codes exact ({ties} midpoint ties)")
    assert math.isfinite(ties)
