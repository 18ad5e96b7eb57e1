"""GPU seal of tiles the fp32 balancing passes cannot resolve, against the
oracle (SJ-KVaRN section 2.2 "Balancing"): staged tiles placed in the ring
through the import hook, sealed by kvq_seal, and compared record by record
with the oracle sealing the same staged tiles.

Tile kinds (every row of a tile shares one random code pattern Q unless
stated; d is the tq6_0 block scale):
* offset1e3 / offset1e5: every other row has one code (whose Q is 0) raised
  by k, so after the first row pass every column is a constant offset plus a
  real spread of about 1e-3 (1e-5) of its RMS;
* pow2: rows are power-of-two multiples of one row (d scaled by 2^k): after
  the first row pass every column is constant in exact arithmetic;
* repeated: identical rows (constant columns, spread exactly zero);
* small_column: random codes, except one column that is zero but for a
  single +-1, so its balancing factor is far above the others';
* normal: random codes and scales (the fast path's own case).
Parity rule: C within 1e-3 relative of the oracle's; given the GPU's C, the
oracle's rounding of the same tile reproduces S, Z and every code (codes
within 1e-6 relative of a rounding midpoint excepted and counted)."""
import sys

import numpy as np
import pytest

from oracle import cache as ocache
from oracle import record, rounding, sinkhorn, tq6
from quantized_kv_cache_seal_amd import configs, inputs, kvq

from harness import BOUNDARY_REL, SCALE_TOL

pytestmark = pytest.mark.gpu

KINDS = ["offset1e3", "offset1e5", "pow2", "repeated", "small_column", "normal"]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tile(kind, D, seed):
    """(d fp16 [128][D/128], u uint8 [128][D]) of one staged tile."""
    nb = D // 128
    Q = np.round(inputs.uniform_np(seed, 1, 0, D) * 62 - 31).clip(-31, 31).astype(np.int64)
    Q[3] = 0
    q = np.tile(Q, (128, 1))
    d = np.full((128, nb), 0.05, np.float16)
    if kind.startswith("offset"):
        k = {("offset1e3", 256): 18, ("offset1e5", 256): 2, ("offset1e3", 128): 13, ("offset1e5", 128): 1}[(kind, D)]
        q[1::2, 3] = k
    elif kind == "pow2":
        d = (d.astype(np.float32) * np.exp2(np.arange(128) % 5 - 2.0)[:, None].astype(np.float32)).astype(np.float16)
    elif kind == "small_column":
        q = np.round(inputs.uniform_np(seed, 2, 0, 128 * D) * 62 - 31).clip(-31, 31).astype(np.int64).reshape(128, D)
        q[:, 7] = 0
        q[3, 7] = 1
    elif kind == "normal":
        q = np.round(inputs.uniform_np(seed, 2, 0, 128 * D) * 62 - 31).clip(-31, 31).astype(np.int64).reshape(128, D)
        d = (0.02 + 0.08 * inputs.uniform_np(seed, 3, 0, 128 * nb)).astype(np.float16).reshape(128, nb)
    return d, (q + 32).astype(np.uint8)


def _slot_bytes(dk, uk, dv, uv, t):
    nb = dk.shape[1]
    out = b""
    for d, u in ((dk, uk), (dv, uv)):
        for b in range(nb):
            out += tq6.block_bytes(d[t, b], u[t, b * 128:(b + 1) * 128])
    return out


def _first_pass_rho(d, u):
    """Median over columns of (column spread / column RMS) after one row pass."""
    x = tq6.decode_blocks(d, u.reshape(128, -1, 128)).reshape(128, -1).astype(np.float64)
    sig, _ = sinkhorn.spread(x, 1)
    y = x / np.where(sig > 0, sig, 1.0)[:, None]
    sc, rms = sinkhorn.spread(y, 0)
    ok = rms > 0
    return float(np.median(sc[ok] / rms[ok]))


SHAPES = {
    256: configs.QWEN27B.scaled(n_layers=1, n_kv_heads=1, n_q_heads=6, tail_min=128, tail_max=1024, margin=0,
                                ctx=1024),
    128: configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=1, n_q_heads=5, tail_min=128, tail_max=1024, margin=0,
                                  ctx=1024),
}


@pytest.mark.parametrize("D", [256, 128])
def test_seal_ill_conditioned_tiles(D):
    import torch
    w = SHAPES[D]
    G = len(KINDS)
    n = 128 + 128 * (G + 1)
    _say(f"[seal-exact D={D}] {G} groups, k_bits {w.k_bits}")
    signs = inputs.rotation_signs(w.seed) if D == 128 else None
    words = inputs.signs_to_words(signs) if signs is not None else [0, 0, 0, 0]
    gpu = kvq.Cache(kvq.config_for(w, max_ctx=n, max_seqs=1, sign_words=words))
    ora = ocache.OracleCache(1, 1, D, w.n_q_heads, 1, n, w.tail_min, w.tail_max, w.margin, w.k_bits, w.v_bits,
                             w.passes, signs)
    z = np.zeros((1, n, 1, D), np.float16)
    gpu.append(0, [0], torch.from_numpy(z).cuda(), torch.from_numpy(z).cuda())
    assert ora.append(0, [0], z, z) == ocache.OK
    kinds = {}
    for r in range(G):
        kk, vk = KINDS[r], KINDS[(r + 1) % G]
        dk, uk = _tile(kk, D, 100 + r)
        dv, uv = _tile(vk, D, 200 + r)
        kinds[r] = (kk, vk)
        for side, (dd, uu, kind) in enumerate(((dk, uk, kk), (dv, uv, vk))):
            if kind.startswith("offset"):
                rho = _first_pass_rho(dd, uu)
                want = 1e-3 if kind == "offset1e3" else 1e-5
                _say(f"[seal-exact D={D}] group {r} side {side} {kind}: column spread / RMS after one row pass "
                     f"{rho:.2e}")
                assert want / 5 <= rho <= want * 5
        for t in range(128):
            buf = _slot_bytes(dk, uk, dv, uv, t)
            slot = 128 * r + t
            gpu.import_(0, 0, 0, kvq.REGION_RING, slot, buf)
            ora.import_ring(0, 0, 0, slot, buf)
    assert gpu.seal(-1, kvq.SEAL_TO_MIN) == ora.seal(-1, ocache.SEAL_TO_MIN) == G
    torch.cuda.synchronize()
    sub = record.sub_width(D)
    worst = {}
    for r in range(G):
        gsub = record.parse_record(gpu.export(0, 0, 0, kvq.REGION_BODY, r), D, w.k_bits, w.v_bits)
        osub = record.parse_record(ora.export(0, 0, 0, ocache.REGION_BODY, r), D, w.k_bits, w.v_bits)
        for side, bits in ((0, w.k_bits), (1, w.v_bits)):
            kind = kinds[r][side]
            x = ora.ring_tile(0, 0, 0, 128 + 128 * r, side)
            for i in range(len(gsub)):
                g, o = gsub[i][side], osub[i][side]
                xs = x[:, i * sub:(i + 1) * sub]
                assert np.all(np.isfinite(g["C"].astype(np.float64)))
                rel = float(np.max(np.abs(g["C"].astype(np.float64) / o["C"].astype(np.float64) - 1)))
                worst[kind] = max(worst.get(kind, 0.0), rel)
                assert rel <= SCALE_TOL, (kind, r, side, rel)
                if kind in ("pow2", "repeated"):
                    assert np.all(o["C"] == np.float16(1.0)) and np.all(g["C"] == np.float16(1.0)), kind
                codes, S, Z = rounding.round_rows(xs, g["C"], bits)
                assert np.array_equal(S, g["S"]) and np.array_equal(Z, g["Z"]), (kind, r, side)
                bad = codes != g["codes"]
                if bad.any():
                    t = rounding.pre_round_values(xs, g["C"], g["S"], g["Z"])
                    k = np.floor(t[bad])
                    assert np.all(np.abs(t[bad] - (k + 0.5)) <= BOUNDARY_REL * np.abs(k + 0.5)), (kind, r, side)
    _say(f"[seal-exact D={D}] max C relative error by kind: " +
         ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    gpu.close()
