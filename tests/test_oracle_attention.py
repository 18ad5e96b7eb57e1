"""Pins for the oracle's float64 attention (SJ-KVaRN section 2.1; KV Cache
Precision Tail section 2: all regions under one softmax; KV cache math: q.k
survives rotation)."""
import math

import numpy as np

from oracle import attention, rotation
from quantized_kv_cache_seal_amd import inputs


def _brute(q, k, v, scale):
    s = [scale * sum(q[c] * k[t][c] for c in range(len(q))) for t in range(len(k))]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = sum(w)
    return [sum(w[t] * v[t][c] for t in range(len(k))) / tot for c in range(len(q))]


def test_against_pure_python_brute_force():
    q = inputs.normal_np(1, 1, 0, 8)
    k = inputs.normal_np(1, 2, 0, 40).reshape(5, 8)
    v = inputs.normal_np(1, 3, 0, 40).reshape(5, 8)
    got = attention.attend(q, k, v, 0.7)
    ref = _brute(q.tolist(), k.tolist(), v.tolist(), 0.7)
    assert np.allclose(got, ref, rtol=0, atol=1e-14)


def test_degenerate_cases():
    v = inputs.normal_np(2, 3, 0, 64).reshape(4, 16)
    q = inputs.normal_np(2, 1, 0, 16)
    assert np.allclose(attention.attend(q, v[:1] * 0 + 1, v[:1], 1.0), v[0], atol=0)
    same = np.repeat(inputs.normal_np(2, 2, 0, 16)[None], 4, axis=0)
    assert np.allclose(attention.attend(q, same, v, 1.0), v.mean(axis=0), atol=1e-15)


def test_split_invariance():
    q = inputs.normal_np(3, 1, 0, 32)
    k = inputs.normal_np(3, 2, 0, 32 * 300).reshape(300, 32)
    v = inputs.normal_np(3, 3, 0, 32 * 300).reshape(300, 32)
    one = attention.attend(q, k, v, 0.3)
    for cuts in ([0, 128, 300], [0, 1, 7, 200, 299, 300], [0, 300]):
        parts = [attention.partial(q, k[a:b], v[a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
        assert np.max(np.abs(attention.merge_partials(parts) - one)) < 1e-13


def test_rotated_domain_equals_original():
    signs = inputs.rotation_signs(5)
    for d in (128, 256, 512):
        q = inputs.normal_np(4, 1, 0, d)
        k = inputs.normal_np(4, 2, 0, 50 * d).reshape(50, d)
        v = inputs.normal_np(4, 3, 0, 50 * d).reshape(50, d)
        ref = attention.attend(q, k, v, 1 / math.sqrt(d))
        rq = rotation.rotate_exact(q, d, signs)
        rk = rotation.rotate_exact(k, d, signs)
        rv = rotation.rotate_exact(v, d, signs)
        out = rotation.inverse_exact(attention.attend(rq, rk, rv, 1 / math.sqrt(d)), d, signs)
        assert np.max(np.abs(out - ref)) < 1e-12


def test_gqa_mapping():
    q = inputs.normal_np(6, 1, 0, 6 * 16).reshape(6, 16)
    ks = [inputs.normal_np(6, 2 + h, 0, 160).reshape(10, 16) for h in range(2)]
    vs = [inputs.normal_np(6, 4 + h, 0, 160).reshape(10, 16) for h in range(2)]
    out = attention.attend_gqa(q, ks, vs, 0.5)
    for h in range(6):
        assert np.array_equal(out[h], attention.attend(q[h], ks[h // 3], vs[h // 3], 0.5))
