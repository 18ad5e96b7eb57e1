"""GPU parity of block attention (prefill chunks and speculative verify
blocks): kvq_attn_prefill through the C ABI against the oracle's float64 causal
attention over the same cache, element by element.

The GPU cache takes the oracle's records (import), so both sides read the same
bytes; each case builds the cache with the seal rule as the workloads do, then
attends the newest n_q tokens.  Block sizes cover one row, single and several
16-row tiles with ragged ends, blocks longer than the unsealed tail (rows whose
own tokens are sealed: the body's causal mask), and blocks that start inside
the sink; 48-row blocks (three row tiles per record item); every body width (4/4, 8/4, 3/3, 3/2, 2/2, 2/3) and both staging
formats.  Criterion per (sequence, query token): max |o_gpu - o_ref| over the
token's heads and channels / rms of the token's reference outputs <= 2e-3."""
import math
import sys

import numpy as np
import pytest

from quantized_kv_cache_seal_amd import configs, inputs, kvq

from harness import ATTN_TOL, Pair

pytestmark = pytest.mark.gpu

CASES = {
    # config 1 (256-wide, GQA 4, 4/4): verify-sized blocks, a long chunk, one reaching 44 tokens into the body
    "tiny": (configs.TINY, [2048], 512, None, [1, 7, 12, 64, 300]),
    # f16 staging ring (exact tail in the original domain)
    "tiny_f16": (configs.TINY_F16, [2048], 512, None, [5, 130, 400]),
    # config 2 shape (4 KV heads x 256, GQA 6), two sequences of different lengths
    "qwen27b": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=2600), [2600, 1300], 300,
                None, [3, 8, 16, 100]),
    # 8-bit keys at 256-wide heads: a 48-row verify block (three row tiles) and a longer one
    "qwen27b_k8": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=1800, k_bits=8), [1800], 300,
                   None, [8, 40]),
    # config 3 shape: 512-wide heads as two 256-point halves, GQA 8
    "gemma": (configs.GEMMA31B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=1500), [1500], 256, None,
              [2, 40, 300]),
    # config 4 shape: 128-wide heads, randomized WHT, 8-bit keys, GQA 5
    "qwen14b": (configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2, n_q_heads=10, tail_min=256, tail_max=512,
                                         ctx=1900), [1900, 700], 500, "signs", [1, 9, 100]),
    "qwen14b_f16": (configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2, n_q_heads=10, tail_min=256, tail_max=512,
                                             ctx=1500, stage="f16"), [1500], 300, "signs", [33]),
    # lower scalar bodies at the config 2 shape (SJ-KVaRN 2.3: 3/3, 3/2; and 2/2 with f16 staging, 2/3)
    "qwen27b_33": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=2600, k_bits=3, v_bits=3),
                   [2600, 1300], 300, None, [5, 100, 300]),
    "qwen27b_32": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=2600, k_bits=3, v_bits=2),
                   [2600], 300, None, [16, 64]),
    "qwen27b_22": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=2600, k_bits=2, v_bits=2,
                                          stage="f16"), [2600], 300, None, [8, 200]),
    "qwen27b_23": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=1800, k_bits=2, v_bits=3),
                   [1800], 300, None, [40]),
    # config 5 shape: a ragged batch, one block starting inside the sink
    "batched": (configs.BATCHED.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=3000), [130, 700, 3000], 128,
                None, [1, 100, 130]),
}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    w, lens, chunk, signs, blocks = CASES[request.param]
    _say(f"[prefill {request.param}] build lens={lens} chunk={chunk}")
    sg = inputs.rotation_signs(w.seed) if signs else None
    p = Pair(w, lens, sg).build(chunk)
    p.import_oracle_records()
    p.name = request.param
    p.blocks = blocks
    return p


def block_errors(p, layer, n_q, step, scale=1.0, out_f16=False):
    """Per (sequence, token) errors of one block attention call; also the GPU output."""
    t = p.torch
    q = inputs.block_queries(p.w.seed, step, layer, p.n, n_q, p.w.n_q_heads, p.w.head_dim)
    out = p.gpu.attn_prefill(layer, list(range(p.n)), t.from_numpy(q).cuda(), scale=scale, out_f16=out_f16)
    got = out.float().cpu().numpy().astype(np.float64)
    errs = np.zeros((p.n, n_q))
    refs = []
    for s in range(p.n):
        ref = p.ora.attention_block(layer, s, q[s], scale)
        refs.append(ref)
        for i in range(n_q):
            rms = math.sqrt(np.mean(ref[i] ** 2))
            d = np.abs(got[s, i] - ref[i])
            if out_f16:
                d = d - np.abs(ref[i]) * 2.0 ** -11  # fp16's own rounding, half an ulp
            errs[s, i] = float(d.max() / rms)
    return errs, got, refs


def test_block_attention_matches_oracle(case):
    for n_q in case.blocks:
        errs, _, _ = block_errors(case, 0, n_q, step=n_q)
        info = [case.ora.info(s, 0) for s in range(case.n)]
        _say(f"[prefill {case.name}] n_q={n_q} (n_tok, n_rec, ring)={info} err={errs.max():.2e} "
             f"at (seq, token)={np.unravel_index(np.argmax(errs), errs.shape)}")
        assert errs.max() <= ATTN_TOL


def test_block_attention_f16_output_and_scale(case):
    n_q = case.blocks[-1]
    errs, _, _ = block_errors(case, 0, n_q, step=1000 + n_q, scale=0.7, out_f16=True)
    _say(f"[prefill {case.name}] n_q={n_q} f16 out, scale 0.7: err beyond fp16 rounding={errs.max():.2e}")
    assert errs.max() <= ATTN_TOL


def test_block_attention_deterministic(case):
    t = case.torch
    n_q = case.blocks[-1]
    q = inputs.block_queries(case.w.seed, 7, 0, case.n, n_q, case.w.n_q_heads, case.w.head_dim)
    qd = t.from_numpy(q).cuda()
    a = case.gpu.attn_prefill(0, list(range(case.n)), qd).cpu().numpy()
    b = case.gpu.attn_prefill(0, list(range(case.n)), qd).cpu().numpy()
    assert np.array_equal(a, b)


def test_whole_cache_as_the_block():
    """Every cached token is in the block (a fresh prefill): the first row sees
    one token and equals its value; the causal mask runs over sink and ring."""
    w = configs.TINY.scaled(tail_min=256, tail_max=512)
    p = Pair(w, [600]).build(600, seal_to_min=False, seal_every=False)
    assert p.ora.info(0, 0) == (600, 0, 600 - 128)
    errs, got, refs = block_errors(p, 0, 600, step=3)
    _say(f"[prefill whole] n_q=600 err={errs.max():.2e}")
    assert errs.max() <= ATTN_TOL
    v0 = p.kv[(0, 0)][1][0, 0].astype(np.float64)
    assert np.allclose(got[0, 0], np.tile(v0, (w.n_q_heads, 1)), rtol=0, atol=1e-3 * np.abs(v0).max())


def test_block_attention_errors():
    w = configs.TINY.scaled(tail_min=256, tail_max=512)
    p = Pair(w, [300]).build(300)
    t = p.torch
    q = t.from_numpy(inputs.block_queries(w.seed, 0, 0, 1, 301, w.n_q_heads, w.head_dim)).cuda()
    with pytest.raises(kvq.KVQError) as e:  # more queries than cached tokens
        p.gpu.attn_prefill(0, [0], q)
    assert e.value.status == kvq.ERR_INVALID
    small = t.empty(64, dtype=t.uint8, device="cuda")
    with pytest.raises(kvq.KVQError) as e:
        p.gpu.attn_prefill(0, [0], q[:, :10].contiguous(), workspace=small)
    assert e.value.status == kvq.ERR_CAPACITY
    # the 2- and 3-bit bodies of 128-wide heads (their decode is the vector-ALU scan)
    w128 = configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=1, n_q_heads=5, tail_min=256, tail_max=512, k_bits=3,
                                    v_bits=3)
    lb = Pair(w128, [300], inputs.rotation_signs(w128.seed)).build(300)
    q128 = t.from_numpy(inputs.block_queries(w128.seed, 0, 0, 1, 10, 5, 128)).cuda()
    with pytest.raises(kvq.KVQError) as e:
        lb.gpu.attn_prefill(0, [0], q128)
    assert e.value.status == kvq.ERR_UNSUPPORTED
