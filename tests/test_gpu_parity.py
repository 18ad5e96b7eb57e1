"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs shaped like the five workloads at sizes the oracle
finishes in seconds (several tiles, ragged tails, ring wrap-around)."""
import sys

import numpy as np
import pytest

from oracle import cache as ocache
from oracle import record
from quantized_kv_cache_seal_amd import configs, inputs, kvq

from harness import ATTN_TOL, Pair

pytestmark = pytest.mark.gpu

SMALL = {
    # config 1 as specified (1 layer, 1 KV head, 256, GQA 4, 2,048 tokens, 8 passes, tail 256/512)
    "tiny": (configs.TINY, [2048], 512, None),
    # config 1 as specified with the f16 staging ring (KVarN-style exact tail)
    "tiny_f16": (configs.TINY_F16, [2048], 512, None),
    # f16 staging at 128-wide heads (randomized WHT at seal time) and at 512-wide heads, ragged
    "qwen14b_f16": (configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2, n_q_heads=10, tail_min=256, tail_max=512,
                                             ctx=1500, stage="f16"), [1500, 700], 300, "signs"),
    "gemma_f16": (configs.GEMMA31B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=1300, stage="f16"),
                  [1300], 256, None),
    # lower scalar bodies at the config 2 shape (SJ-KVaRN 2.3: 3/3, 3/2; and 2/2), two layers, ragged
    "qwen27b_33": (configs.QWEN27B.scaled(n_layers=2, tail_min=256, tail_max=512, ctx=2600, k_bits=3, v_bits=3),
                   [2600, 1300], 300, None),
    "qwen27b_32": (configs.QWEN27B.scaled(n_layers=2, tail_min=256, tail_max=512, ctx=2600, k_bits=3, v_bits=2),
                   [2600], 300, None),
    "qwen27b_22": (configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=2600, k_bits=2, v_bits=2,
                                          stage="f16"), [2600], 300, None),
    # config 2 shape, two layers, ragged chunking
    "qwen27b": (configs.QWEN27B.scaled(n_layers=2, tail_min=256, tail_max=512, ctx=2600), [2600], 300, None),
    # config 3 shape: 512-wide heads as two 256-point halves, Student-t keys
    "gemma": (configs.GEMMA31B.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=1500), [1500], 256, None),
    # config 4 shape: 128-wide heads, randomized WHT, 8-bit keys
    "qwen14b": (configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2, n_q_heads=10, tail_min=256, tail_max=512,
                                         ctx=1900), [1900], 500, "signs"),
    # config 5 shape: a ragged batch (sink-only, exact boundaries, ring-only, wrap-around)
    "batched": (configs.BATCHED.scaled(n_layers=1, tail_min=256, tail_max=512, ctx=3000),
                [1, 127, 128, 129, 700, 3000], 128, None),
}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=list(SMALL))
def pair(request):
    w, lens, chunk, signs = SMALL[request.param]
    _say(f"[case {request.param}] build lens={lens} chunk={chunk}")
    sg = inputs.rotation_signs(w.seed) if signs else None
    p = Pair(w, lens, sg).build(chunk)
    p.name = request.param
    return p


def test_counts(pair):
    pair.check_info()


def test_sink_and_ring_bytes_exact(pair):
    n = pair.check_sink_ring()
    _say(f"[{pair.name}] sink+ring units bit-exact: {n}")
    assert n > 0


def test_records_conditional_parity(pair):
    st = pair.check_records()
    _say(f"[{pair.name}] records: {st}")
    if pair.name != "batched" or any(pair.ora.info(s, 0)[1] for s in range(pair.n)):
        assert st["scales"] > 0
    assert st["boundary"] <= max(1, st["codes"] // 10 ** 5)
    # every code that differs from the oracle's own is explained (check_records
    # asserts it); the fp16 flips of C that explain them are rare
    assert st["c_flips"] <= max(2, st["scales"])


def test_decode_gpu_built_cache(pair):
    """GPU decode over the GPU-built cache against float64 attention over the
    same cache (the GPU's exported records dequantised by the oracle), the
    decode criterion.  The float64 difference between attention over the GPU's
    records and over the oracle's (they differ where an fp16 column scale
    rounded the other way, which the parity rules allow) is reported: one such
    flip in a key channel moves peaked attention by up to ~2e-2 of its RMS."""
    for layer in range(pair.w.n_layers):
        errs, cross = pair.own_record_errors(layer, pair.queries(0, layer))
        _say(f"[{pair.name}] layer={layer} decode (GPU-built cache) err={max(errs):.2e}, "
             f"GPU vs oracle records {max(cross):.2e}")
        assert max(errs) <= ATTN_TOL


@pytest.mark.parametrize("path", [kvq.PATH_VALU, kvq.PATH_MFMA])
def test_decode_on_oracle_records(pair, path):
    """Every small shape has a matrix-core body scan (256 and 512 wide at 4/4
    bits, 128 wide with 8-bit keys) and the vector-ALU reference."""
    pair.import_oracle_records()
    for layer in range(pair.w.n_layers):
        q = pair.queries(0, layer)
        errs, _ = pair.decode_errors(layer, q, path=path)
        _say(f"[{pair.name}] path={path} layer={layer} decode err={max(errs):.2e}")
        assert max(errs) <= ATTN_TOL


def test_decode_f16_output_and_scale(pair):
    """fp16 output: the bound adds fp16's own rounding, half an ulp of each value."""
    pair.import_oracle_records()
    q = pair.queries(1, 0)
    _, got = pair.decode_errors(0, q, scale=0.7, out_f16=True)
    worst = 0.0
    for s in range(pair.n):
        ref = pair.ora.attention(0, s, q[s], 0.7)
        excess = np.abs(got[s] - ref) - np.abs(ref) * 2.0 ** -11
        worst = max(worst, float(excess.max() / np.sqrt(np.mean(ref ** 2))))
    _say(f"[{pair.name}] f16 out, scale 0.7: err beyond fp16 rounding={worst:.2e}")
    assert worst <= ATTN_TOL


def test_streaming_one_token_per_step():
    """Decode-style appends (one token per call) with the seal rule checked after
    every step, through several ring wrap-arounds."""
    w = configs.QWEN27B.scaled(n_layers=1, n_kv_heads=1, n_q_heads=6, tail_min=256, tail_max=384, margin=128,
                               ctx=1200)
    _say("[streaming] build")
    p = Pair(w, [1200]).build(1)
    p.check_info()
    assert p.check_sink_ring() > 0
    st = p.check_records()
    assert st["scales"] == 2 * p.ora.info(0, 0)[1] == 2 * ((1200 - 128 - 256) // 128)
    p.import_oracle_records()
    errs, _ = p.decode_errors(0, p.queries(0, 0))
    assert max(errs) <= ATTN_TOL


def test_many_sequences_split_launches():
    """More sequences than one launch carries (32 per decode launch) and more
    (sequence, layer) seal tasks than one seal launch carries (64): appends,
    seals and decodes split over several launches, each against the oracle."""
    w = configs.QWEN27B.scaled(n_layers=2, n_kv_heads=1, n_q_heads=6, tail_min=256, tail_max=384, ctx=1400)
    lens = [40 + 41 * i for i in range(36)]  # 40 .. 1475: sink-only, ring-only and sealed sequences
    _say(f"[many] build {len(lens)} sequences")
    p = Pair(w, lens, extra_ctx=2).build(128)
    p.check_info()
    assert p.check_sink_ring() > 0
    st = p.check_records()
    _say(f"[many] records: {st}")
    assert st["scales"] > 0 and st["boundary"] == 0
    for layer in range(w.n_layers):
        errs, cross = p.own_record_errors(layer, p.queries(0, layer))
        _say(f"[many] layer={layer} decode (GPU-built cache) err={max(errs):.2e}, GPU vs oracle records {max(cross):.2e}")
        assert max(errs) <= ATTN_TOL
    p.import_oracle_records()
    for path in (kvq.PATH_VALU, kvq.PATH_MFMA):
        errs, _ = p.decode_errors(1, p.queries(1, 1), path=path)
        _say(f"[many] path={path} decode err={max(errs):.2e}")
        assert max(errs) <= ATTN_TOL
    # decode steps: all sequences (three calls: some are still in the sink),
    # then the 33 that have left it (one fused launch per 32 sequences)
    t = p.torch
    for step, seqs in ((7, list(range(p.n))), (8, list(range(3, p.n)))):
        pos = [p.ora.info(s, 0)[0] for s in seqs]
        k = np.stack([p.specs[s].tokens(0, "k", pos[i], 1)[0] for i, s in enumerate(seqs)])
        v = np.stack([p.specs[s].tokens(0, "v", pos[i], 1)[0] for i, s in enumerate(seqs)])
        q = inputs.queries(w.seed, step, 0, len(seqs), w.n_q_heads, w.head_dim)
        rec0 = [p.ora.info(s, 0)[1] for s in seqs]
        out, g = p.gpu.decode_step(0, seqs, t.from_numpy(k).cuda(), t.from_numpy(v).cuda(), t.from_numpy(q).cuda())
        assert p.ora.append(0, seqs, k[:, None], v[:, None]) == ocache.OK
        assert g == p.ora.seal(0, ocache.SEAL_IF_FULL)
        for i, s in enumerate(seqs):
            for r in range(rec0[i], p.ora.info(s, 0)[1]):
                p.ora.import_record(s, 0, 0, r, p.gpu.export(s, 0, 0, kvq.REGION_BODY, r))
        got = out.cpu().numpy().astype(np.float64)
        worst = 0.0
        for i, s in enumerate(seqs):
            ref = p.ora.attention(0, s, q[i], 1.0)
            worst = max(worst, float(np.max(np.abs(got[i] - ref)) / np.sqrt(np.mean(ref ** 2))))
        _say(f"[many] decode step over {len(seqs)} sequences ({g} groups sealed): err={worst:.2e}")
        assert worst <= ATTN_TOL
    p.check_info()
    assert p.check_sink_ring() > 0


@pytest.mark.parametrize("shape", ["d128k4", "d256k8", "d512k8"])
def test_other_body_shapes(shape):
    """The record shapes no configuration uses (128-wide heads with 4-bit keys,
    8-bit keys at 256 and 512): records against the oracle, the matrix-core and
    vector-ALU decodes against float64 attention, and fused decode steps."""
    base = {"d128k4": configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2, n_q_heads=10, k_bits=4),
            "d256k8": configs.QWEN27B.scaled(n_layers=1, n_kv_heads=2, n_q_heads=12, k_bits=8),
            "d512k8": configs.GEMMA31B.scaled(n_layers=1, k_bits=8)}[shape]
    w = base.scaled(tail_min=256, tail_max=512, ctx=1300)
    signs = inputs.rotation_signs(w.seed) if w.head_dim == 128 else None
    _say(f"[{shape}] build")
    p = Pair(w, [1300, 700], signs, extra_ctx=3).build(300)
    p.check_info()
    assert p.check_sink_ring() > 0
    st = p.check_records()
    _say(f"[{shape}] records: {st}")
    assert st["scales"] > 0 and st["boundary"] <= max(1, st["codes"] // 10 ** 5)
    errs, cross = p.own_record_errors(0, p.queries(0, 0))
    _say(f"[{shape}] decode (GPU-built cache) err={max(errs):.2e}, GPU vs oracle records {max(cross):.2e}")
    assert max(errs) <= ATTN_TOL
    p.import_oracle_records()
    for path in (kvq.PATH_VALU, kvq.PATH_MFMA):
        errs, _ = p.decode_errors(0, p.queries(1, 0), path=path)
        _say(f"[{shape}] path={path} decode err={max(errs):.2e}")
        assert max(errs) <= ATTN_TOL
    p.gpu.set_decode_path(kvq.PATH_AUTO)
    t = p.torch
    seqs = [0, 1]
    for step in range(3):
        pos = [p.ora.info(s, 0)[0] for s in seqs]
        k = np.stack([p.specs[s].tokens(0, "k", pos[s], 1)[0] for s in seqs])
        v = np.stack([p.specs[s].tokens(0, "v", pos[s], 1)[0] for s in seqs])
        q = inputs.queries(w.seed, 50 + step, 0, 2, w.n_q_heads, w.head_dim)
        out, g = p.gpu.decode_step(0, seqs, t.from_numpy(k).cuda(), t.from_numpy(v).cuda(), t.from_numpy(q).cuda())
        assert p.ora.append(0, seqs, k[:, None], v[:, None]) == ocache.OK
        assert g == 0 == p.ora.seal(0, ocache.SEAL_IF_FULL)
        got = out.cpu().numpy().astype(np.float64)
        for s in seqs:
            ref = p.ora.attention(0, s, q[s], 1.0)
            err = float(np.max(np.abs(got[s] - ref)) / np.sqrt(np.mean(ref ** 2)))
            assert err <= ATTN_TOL, (shape, step, s, err)
    assert p.check_sink_ring() > 0


@pytest.mark.parametrize("shape,group", [("d256k4", 16), ("d128k8", 12), ("d512k4", 9)])
def test_groups_over_eight(shape, group):
    """Groups of more than 8 query heads per KV head (no configuration has
    one): the matrix-core body then carries hi and lo in separate products,
    and q~ rows i + 8.  Both decode paths against float64 attention over the
    oracle's records, and fused decode steps."""
    base = {"d256k4": configs.QWEN27B.scaled(n_layers=1, n_kv_heads=1),
            "d128k8": configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2),
            "d512k4": configs.GEMMA31B.scaled(n_layers=1, n_kv_heads=2)}[shape]
    w = base.scaled(n_q_heads=group * base.n_kv_heads, tail_min=256, tail_max=512, ctx=1300)
    signs = inputs.rotation_signs(w.seed) if w.head_dim == 128 else None
    _say(f"[{shape} g{group}] build")
    p = Pair(w, [1300, 900], signs, extra_ctx=3).build(300)
    p.check_info()
    p.import_oracle_records()
    for path in (kvq.PATH_VALU, kvq.PATH_MFMA):
        errs, _ = p.decode_errors(0, p.queries(1, 0), path=path)
        _say(f"[{shape} g{group}] path={path} decode err={max(errs):.2e}")
        assert max(errs) <= ATTN_TOL
    p.gpu.set_decode_path(kvq.PATH_AUTO)
    t = p.torch
    seqs = [0, 1]
    for step in range(2):
        pos = [p.ora.info(s, 0)[0] for s in seqs]
        k = np.stack([p.specs[s].tokens(0, "k", pos[s], 1)[0] for s in seqs])
        v = np.stack([p.specs[s].tokens(0, "v", pos[s], 1)[0] for s in seqs])
        q = inputs.queries(w.seed, 70 + step, 0, 2, w.n_q_heads, w.head_dim)
        out, g = p.gpu.decode_step(0, seqs, t.from_numpy(k).cuda(), t.from_numpy(v).cuda(), t.from_numpy(q).cuda())
        assert p.ora.append(0, seqs, k[:, None], v[:, None]) == ocache.OK
        assert g == 0 == p.ora.seal(0, ocache.SEAL_IF_FULL)
        got = out.cpu().numpy().astype(np.float64)
        for s in seqs:
            ref = p.ora.attention(0, s, q[s], 1.0)
            err = float(np.max(np.abs(got[s] - ref)) / np.sqrt(np.mean(ref ** 2)))
            assert err <= ATTN_TOL, (shape, group, step, s, err)
    assert p.check_sink_ring() > 0


@pytest.mark.parametrize("passes", [0, 1, 3, 5])
def test_records_other_pass_counts(passes):
    """Balancing pass counts other than the configurations' 8 and 16 (SJ-KVaRN
    2.2: alternating passes, rows first): none and a single row pass (every
    column scale stays 1), and odd counts, whose last pass is a row pass (the
    column scales come from the column pass before it).  Records by the
    conditional rule at the config 2 shape and at 128-wide heads."""
    for base, signs in ((configs.QWEN27B, False), (configs.QWEN14B1M, True)):
        w = base.scaled(n_layers=1, n_kv_heads=2, n_q_heads=2 * (base.n_q_heads // base.n_kv_heads), tail_min=256,
                        tail_max=512, ctx=1200, passes=passes)
        sg = inputs.rotation_signs(w.seed) if signs else None
        _say(f"[passes {passes}] {w.name} build")
        p = Pair(w, [1200], sg).build(300)
        st = p.check_records()
        _say(f"[passes {passes}] {w.name} records: {st}")
        assert st["scales"] > 0 and st["boundary"] <= max(1, st["codes"] // 10 ** 5)
        if passes < 2:
            for r in range(p.ora.info(0, 0)[1]):
                for sub in record.parse_record(p.gpu.export(0, 0, 0, kvq.REGION_BODY, r), w.head_dim, w.k_bits,
                                               w.v_bits):
                    assert np.all(sub[0]["C"] == np.float16(1.0)) and np.all(sub[1]["C"] == np.float16(1.0))


@pytest.mark.parametrize("shape", [(512, 3, 2), (128, 3, 3), (128, 2, 2)])
def test_low_bit_bodies_other_widths(shape):
    """Lower scalar bodies at 512- and 128-wide heads (the vector-ALU body scan
    takes them; the matrix-core scan refuses them): records by the conditional
    rule, decode against float64 attention."""
    D, kb, vb = shape
    base = configs.GEMMA31B if D == 512 else configs.QWEN14B1M
    w = base.scaled(n_layers=1, n_kv_heads=2, n_q_heads=8 if D == 512 else 10, tail_min=256, tail_max=512,
                    ctx=1400, k_bits=kb, v_bits=vb)
    signs = inputs.rotation_signs(w.seed) if D == 128 else None
    _say(f"[lowbit {shape}] build")
    p = Pair(w, [1400], signs).build(200)
    p.check_info()
    assert p.check_sink_ring() > 0
    st = p.check_records()
    _say(f"[lowbit {shape}] records: {st}")
    assert st["scales"] > 0 and st["boundary"] <= max(1, st["codes"] // 10 ** 5)
    errs, _ = p.own_record_errors(0, p.queries(0, 0))
    _say(f"[lowbit {shape}] decode (GPU-built cache) err={max(errs):.2e}")
    assert max(errs) <= ATTN_TOL
    p.gpu.set_decode_path(kvq.PATH_MFMA)
    with pytest.raises(kvq.KVQError):
        p.gpu.attn_decode(0, [0], p.torch.from_numpy(p.queries(0, 0)).cuda())


@pytest.mark.parametrize("name", ["qwen27b", "batched", "gemma", "qwen14b", "tiny_f16", "qwen14b_f16", "qwen27b_32"])
def test_decode_step(name):
    """kvq_decode_step (append one token, seal if full, decode) step after step:
    one fused launch while every new token lands in the ring and no seal is due,
    the three calls otherwise (a sequence still in the sink, a seal step).  Ring
    bytes stay bit-exact with the oracle's appends; the attention of each step
    is checked against float64 attention over the oracle cache (records
    imported from the oracle; on a seal step the just-sealed records are the
    GPU's own: the oracle takes them too before its reference is computed, the
    decode criterion on the same cache)."""
    steps = 40
    signs = None
    if name == "qwen27b":  # ring 360 after the build: the seal fires at step 24
        w = configs.QWEN27B.scaled(n_layers=2, tail_min=256, tail_max=384, ctx=1000)
        lens = [1000]
    elif name == "qwen27b_32":  # a 3/2 body
        w = configs.QWEN27B.scaled(n_layers=1, tail_min=256, tail_max=384, ctx=1000, k_bits=3, v_bits=2)
        lens = [1000, 600]
    elif name == "batched":  # one sequence starts in the sink: unfused until it leaves it
        w = configs.BATCHED.scaled(n_layers=1, n_kv_heads=2, n_q_heads=12, tail_min=256, tail_max=384, ctx=1000)
        lens = [1000, 897, 120]
    elif name == "gemma":  # 512-wide heads, two sequences
        w = configs.GEMMA31B.scaled(n_layers=1, tail_min=256, tail_max=384, ctx=1000)
        lens = [1000, 700]
    elif name == "tiny_f16":  # config 1 with the f16 staging ring
        w = configs.TINY_F16.scaled(tail_min=256, tail_max=384, ctx=1000)
        lens = [1000]
    else:                    # 128-wide heads, randomized WHT, 8-bit keys (f16 staging too)
        w = configs.QWEN14B1M.scaled(n_layers=1, n_kv_heads=2, n_q_heads=10, tail_min=256, tail_max=384, ctx=1000,
                                     stage="f16" if name.endswith("f16") else "tq6")
        lens = [1000]
        signs = inputs.rotation_signs(w.seed)
    _say(f"[step {name}] build lens={lens}")
    p = Pair(w, lens, signs, extra_ctx=steps).build(128)
    p.import_oracle_records()
    t = p.torch
    seqs = list(range(p.n))
    n_seal_steps = 0
    for st in range(steps):
        for l in range(w.n_layers):
            pos = [p.ora.info(s, l)[0] for s in seqs]
            k = np.stack([p.specs[s].tokens(l, "k", pos[s], 1)[0] for s in seqs])
            v = np.stack([p.specs[s].tokens(l, "v", pos[s], 1)[0] for s in seqs])
            q = inputs.queries(w.seed, 100 + st, l, p.n, w.n_q_heads, w.head_dim)
            rec0 = [p.ora.info(s, l)[1] for s in seqs]
            out, g = p.gpu.decode_step(l, seqs, t.from_numpy(k).cuda(), t.from_numpy(v).cuda(),
                                       t.from_numpy(q).cuda(), scale=0.9)
            assert p.ora.append(l, seqs, k[:, None], v[:, None]) == ocache.OK
            assert g == p.ora.seal(l, ocache.SEAL_IF_FULL)
            got = out.cpu().numpy().astype(np.float64)
            n_seal_steps += g > 0
            if g:  # both caches hold the GPU's new records from here on
                for s in seqs:
                    for h in range(w.n_kv_heads):
                        for r in range(rec0[s], p.ora.info(s, l)[1]):
                            p.ora.import_record(s, l, h, r, p.gpu.export(s, l, h, kvq.REGION_BODY, r))
            for s in seqs:
                ref = p.ora.attention(l, s, q[s], 0.9)
                err = float(np.max(np.abs(got[s] - ref)) / np.sqrt(np.mean(ref ** 2)))
                assert err <= ATTN_TOL, (st, l, s, err, g)
    _say(f"[step {name}] {steps} steps, {n_seal_steps} seal steps")
    assert n_seal_steps > 0
    p.check_info()
    assert p.check_sink_ring() > 0


def test_decode_deterministic():
    w = configs.TINY
    p = Pair(w, [1000]).build(256)
    q = p.torch.from_numpy(p.queries(0, 0)).cuda()
    a = p.gpu.attn_decode(0, [0], q).cpu().numpy()
    b = p.gpu.attn_decode(0, [0], q).cpu().numpy()
    assert np.array_equal(a, b)


def test_save_restore_and_rollback():
    """kvq_seq_save / kvq_seq_restore: a restored sequence decodes bit for bit
    as the saved one did, into its own slot or another; restoring a snapshot
    taken before more tokens were appended and sealed rolls the sequence back
    past the new seal boundary; blobs that do not match are refused and
    change nothing."""
    w = configs.QWEN27B.scaled(n_layers=2, n_kv_heads=2, n_q_heads=12, tail_min=256, tail_max=384, ctx=1300)
    p = Pair(w, [1300, 700], extra_ctx=600).build(300)
    p.import_oracle_records()
    t = p.torch
    q = p.queries(7, 0)
    _, out0 = p.decode_errors(0, q)
    counts0 = [p.gpu.info(0, l) for l in range(w.n_layers)]
    blob = p.gpu.save(0)
    assert blob.nbytes == p.gpu.save_bytes(0)
    _say(f"[save] seq 0 counts {counts0}, {blob.nbytes} bytes")

    # roll forward: 512 more tokens in every layer, sealed as they fill
    extra = 512
    for l in range(w.n_layers):
        n = p.gpu.info(0, l)[0]
        k = p.specs[0].tokens(l, "k", n, extra)[None]
        v = p.specs[0].tokens(l, "v", n, extra)[None]
        for c0 in range(0, extra, 128):
            p.gpu.append(l, [0], t.from_numpy(k[:, c0:c0 + 128].copy()).cuda(), t.from_numpy(v[:, c0:c0 + 128].copy()).cuda())
            p.gpu.seal(l, kvq.SEAL_IF_FULL)
    grown = [p.gpu.info(0, l) for l in range(w.n_layers)]
    assert all(g[1] > c[1] for g, c in zip(grown, counts0)), (grown, counts0)  # records were sealed
    assert p.gpu.truncate(0, -1, counts0[0][0]) == kvq.ERR_SEALED           # truncate cannot go back

    # rollback by restore: counts and decode exactly as saved
    assert p.gpu.restore(0, blob) == kvq.OK
    assert [p.gpu.info(0, l) for l in range(w.n_layers)] == counts0
    _, out1 = p.decode_errors(0, q)
    assert np.array_equal(out1, out0)
    errs, _ = p.decode_errors(0, q)
    assert max(errs) <= ATTN_TOL

    # into another slot: seq 1 becomes a copy of seq 0
    assert p.gpu.restore(1, blob) == kvq.OK
    q2 = q.copy()
    q2[1] = q[0]
    _, out2 = p.decode_errors(0, q2)
    assert np.array_equal(out2[1], out0[0])
    for l in range(w.n_layers):
        for h in range(w.n_kv_heads):
            for region, idx in ((kvq.REGION_SINK, 5), (kvq.REGION_RING, 3), (kvq.REGION_BODY, counts0[l][1] - 1)):
                assert p.gpu.export(1, l, h, region, idx) == p.gpu.export(0, l, h, region, idx)

    # refused blobs change nothing
    bad = blob.copy()
    bad[0] ^= 0xFF
    assert p.gpu.restore(1, bad) == kvq.ERR_INVALID
    assert p.gpu.restore(1, blob[:-1]) == kvq.ERR_INVALID
    other = kvq.Cache(kvq.config_for(configs.QWEN27B.scaled(n_layers=2, n_kv_heads=2, n_q_heads=12, tail_min=256,
                                                            tail_max=512, ctx=1300), max_ctx=2000, max_seqs=1))
    assert other.restore(0, blob) == kvq.ERR_INVALID  # another ring capacity
    assert [p.gpu.info(1, l) for l in range(w.n_layers)] == counts0


def test_degenerate_inputs():
    """The method's degenerate cases through append, seal and decode, against
    the oracle: all-zero tokens (tq6_0 scale 0, an all-zero tile through the
    balancing, row scale 0 read as 1), a one-token sequence (the output is its
    value), one token repeated 1,000 times (constant columns: they keep their
    scales), and keys with channels far above the rest (+-2,000, and +-60,000
    near the fp16 maximum); sink and ring bytes exact, records by the
    conditional rule, attention within tolerance."""
    w = configs.QWEN27B.scaled(n_layers=1, n_kv_heads=2, n_q_heads=8, tail_min=256, tail_max=384, ctx=1000)
    lens = [1000, 1, 1000, 1000, 1000]
    p = Pair(w, lens, extra_ctx=4)
    H, D = w.n_kv_heads, w.head_dim
    zeros = np.zeros((lens[0], H, D), dtype=np.float16)
    p.kv[(0, 0)] = (zeros, zeros.copy())
    k4, v4 = (np.repeat(a[:1], lens[4], axis=0) for a in p.kv[(4, 0)])  # one token repeated
    p.kv[(4, 0)] = (k4, v4)
    for s, big in ((2, 2000.0), (3, 60000.0)):
        k, v = (a.copy() for a in p.kv[(s, 0)])
        k[:, :, 7] = np.where(np.arange(lens[s]) % 2 == 0, big, -big)[:, None].astype(np.float16)
        k[:, 1, 100] = np.float16(big / 2)
        p.kv[(s, 0)] = (k, v)
    p.build(300)
    p.check_info()
    assert p.check_sink_ring() > 0
    st = p.check_records()
    _say(f"[degenerate] records: {st}")
    assert st["scales"] > 0 and st["boundary"] <= max(1, st["codes"] // 10 ** 5)
    p.import_oracle_records()
    q = p.queries(3, 0)
    t = p.torch
    for path in (kvq.PATH_VALU, kvq.PATH_MFMA):
        p.gpu.set_decode_path(path)
        got = p.gpu.attn_decode(0, list(range(len(lens))), t.from_numpy(q).cuda()).float().cpu().numpy()
        got = got.astype(np.float64)
        assert np.all(np.isfinite(got)), path
        assert np.abs(got[0]).max() <= 1e-30, (path, np.abs(got[0]).max())  # zero values everywhere
        one = p.kv[(1, 0)][1][0].astype(np.float64)                           # [H][D]
        want = np.repeat(one, w.n_q_heads // H, axis=0)
        assert np.abs(got[1] - want).max() <= 1e-6 * np.abs(want).max(), path
        ref4 = p.ora.attention(0, 4, q[4], 1.0)
        err4 = float(np.max(np.abs(got[4] - ref4)) / np.sqrt(np.mean(ref4 ** 2)))
        _say(f"[degenerate] path={path} repeated token err={err4:.2e}")
        assert err4 <= ATTN_TOL
        for s in (2, 3):
            # +-2,000 and +-60,000 keys (near the fp16 maximum): the key codes
            # enter the score centred, with the zero point Z + mid S, so no two
            # fp32 terms of the row's range cancel to the score
            ref = p.ora.attention(0, s, q[s], 1.0)
            err = float(np.max(np.abs(got[s] - ref)) / np.sqrt(np.mean(ref ** 2)))
            _say(f"[degenerate] path={path} seq {s} err={err:.2e}")
            assert err <= ATTN_TOL, (path, s, err)

def test_read_probe_checksum():
    """The read probe (the bench's HBM read ceiling) reads every 16 bytes of
    its buffer once: the XOR of its output words equals the XOR of the
    buffer's 32-bit words.  Nine and a half grid strides of 64 MiB (past the
    eight loads a thread has in flight) and a ragged tail."""
    import torch
    n = 9 * (64 << 20) + (32 << 20) + 4096 + 16
    host = np.random.default_rng(5).integers(0, 2 ** 32, size=n // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.uint8)).cuda()
    out = kvq.read_probe(src)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)
