"""The allocation-free decode (kvq_attn_decode_noalloc) against kvq_attn_decode
with a caller workspace: the same kernels, so the outputs must be equal bit
for bit.  Two calls in a row on the same GPU, the second with a smaller input
(fewer sequences, a shorter context), so the second reads nothing the first
left in the shared scratch array; then a call whose partials exceed the
array is refused with KVQ_ERR_CAPACITY before anything is enqueued."""
import sys

import numpy as np
import pytest

from quantized_kv_cache_seal_amd import configs, inputs, kvq

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _cache(w, lens, chunk=512):
    import torch
    gpu = kvq.Cache(kvq.config_for(w, max_ctx=max(lens), max_seqs=len(lens)))
    specs = [inputs.KVSpec(w.n_layers, w.n_kv_heads, w.head_dim, w.seed + 31 * s, w.k_dist, w.outliers,
                           w.outlier_scale) for s in range(len(lens))]
    for s, n in enumerate(lens):
        for t0 in range(0, n, chunk):
            m = min(chunk, n - t0)
            for l in range(w.n_layers):
                k = torch.from_numpy(specs[s].tokens(l, "k", t0, m)[None]).cuda()
                v = torch.from_numpy(specs[s].tokens(l, "v", t0, m)[None]).cuda()
                gpu.append(l, [s], k, v)
            gpu.seal(-1, kvq.SEAL_IF_FULL)
    gpu.seal(-1, kvq.SEAL_TO_MIN)
    return gpu


def test_noalloc_decode_matches_workspace_decode():
    import torch
    w = configs.QWEN27B.scaled(n_layers=2, tail_min=256, tail_max=512)
    lens = [3000, 1700, 900]
    gpu = _cache(w, lens)
    for call, (layer, seqs) in enumerate(((1, [0, 1, 2]), (0, [2]))):
        q = torch.from_numpy(inputs.queries(w.seed, call, layer, len(seqs), w.n_q_heads, w.head_dim)).cuda()
        for path in (kvq.PATH_MFMA, kvq.PATH_VALU):
            gpu.set_decode_path(path)
            for f16 in (False, True):
                want = gpu.attn_decode(layer, seqs, q, scale=0.9, out_f16=f16)
                got = gpu.attn_decode_noalloc(layer, seqs, q, scale=0.9, out_f16=f16)
                torch.cuda.synchronize()
                same = torch.equal(got, want)
                _say(f"[noalloc] call {call} layer {layer} seqs {seqs} path {path} f16 {f16}: equal {same}")
                assert same
                assert torch.isfinite(got.float()).all()
    gpu.close()


def test_noalloc_refuses_calls_beyond_its_scratch():
    """16 sequences with a 4,096-token ring each on the vector-ALU path (one
    partial per 128 ring tokens, plus the sink): 16 x 16 query heads x 33
    partials x 1,040 bytes = 8.8 MB of partials, beyond the 8 MiB array: the
    call is refused; half the sequences fit, and match the workspace decode."""
    import torch
    w = configs.QWEN27B.scaled(n_layers=1, n_kv_heads=1, n_q_heads=16, tail_min=4096, tail_max=4096, margin=0,
                               outliers=0)
    n, lens = 16, 128 + 4096
    gpu = kvq.Cache(kvq.config_for(w, max_ctx=lens, max_seqs=n))
    kv = torch.from_numpy(inputs.normal_np(9, 1, 0, n * lens * 256).astype(np.float16).reshape(n, lens, 1, 256))
    kv = kv.cuda()
    gpu.append(0, list(range(n)), kv, kv)
    q = torch.from_numpy(inputs.queries(w.seed, 0, 0, n, 16, 256)).cuda()
    gpu.set_decode_path(kvq.PATH_VALU)
    with pytest.raises(kvq.KVQError) as e:
        gpu.attn_decode_noalloc(0, list(range(n)), q)
    assert e.value.status == kvq.ERR_CAPACITY
    _say(f"[noalloc] refused: {e.value}")
    half = list(range(n // 2))
    qh = q[: n // 2].contiguous()
    got = gpu.attn_decode_noalloc(0, half, qh)
    want = gpu.attn_decode(0, half, qh)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    gpu.close()
