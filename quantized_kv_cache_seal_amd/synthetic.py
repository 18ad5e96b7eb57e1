"""Build a cache of a synthetic workload through the real path (chunked append
plus seal-if-full, finishing with the idle seal-back), with every key and value
drawn on the device by the seeded generator.  The result is the "just sealed"
state: ring length tail_min (SJ-KVaRN 4.3: an idle server seals back to
4,096)."""
from __future__ import annotations

import torch

from . import inputs, kvq


def spec_for(w, seq: int = 0) -> inputs.KVSpec:
    return inputs.KVSpec(w.n_layers, w.n_kv_heads, w.head_dim, w.seed + 7919 * seq, w.k_dist,
                         w.outliers, w.outlier_scale)


def sign_words(w):
    return inputs.signs_to_words(inputs.rotation_signs(w.seed)) if w.head_dim == 128 else [0, 0, 0, 0]


def signs(w):
    return inputs.rotation_signs(w.seed) if w.head_dim == 128 else None


def build(w, ctx: int = None, max_ctx: int = None, n_seqs: int = None, chunk: int = None,
          device="cuda", seal_to_min=True, seal_if_full=True, log=None) -> kvq.Cache:
    ctx = w.ctx if ctx is None else ctx
    n_seqs = w.n_seqs if n_seqs is None else n_seqs
    chunk = w.margin if chunk is None else chunk
    cfg = kvq.config_for(w, max_ctx=max_ctx or ctx, max_seqs=n_seqs, sign_words=sign_words(w))
    cache = kvq.Cache(cfg, device=device)
    specs = [spec_for(w, s) for s in range(n_seqs)]
    seqs = list(range(n_seqs))
    for layer in range(w.n_layers):
        for t0 in range(0, ctx, chunk):
            n = min(chunk, ctx - t0)
            k = torch.stack([sp.tokens(layer, "k", t0, n, backend="torch", device=device) for sp in specs])
            v = torch.stack([sp.tokens(layer, "v", t0, n, backend="torch", device=device) for sp in specs])
            cache.append(layer, seqs, k.contiguous(), v.contiguous())
            if seal_if_full:
                cache.seal(layer, kvq.SEAL_IF_FULL)
        if log:
            log(f"built layer {layer}: {cache.info(0, layer)}")
    if seal_to_min:
        cache.seal(-1, kvq.SEAL_TO_MIN)
    torch.cuda.synchronize()
    return cache
