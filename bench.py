#!/usr/bin/env python
"""Decode-step benchmark of the quantized KV-cache hot path on one MI355X.

Workload: the Qwen 27B-class full-attention shape (16 layers, 4 KV heads x 256,
24 query heads) at a 110,592-token context in the just-sealed state (sink 128,
831 sealed records per head, 4,096 ring tokens), keys and values drawn by the
seeded generator.  One step = for every layer one kvq_decode_step: append one
token (rotation + tq6_0 staging), the seal-if-full check, and decode attention
of one query over all four regions (--calls: the three separate calls).  Inputs for every step are resident in HBM before timing.

value = decode-attention effective KV GB/s: the compressed bytes the step must
read (sink fp16 + ring tq6_0 + sealed records, all layers and heads) divided by
the measured time per step.  The seal is measured separately as sealed
tokens/s on a full 4,096-token seal batch (32 groups per layer, 16 layers, 4 KV
heads, K and V).  The oracle (CPU) is timed on a bounded sample for the
cpu_baseline entry.  Progress goes to stderr; stdout carries one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn effective KV GB/s (% HBM peak) at 110,592 ctx; seal tokens/s"
HBM_PEAK_GBS = 8000.0
FP32_VALU_NONPACKED_TFLOPS = 78.6  # fp32 vector peak without packed instructions (disabled in this build)
FP32_VALU_PEAK_TFLOPS = 157.3
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_main_kernel_qwen27b_ctx110592.md")
# the decode kernel's source and the headers it includes
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_kv_cache_seal_amd", "csrc", f) for f in
                  ("kvq_decode_fused.hip", "kvq_codes.h", "kvq_mfma.h", "kvq_encode.h", "kvq_device.h",
                   "kvq_layout.h")]


def kernel_sha():
    """First 16 hex digits of the SHA-256 of the decode kernel's sources, concatenated."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def profile_record(key):
    """The `key:` record line of the decode profile summary as a dict, or None
    when the summary is missing or the kernel sources have changed since it was
    taken."""
    try:
        line = next(l for l in open(TRAFFIC_PROFILE) if l.startswith(key + ":"))
    except (OSError, StopIteration):
        return None
    rec = dict(kv.split("=", 1) for kv in line.split()[1:])
    return rec if rec.get("kernel_sha256") == kernel_sha() else None


def measured_traffic():
    """HBM bytes per launch of the main decode kernel from the counter runs
    recorded in the profile summary (FETCH_SIZE and WRITE_SIZE in KiB per
    dispatch, each times its copy-calibrated scale), or None when the kernel
    source has changed since the counters were taken."""
    rec = profile_record("traffic-record")
    if rec is None:
        return None
    return (float(rec["fetch_kib"]) * float(rec["fetch_scale"]) + float(rec["write_kib"]) * float(rec["write_scale"])) * 1024


def region_bytes(w, rec_bytes, n_tok, n_rec, ring):
    """Algorithmic compressed bytes one decode call reads for one layer (all KV
    heads): the fp16 sink, the tq6_0 ring (98 B per 128 values) and the sealed
    records (rec_bytes each: 34,816 B at head_dim 256, 4-bit K and V)."""
    sink = min(n_tok, 128)
    per_head = sink * 2 * w.head_dim * 2 + ring * 2 * (w.head_dim // 128) * 98 + n_rec * rec_bytes
    return per_head * w.n_kv_heads


def seal_flops_per_tile(passes, rows=128, cols=256):
    # per pass: scale, add, square-accumulate over the tile (3 ops, 4 flops with the fma)
    # plus the final rounding (scale, min/max, subtract, multiply, round: ~6 ops per element)
    return passes * 4 * rows * cols + 6 * rows * cols


kPreWarmMaxSteps = 1000


def run_decode(args, w, torch, kvq, synthetic, inputs, read_first=False):
    L, H, D, Hq, N = w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads, w.n_seqs
    W, K = args.warmup, args.steps
    t0 = time.time()
    cache = synthetic.build(w, ctx=w.ctx, max_ctx=w.ctx + W + 3 * K + kPreWarmMaxSteps + 1)
    log(f"[bench] built {w.name} in {time.time() - t0:.1f}s: layer0 info {cache.info(0, 0)}")
    path = {"auto": kvq.PATH_AUTO, "valu": kvq.PATH_VALU, "mfma": kvq.PATH_MFMA}[args.path]
    cache.set_decode_path(path)
    dev = "cuda"
    seqs = list(range(N))
    specs = [synthetic.spec_for(w, s) for s in seqs]
    # per layer: the new tokens of every step, [step][sequence][H][D], contiguous per step
    nk, nv = [], []
    for l in range(L):
        for kind, dst in (("k", nk), ("v", nv)):
            t = torch.stack([sp.tokens(l, kind, w.ctx, W + 3 * K, backend="torch", device=dev) for sp in specs],
                            dim=1)
            dst.append(t.contiguous())
    qs = [[inputs.queries(w.seed, s, l, N, Hq, D, backend="torch", device=dev).contiguous() for l in range(L)]
          for s in range(W + 3 * K)]
    out = torch.empty((L, N, Hq, D), dtype=torch.float32, device=dev)
    ws = cache.workspace(N)
    stream = torch.cuda.current_stream()

    # host-side counts of every (sequence, layer), advanced by the step itself
    # (one token appended; a seal, which is rare, re-reads the counts), so
    # that the timed loop makes no extra calls
    state = [[list(cache.info(s, l)) for s in seqs] for l in range(L)]   # [n_tok, n_rec, ring]
    rec_bytes = cache.unit_bytes(kvq.REGION_BODY)
    read_ceiling = run_read_ceiling(torch, kvq) if read_first else None

    def one_step(s):
        nbytes = 0
        for l in range(L):
            if args.calls:
                cache.append(l, seqs, nk[l][s], nv[l][s], stream=stream)
                g = cache.seal(l, kvq.SEAL_IF_FULL, stream=stream)
                cache.attn_decode(l, seqs, qs[s][l], out=out[l], workspace=ws, stream=stream)
            else:
                _, g = cache.decode_step(l, seqs, nk[l][s], nv[l][s], qs[s][l], out=out[l], workspace=ws,
                                         stream=stream)
            if g:
                state[l] = [list(cache.info(q, l)) for q in seqs]
            else:
                for st in state[l]:
                    st[0] += 1
                    st[2] += 1
            nbytes += sum(region_bytes(w, rec_bytes, *st) for st in state[l])
        return nbytes

    # Pre-warm: the device's power management settles only after some tens of
    # milliseconds of this load (measured step by step after an idle second:
    # ~565 us for the first 10 steps, 600-666 us for the next 10, then
    # 545 -> 537 us), so the same steps run untimed for prewarm_ms first; their
    # inputs cycle over the generated ones, and the host counts follow them.
    # Python's cyclic garbage collector stays off while steps run: a full
    # collection inside the timed loop (tens of ms, triggered by the objects the
    # calls allocate) would leave the device waiting for work
    gc.collect()
    gc.disable()
    n_pre = 0
    if args.prewarm_ms > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.prewarm_ms and n_pre < kPreWarmMaxSteps:
            one_step(n_pre % (W + 3 * K))
            n_pre += 1
            if n_pre % 8 == 0:  # keep the device fed, the queue short
                torch.cuda.synchronize()
    torch.cuda.synchronize()
    for s in range(W):
        one_step(s)
    torch.cuda.synchronize()
    # the timed steps: nothing but the steps between the two events
    tot_bytes = 0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for s in range(K):
        tot_bytes += one_step(W + s)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / K
    bytes_step = tot_bytes / K
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    # the main kernel's own duration: a second pass of K steps with the
    # library's wall-clock stamps on (two atomics per workgroup, so kept out of
    # the timed steps)
    cache.profile_start(K * L)
    stamp_bytes = 0
    for s in range(K):
        stamp_bytes += one_step(W + K + s)
    kernel_us = cache.profile_stop()
    per_call_bytes = stamp_bytes / (K * L)
    avg_kernel_us = sum(kernel_us) / len(kernel_us)
    achieved = per_call_bytes / (avg_kernel_us * 1e-6) / 1e9
    # the spread of single steps: a third pass of K steps, one event recorded
    # on the stream between consecutive steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for s in range(K):
        one_step(W + 2 * K + s)
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    gc.enable()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(K))
    step_us = {f"p{q}": round(per[min(K - 1, int(round(q / 100 * (K - 1))))], 1) for q in (10, 50, 90)}
    for l in (0, L - 1):
        assert [list(cache.info(q, l)) for q in seqs] == state[l]
    log(f"[bench] decode: {ms_step * 1e3:.1f} us/step (wall {wall / K * 1e3:.1f} ms), {bytes_step / 1e9:.4f} GB/step, "
        f"{gbs:.1f} GB/s; main decode kernel avg {avg_kernel_us:.1f} us over {len(kernel_us)} calls -> "
        f"{achieved:.1f} GB/s; single steps p10/p50/p90 {step_us['p10']}/{step_us['p50']}/{step_us['p90']} us")
    info = cache.info(0, 0)
    sr = run_save_restore(cache, torch, kvq, qs[0][0], ws, stream) if args.save_restore else None
    del cache
    torch.cuda.empty_cache()
    return {
        "ms_per_step": ms_step, "gbs": gbs, "bytes_step": bytes_step, "avg_kernel_us": avg_kernel_us, "step_us": step_us,
        "read_ceiling": read_ceiling, "prewarm_steps": n_pre,
        "achieved": achieved, "per_call_bytes": per_call_bytes, "info_after": info, "save_restore": sr,
    }


def run_prefill(args, w, torch, kvq, synthetic, inputs, blocks):
    """Block attention of the newest n_q tokens (a prefill chunk, a verify
    block) of the built cache, every layer per step, for each n_q in blocks.
    The record launch's matrix-core roofline: algorithmic flops per launch =
    4 D x query rows x sealed tokens (q.k and p.v, two flops per product; the
    block lies in the ring, so every sealed token is visible to every row)."""
    L, H, D, Hq, N = w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads, w.n_seqs
    t0 = time.time()
    cache = synthetic.build(w, ctx=w.ctx, max_ctx=w.ctx)
    n_tok, n_rec, ring = cache.info(0, 0)
    log(f"[bench] prefill cache {w.name} built in {time.time() - t0:.1f}s: layer0 info {(n_tok, n_rec, ring)}")
    stream = torch.cuda.current_stream()
    out = {}
    for n_q in blocks:
        assert n_q <= ring, "the block lies in the ring"
        qs = [inputs.block_queries(w.seed, 500 + l, l, N, n_q, Hq, D, backend="torch", device="cuda").contiguous()
              for l in range(L)]
        o = torch.empty((N, n_q, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(256, cache.prefill_workspace_bytes(N, n_q)), dtype=torch.uint8, device="cuda")
        seqs = list(range(N))

        def step():
            for l in range(L):
                cache.attn_prefill(l, seqs, qs[l], out=o, workspace=ws, stream=stream)

        W, K = max(1, args.warmup // 5), args.prefill_steps
        gc.collect()
        gc.disable()  # as in the decode timing
        for _ in range(W):
            step()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(K):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / K
        cache.profile_start(K * L)  # the record launch's own duration, in a pass of its own
        for _ in range(K):
            step()
        body_us = cache.profile_stop()
        gc.enable()
        rows = N * n_q * Hq
        flops_body = 4.0 * D * rows * kvq_group_tokens(n_rec)
        flops_all = sum(4.0 * D * N * Hq * (n_tok - n_q + t + 1) for t in range(n_q)) * L
        avg_body = sum(body_us) / len(body_us)
        tf_body = flops_body / (avg_body * 1e-6) / 1e12
        cache_bytes = N * region_bytes(w, cache.unit_bytes(kvq.REGION_BODY), n_tok, n_rec, ring) * L
        log(f"[bench] block attention n_q={n_q}: {ms_step * 1e3:.1f} us/step ({L} layers), "
            f"{N * n_q / (ms_step * 1e-3):.0f} tokens/s; record launch avg {avg_body:.1f} us -> {tf_body:.1f} TFLOP/s")
        out[str(n_q)] = {
            "n_q": n_q, "us_per_step": round(ms_step * 1e3, 2),
            "tokens_per_s": round(N * n_q / (ms_step * 1e-3), 1),
            "attn_tflops": round(flops_all / (ms_step * 1e-3) / 1e12, 2),
            "cache_gbs": round(cache_bytes / (ms_step * 1e-3) / 1e9, 1),
            "record_launch_us": round(avg_body, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf_body, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf_body / MFMA_F16_PEAK_TFLOPS, 4),
                         "kernel": "prefill_body_kernel (sealed records of one layer)",
                         "flops_per_launch": flops_body,
                         "flops_basis": "4 x head_dim x query rows (n_q x q_heads) x sealed tokens; the kernel "
                                        "issues twice that on the matrix cores (hi + lo operands)",
                         "time_basis": "library stamps: start of workgroup 0 to the end of the last workgroup",
                         "hbm_floor_us": round(N * H * n_rec * cache.unit_bytes(kvq.REGION_BODY) /
                                               (HBM_PEAK_GBS * 1e9) * 1e6, 2)},
        }
        del ws
    del cache
    torch.cuda.empty_cache()
    return out


def kvq_group_tokens(n_rec):
    return 128 * n_rec


def run_read_ceiling(torch, kvq, gib=4, reps=10, warm_ms=100.0):
    """The device's achievable HBM read rate: kvq_read_probe over a buffer of
    `gib` GiB (16 times the 256 MB Infinity Cache), timed with one event pair
    around `reps` reads after untimed ones that keep the device reading for
    `warm_ms` (its clocks reach their sustained level only after some tens of
    milliseconds of load)."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    out = torch.empty(kvq.READ_PROBE_OUT_BYTES, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        kvq.read_probe(src, out, stream)
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        kvq.read_probe(src, out, stream)
    b.record(stream)
    torch.cuda.synchronize()
    gbs = n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    log(f"[bench] read ceiling: {gbs:.1f} GB/s ({reps} reads of {gib} GiB)")
    del src, out
    torch.cuda.empty_cache()
    return gbs


def run_save_restore(cache, torch, kvq, q, ws, stream):
    """Save sequence 0 (every layer) to host memory and restore it, timed on
    the host around each call (each synchronises its stream), into and out of
    a pinned host buffer allocated beforehand; the decode of layer 0 after the
    restore must equal the one before bit for bit."""
    seqs = [0]
    before = cache.attn_decode(0, seqs, q[:1].contiguous(), workspace=ws, stream=stream).clone()
    host = torch.empty(cache.save_bytes(0), dtype=torch.uint8, pin_memory=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    blob = cache.save(0, stream=stream, out=host.numpy())
    t1 = time.perf_counter()
    assert cache.restore(0, blob, stream=stream) == kvq.OK
    t2 = time.perf_counter()
    after = cache.attn_decode(0, seqs, q[:1].contiguous(), workspace=ws, stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(before, after)
    gb = blob.nbytes / 1e9
    del blob, host
    log(f"[bench] save/restore of sequence 0 (pinned host buffer): {gb:.3f} GB, save {(t1 - t0) * 1e3:.1f} ms "
        f"({gb / (t1 - t0):.1f} GB/s), restore {(t2 - t1) * 1e3:.1f} ms ({gb / (t2 - t1):.1f} GB/s), "
        f"decode after restore bit-identical")
    return {"bytes": int(gb * 1e9), "save_ms": round((t1 - t0) * 1e3, 2), "restore_ms": round((t2 - t1) * 1e3, 2),
            "save_gbs": round(gb / (t1 - t0), 2), "restore_gbs": round(gb / (t2 - t1), 2)}


def run_seal(args, w, torch, kvq, synthetic):
    """Seal batch: the ring of every sequence filled to tail_max in every
    layer, then one seal-if-full seals the oldest (tail_max - tail_min) / 128
    groups of every sequence, layer and head: 32 groups per layer in the
    one-sequence workload (ring 8,192 -> 4,096), 16 x 2 in the batched one
    (4,352 -> 4,096: the batch its decode steps meet every 256 steps)."""
    L, N = w.n_layers, w.n_seqs
    ctx = 128 + w.tail_max
    cache = synthetic.build(w, ctx=ctx, max_ctx=ctx, seal_to_min=False, seal_if_full=False, chunk=512)
    ring = cache.info(0, 0)[2]
    assert ring == w.tail_max, ring
    rec_bytes = cache.unit_bytes(kvq.REGION_BODY)
    specs = [synthetic.spec_for(w, s) for s in range(N)]
    seqs = list(range(N))
    dev = "cuda"
    # the same tokens again after each timed seal (untimed): reset and refill
    def chunk(l, kind, t0):
        n = min(512, ctx - t0)
        return torch.stack([sp.tokens(l, kind, t0, n, backend="torch", device=dev) for sp in specs]).contiguous()
    ks = [[chunk(l, "k", t0) for t0 in range(0, ctx, 512)] for l in range(L)]
    vs = [[chunk(l, "v", t0) for t0 in range(0, ctx, 512)] for l in range(L)]
    stream = torch.cuda.current_stream()
    times, groups = [], 0
    for rep in range(args.seal_reps + 1):
        if rep > 0:
            for q in seqs:
                cache.reset(q)
            for l in range(L):
                for k, v in zip(ks[l], vs[l]):
                    cache.append(l, seqs, k, v, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g = cache.seal(-1, kvq.SEAL_IF_FULL, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        if rep > 0:            # the first seal is a warm-up
            times.append(a.elapsed_time(b))
            groups = g
    ms = sorted(times)[len(times) // 2]
    tokens = groups * 128 // L          # groups summed over layers; every layer seals the same tokens
    tiles = groups * w.n_kv_heads * 2 * max(1, w.head_dim // 256)
    sub = min(w.head_dim, 256)
    flops = tiles * seal_flops_per_tile(w.passes, 128, sub)
    tflops = flops / (ms * 1e-3) / 1e12
    # bytes: the tq6_0 tiles read, the records written
    hbm = tiles * (128 * (sub // 128) * 98) + groups * w.n_kv_heads * rec_bytes
    log(f"[bench] seal: {groups} groups ({tokens} tokens x {L} layers), {ms * 1e3:.1f} us -> "
        f"{tokens / (ms * 1e-3) / 1e6:.2f} M tokens/s, {tflops:.2f} TFLOP/s (VALU)")
    del cache
    torch.cuda.empty_cache()
    return {"ms": ms, "tokens": tokens, "tokens_per_s": tokens / (ms * 1e-3), "tiles": tiles, "tflops": tflops,
            "hbm_bytes": hbm}


def run_tbq4(args, w, torch, kvq, inputs, sealed_us):
    """The TBQ4 comparator at the same shape: one layer of every sequence held
    whole as TBQ4 blocks (66 bytes per 128 values; no sink, ring or exact
    tail), one fused rotated-domain decode per call, timed with HIP events on
    the current stream over `steps` calls after `warmup`; the encoder is timed
    the same way over the layer's keys.  Bytes per call = the K and V blocks
    of every token (all decoded), partial rows excluded."""
    n, h, hq, d, t = w.n_seqs, w.n_kv_heads, w.n_q_heads, w.head_dim, w.ctx
    if d not in (128, 256):
        log(f"[bench] TBQ4 comparator skipped: head_dim {d}")
        return None
    nb = d // 128
    words = inputs.signs_to_words(inputs.rotation_signs(7))
    dev = "cuda"
    kv = [inputs.normal_t(70 + i, 140, 0, n * h * t * d, dev).to(torch.float16).view(-1, 128) for i in range(2)]
    k4 = kv[0].view(n, h, t, d)
    for hh in range(h):  # 2% outlier key channels x15, as in the workload recipe
        ch = torch.from_numpy(inputs.outlier_channels(70, 0, hh, d, max(1, round(0.02 * d)))).to(dev)
        k4[:, hh, :, ch] *= 15.0
    blocks = [torch.empty((n, h, t, nb, 66), dtype=torch.uint8, device=dev) for _ in range(2)]
    q = inputs.normal_t(72, 141, 0, n * hq * d, dev).to(torch.float16).view(n, hq, d)
    lens = [t] * n
    ws = torch.empty(kvq.tbq4_workspace_bytes(n, hq, h, d, t), dtype=torch.uint8, device=dev)
    out = torch.empty((n, hq, d), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for i in range(2):
        kvq.tbq4_encode(kv[i], words, out=blocks[i])
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(max(1, args.steps // 5)):
        kvq.tbq4_encode(kv[0], words, out=blocks[0])
    ev[1].record()
    for _ in range(args.warmup):
        kvq.tbq4_attn_decode(q, blocks[0], blocks[1], lens, words, 1.0 / d ** 0.5, out=out, workspace=ws)
    ev[2].record()
    for _ in range(args.steps):
        kvq.tbq4_attn_decode(q, blocks[0], blocks[1], lens, words, 1.0 / d ** 0.5, out=out, workspace=ws)
    ev[3].record()
    torch.cuda.synchronize()
    enc_us = ev[0].elapsed_time(ev[1]) * 1e3 / max(1, args.steps // 5)
    dec_us = ev[2].elapsed_time(ev[3]) * 1e3 / args.steps
    nbytes = 2 * n * h * t * nb * 66
    gbs = nbytes / (dec_us * 1e-6) / 1e9
    vals = n * h * t * d
    log(f"[bench] TBQ4 comparator: {nbytes / 1e6:.1f} MB per layer, fused decode {dec_us:.1f} us "
        f"({gbs:.1f} GB/s, {gbs / HBM_PEAK_GBS:.3f} of HBM peak) vs sealed-cache decode kernel {sealed_us:.1f} us; "
        f"encode {vals / (enc_us * 1e-6) / 1e9:.2f} G values/s")
    quality = {}
    for name, bits, fb in (("tbq4", None, 4.125), ("tq5_0", 5, 5.125), ("tq6_0", 6, 6.125)):
        rel = []
        for x in kv:
            if bits is None:
                xh = kvq.tbq4_decode(kvq.tbq4_encode(x, words), words)
            else:
                xh = kvq.tq_decode(kvq.tq_encode(x, bits, words), bits, words)
            xf = x.float()
            rel.append(float(((xh - xf) ** 2).sum() / (xf ** 2).sum()))
            del xh, xf
        quality[name] = {"bits": fb, "rel_sq_err_k": round(rel[0], 6), "rel_sq_err_v": round(rel[1], 6)}
    log("[bench] quality per bit (relative squared error, K with outliers / V): " +
        ", ".join(f"{k} {v['bits']} bits {v['rel_sq_err_k']:.2e} / {v['rel_sq_err_v']:.2e}" for k, v in quality.items()))
    del kv, blocks
    # fp32 FMAs per call: one per value and query head for the scores, one
    # for the outputs (the scan is bound by this vector arithmetic, not HBM)
    flops = 2 * 2 * n * h * t * d * (hq // h)
    tflops = flops / (dec_us * 1e-6) / 1e12
    return {"roofline": {"bound": "alu", "achieved": round(tflops, 2), "peak": FP32_VALU_NONPACKED_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / FP32_VALU_NONPACKED_TFLOPS, 4),
                         "flops_per_call": flops, "time_basis": "whole call (query prologue, scan, merge)"},
            "quality_per_bit": quality, "bytes_per_call": nbytes, "decode_us": round(dec_us, 2), "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "sealed_decode_kernel_us": round(sealed_us, 2),
            "encode_gvalues_per_s": round(vals / (enc_us * 1e-6) / 1e9, 2),
            "note": "whole layer as TBQ4 blocks, fused rotated-domain decode incl. merge"}


def _oracle_unit(args):
    """One oracle unit on one thread: a one-layer, one-KV-head cache of the
    workload's shape built at `ctx` tokens (timed seal), then decode calls
    for `budget_s` seconds.  Returns (decode bytes, decode seconds, calls,
    sealed groups, seal seconds, info)."""
    w, unit, ctx, budget_s = args
    from threadpoolctl import threadpool_limits

    from oracle import cache as ocache
    from oracle import record as orecord
    from quantized_kv_cache_seal_amd import inputs, synthetic

    with threadpool_limits(limits=1):
        oc = ocache.OracleCache(1, 1, w.head_dim, w.group, 1, ctx, w.tail_min, w.tail_max, w.margin,
                                w.k_bits, w.v_bits, w.passes, synthetic.signs(w))
        spec = inputs.KVSpec(1, 1, w.head_dim, w.seed + 101 * unit, w.k_dist, w.outliers, w.outlier_scale)
        t_seal, groups = 0.0, 0
        for t0 in range(0, ctx, 512):
            k = spec.tokens(0, "k", t0, 512)[None]
            v = spec.tokens(0, "v", t0, 512)[None]
            oc.append(0, [0], k, v)
            a = time.perf_counter()
            groups += oc.seal(0, ocache.SEAL_IF_FULL)
            t_seal += time.perf_counter() - a
        a = time.perf_counter()
        groups += oc.seal(0, ocache.SEAL_TO_MIN)
        t_seal += time.perf_counter() - a
        n_tok, n_rec, ring = oc.info(0, 0)
        q = inputs.queries(w.seed, unit, 0, 1, w.group, w.head_dim)[0]
        reps, t_dec = 0, 0.0
        while t_dec < budget_s or reps == 0:
            a = time.perf_counter()
            oc.attention(0, 0, q, 1.0)
            t_dec += time.perf_counter() - a
            reps += 1
    nbytes = (128 * 2 * w.head_dim * 2 + ring * 2 * (w.head_dim // 128) * 98
              + n_rec * orecord.record_bytes(w.head_dim, w.k_bits, w.v_bits))
    return nbytes * reps, t_dec, reps, groups, t_seal, (n_tok, n_rec, ring)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def run_cpu_baseline(w, budget_s):
    """The oracle as it stands (float64 numpy, never tuned for speed) on a
    bounded sample of the same workload: one layer and one KV head of its
    shape at 16,384 tokens (built through append and seal, the seal timed),
    then decode calls for `budget_s` seconds; on one thread, and on every
    available core at once (one process per core, each its own layer/head
    unit: the work is independent per (layer, KV head)).  Rates are the
    sample's compressed bytes per second and its sealed tokens per second
    scaled to the full shape (a sealed token is one group row in every layer
    and KV head)."""
    import concurrent.futures
    import multiprocessing as mp

    ctx = 16_384
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))
    per_layer_head = w.n_layers * w.n_kv_heads
    b, t, reps, groups, t_seal, (n_tok, n_rec, ring) = _oracle_unit((w, 0, ctx, budget_s))
    one = {"gbs": b / t / 1e9, "seal_tok_s": groups * 128 / t_seal / per_layer_head}
    log(f"[bench] cpu oracle, 1 thread: decode {one['gbs']:.4f} GB/s over {n_tok} tokens x 1 head "
        f"({reps} calls, {t:.1f}s); seal {one['seal_tok_s']:.1f} tokens/s ({groups} groups in {t_seal:.1f}s)")
    multi = None
    if cores > 1:
        wall0 = time.perf_counter()
        with concurrent.futures.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as ex:
            outs = list(ex.map(_oracle_unit, [(w, u, ctx, budget_s) for u in range(cores)]))
        wall = time.perf_counter() - wall0
        gbs = sum(o[0] / o[1] for o in outs) / 1e9
        seal = sum(o[3] * 128 / o[4] for o in outs) / per_layer_head
        multi = {"gbs": gbs, "seal_tok_s": seal}
        log(f"[bench] cpu oracle, {cores} processes: decode {gbs:.4f} GB/s, seal {seal:.1f} tokens/s "
            f"(wall {wall:.1f}s)")
    best = multi or one
    return {
        "value": best["gbs"], "unit": "GB/s", "cores": cores if multi else 1, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"float64 decode attention of one layer and one KV head ({w.group} query heads) at "
                  f"{n_tok} tokens ({n_rec} records, ring {ring}), repeated for {budget_s:.0f} s per thread, "
                  f"on {cores} processes at once (independent layer/head units); seal of the same units' "
                  f"groups, scaled to {w.n_layers} layers x {w.n_kv_heads} heads",
        "seal_tokens_per_s": best["seal_tok_s"],
        "one_core": {"value": one["gbs"], "seal_tokens_per_s": one["seal_tok_s"]},
        "all_cores": None if multi is None else {"cores": cores, "value": multi["gbs"],
                                                 "seal_tokens_per_s": multi["seal_tok_s"]},
    }


def seal_entry(seal):
    """Sealed tokens/s of one seal batch, against the non-packed fp32 vector
    peak (packed fp32 instructions are disabled in this build) for the
    balancing and rounding flops, and against HBM for its bytes."""
    return {
        "tokens_per_s": round(seal["tokens_per_s"], 1), "batch_tokens": seal["tokens"],
        "us_per_batch": round(seal["ms"] * 1e3, 2), "tiles": seal["tiles"],
        "roofline": {"bound": "alu", "achieved": round(seal["tflops"], 3), "peak": FP32_VALU_NONPACKED_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(seal["tflops"] / FP32_VALU_NONPACKED_TFLOPS, 4),
                     "flops_basis": "per 128 x 256 tile: passes x 4 x 32,768 (two mat-vecs, y and y^2) "
                                    "+ 6 x 32,768 (rounding)",
                     "hbm_floor_us": round(seal["hbm_bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                     "limited_by": "LDS bandwidth of the matrix-core factor operands and each pass's dependent "
                                   "statistics chain (counters: matrix cores 23 % busy, vector issue 32 % of "
                                   "wave life)"},
    }


def workload_entry(w, dec, seal, args):
    """One extra workload's numbers, for the JSON line."""
    e = {
        "workload": w.name, "layers": w.n_layers, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
        "q_heads": w.n_q_heads, "ctx": w.ctx, "batch": w.n_seqs, "body_bits": f"{w.k_bits}/{w.v_bits}",
        "steps": args.steps, "warmup": args.warmup,
        "us_per_step": round(dec["ms_per_step"] * 1e3, 2), "gbs": round(dec["gbs"], 1),
        "pct_hbm_peak": round(100 * dec["gbs"] / HBM_PEAK_GBS, 2), "bytes_per_step": int(dec["bytes_step"]),
        "main_kernel_us": round(dec["avg_kernel_us"], 2),
        "main_kernel_frac_hbm": round(dec["achieved"] / HBM_PEAK_GBS, 4),
    }
    if seal:
        e["seal"] = seal_entry(seal)
        if w.n_seqs > 1:  # one seal batch every 256 steps
            e["amortized_us_per_step"] = round((dec["ms_per_step"] + seal["ms"] / 256) * 1e3, 2)
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--workload", default="qwen27b", choices=["qwen27b", "gemma31b", "qwen14b1m", "batched"],
                    help="qwen27b (the default, the headline line) or another of the measured shapes")
    ap.add_argument("--calls", action="store_true",
                    help="run each layer's step as kvq_append + kvq_seal + kvq_attn_decode instead of kvq_decode_step")
    ap.add_argument("--seal-reps", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle decode timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-seal", action="store_true")
    ap.add_argument("--no-tbq4", action="store_true", help="skip the TBQ4 comparator leg")
    ap.add_argument("--save-restore", action="store_true",
                    help="also time saving and restoring sequence 0 to and from host memory (kvq_seq_save/_restore)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other measured workloads (512-wide heads, 128-wide K8/V4, the 16-sequence batch)")
    ap.add_argument("--extra-steps", type=int, default=10, help="timed steps of each extra workload")
    ap.add_argument("--no-prefill", action="store_true", help="skip the block-attention leg")
    ap.add_argument("--prefill-steps", type=int, default=5, help="timed steps of each block-attention size")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run the block-attention leg alone (for profiling) and print its numbers")
    ap.add_argument("--no-widths", action="store_true",
                    help="skip the lower body widths (3/3, 3/2, 2/2) at the headline shape")
    ap.add_argument("--prewarm-ms", type=float, default=150.0,
                    help="untimed decode steps for this long before the warm-up steps (the device's power "
                         "management settles after some tens of milliseconds of load); 0 turns it off")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the achievable-HBM-read measurement (kvq_read_probe over 4 GiB)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 20 times (calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the cache shards by sequence or KV head without communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_kv_cache_seal_amd import configs, inputs, kvq, synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 20 copies of {n} bytes")
        return
    kvq.lib()
    w = {"qwen27b": configs.QWEN27B, "gemma31b": configs.GEMMA31B, "qwen14b1m": configs.QWEN14B1M,
         "batched": configs.BATCHED}[args.workload]
    if args.prefill_only:
        print(json.dumps({"workload": w.name, "block_attention":
                          run_prefill(args, w, torch, kvq, synthetic, inputs, (512, 8))}), flush=True)
        return
    dec = run_decode(args, w, torch, kvq, synthetic, inputs, read_first=not args.no_read_ceiling)
    read_ceiling = dec["read_ceiling"]
    seal = None if args.no_seal else run_seal(args, w, torch, kvq, synthetic)
    tbq = None if args.no_tbq4 else run_tbq4(args, w, torch, kvq, inputs, dec["avg_kernel_us"])
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(w, args.cpu_budget)
    extra = {}
    if args.workload == "qwen27b" and not args.no_extra:
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup, sub.seal_reps, sub.save_restore = args.extra_steps, 2, 3, False
        for key, wx in (("gemma31b", configs.GEMMA31B), ("qwen14b1m", configs.QWEN14B1M),
                        ("batched", configs.BATCHED)):
            dx = run_decode(sub, wx, torch, kvq, synthetic, inputs)
            sx = None if args.no_seal else run_seal(sub, wx, torch, kvq, synthetic)
            extra[key] = workload_entry(wx, dx, sx, sub)
    widths = {}
    if args.workload == "qwen27b" and not args.no_widths:
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup, sub.seal_reps, sub.save_restore = args.extra_steps, 2, 3, False
        for kb, vb in ((3, 3), (3, 2), (2, 2)):
            wx = w.scaled(name=f"{w.name}-{kb}{vb}", k_bits=kb, v_bits=vb)
            dx = run_decode(sub, wx, torch, kvq, synthetic, inputs)
            sx = None if args.no_seal else run_seal(sub, wx, torch, kvq, synthetic)
            widths[f"{kb}/{vb}"] = workload_entry(wx, dx, sx, sub)
    prefill = {}
    if args.workload == "qwen27b" and not args.no_prefill:
        prefill = run_prefill(args, w, torch, kvq, synthetic, inputs, (512, 8))
    mfma_body = args.path != "valu"
    traffic = measured_traffic() if (args.workload == "qwen27b" and mfma_body) else None
    if traffic is not None:
        traffic = int(traffic)
    durs = profile_record("duration-record") if (args.workload == "qwen27b" and mfma_body) else None
    res = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "step_us": dec["step_us"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if args.path != "valu" else "f32",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * dec["gbs"] / HBM_PEAK_GBS, 2),
        "config": {
            "workload": w.name, "layers": w.n_layers, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
            "q_heads": w.n_q_heads, "ctx": w.ctx, "batch": w.n_seqs, "body_bits": f"{w.k_bits}/{w.v_bits}",
            "sinkhorn_passes": w.passes, "tail": [w.tail_min, w.tail_max], "decode_path": args.path,
            "step_call": "append+seal+attn_decode" if args.calls else "decode_step",
            "bytes_per_step": int(dec["bytes_step"]),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(dec["achieved"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": ("decode_main_kernel (fused sink, ring and body scan of one layer)" if mfma_body else
                       "decode_valu_kernel (body scan of one layer; sink and ring in decode_ring_kernel)"),
            "bytes_per_launch": int(dec["per_call_bytes"]), "avg_launch_us": round(dec["avg_kernel_us"], 2),
            "time_basis": "device wall clock from the start of workgroup 0 to the end of the last workgroup "
                          "(library stamps, every launch of a second pass of the same number of steps)",
            "traffic_over_algorithmic": None if traffic is None else round(traffic / dec["per_call_bytes"], 4),
            # the same kernel's average duration under rocprofv3 --kernel-trace (committed profile of the
            # current source): it also counts the dispatch ramp before workgroup 0 starts
            "avg_launch_us_rocprof": None if durs is None else float(durs["avg_us"]),
            "frac_rocprof": None if durs is None else
            round(dec["per_call_bytes"] / (float(durs["avg_us"]) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            # context, not the peak: what a plain streaming read achieves on this device (kvq_read_probe)
            "read_ceiling_gbs": None if read_ceiling is None else round(read_ceiling, 1),
            "frac_of_read_ceiling": None if read_ceiling is None else round(dec["achieved"] / read_ceiling, 4),
        },
        "cpu_baseline": cpu,
        "prewarm": {"ms": args.prewarm_ms, "steps": dec["prewarm_steps"],
                    "why": "untimed decode steps before the warm-up steps: the device's power management settles "
                           "only after some tens of milliseconds of this load (steps 11-20 after an idle second "
                           "run ~15 % slower than the steady state)"},
    }
    if dec["save_restore"]:
        res["save_restore"] = dec["save_restore"]
    if seal and w.n_seqs > 1:   # the batched workload meets one seal batch every 256 steps
        res["amortized_ms_per_step"] = round(dec["ms_per_step"] + seal["ms"] / 256, 4)
    if seal:
        res["seal"] = seal_entry(seal)
    if tbq:
        res["tbq4_comparator"] = tbq
    if extra:
        res["workloads"] = extra
    if widths:  # bytes vs time per body width at the headline shape (4/4 is the line itself)
        res["body_widths"] = widths
    if prefill:  # block attention at the headline shape: a 512-token prefill chunk and an 8-token verify block
        res["block_attention"] = prefill
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
