"""ctypes binding of libkvq.so (include/kvq.h).  Argument marshalling only:
every step of the path runs in the HIP kernels behind the C ABI.  PyTorch
supplies device memory (the arena, workspace, inputs, outputs) and the stream.

The library must have been built (``python -m quantized_kv_cache_seal_amd.build``
or ``__graft_entry__.build()``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

OK, ERR_INVALID, ERR_CAPACITY, ERR_RING_FULL, ERR_SEALED, ERR_DEVICE, ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
SEAL_IF_FULL, SEAL_TO_MIN = 0, 1
STAGE_TQ6, STAGE_F16 = 0, 1
REGION_SINK, REGION_RING, REGION_BODY = 0, 1, 2
OUT_F32, OUT_F16 = 0, 1
PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2
FLAG_PLAN_ONLY = 1

EXPORTS = [
    "kvq_cache_bytes", "kvq_cache_create", "kvq_cache_destroy", "kvq_append", "kvq_seal",
    "kvq_workspace_bytes", "kvq_attn_decode", "kvq_attn_decode_noalloc", "kvq_prefill_workspace_bytes",
    "kvq_attn_prefill", "kvq_decode_step", "kvq_set_decode_path", "kvq_seq_info", "kvq_seq_reset",
    "kvq_seq_truncate", "kvq_seq_save_bytes", "kvq_seq_save", "kvq_seq_restore", "kvq_export", "kvq_import",
    "kvq_unit_bytes", "kvq_profile_start", "kvq_profile_stop",
    "kvq_tbq4_tables", "kvq_tbq4_encode", "kvq_tbq4_decode", "kvq_tbq4_workspace_bytes", "kvq_tbq4_attn_decode",
    "kvq_tq_encode", "kvq_tq_decode", "kvq_read_probe",
    "kvq_status_string", "kvq_last_error",
]


class KVQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvq status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("max_seqs", ctypes.c_int32), ("tail_min", ctypes.c_int32),
        ("tail_max", ctypes.c_int32), ("margin", ctypes.c_int32), ("max_ctx", ctypes.c_int64),
        ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("sinkhorn_passes", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("rot_signs", ctypes.c_uint64 * 4),
        ("stage_fmt", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m quantized_kv_cache_seal_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER
        sig = {
            "kvq_cache_bytes": [P(Config), P(sz)],
            "kvq_cache_create": [P(Config), vp, sz, P(vp)],
            "kvq_cache_destroy": [vp],
            "kvq_append": [vp, i32, P(i32), i32, vp, vp, i32, vp],
            "kvq_seal": [vp, i32, i32, vp, P(i32)],
            "kvq_workspace_bytes": [vp, i32, P(sz)],
            "kvq_attn_decode": [vp, i32, P(i32), i32, vp, vp, i32, ctypes.c_float, vp, sz, vp],
            "kvq_attn_decode_noalloc": [vp, i32, P(i32), i32, vp, vp, i32, ctypes.c_float, vp],
            "kvq_prefill_workspace_bytes": [vp, i32, i32, P(sz)],
            "kvq_attn_prefill": [vp, i32, P(i32), i32, i32, vp, vp, i32, ctypes.c_float, vp, sz, vp],
            "kvq_decode_step": [vp, i32, P(i32), i32, vp, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp, P(i32)],
            "kvq_set_decode_path": [vp, i32],
            "kvq_seq_info": [vp, i32, i32, P(i64), P(i64), P(i32)],
            "kvq_seq_reset": [vp, i32],
            "kvq_seq_truncate": [vp, i32, i32, i64],
            "kvq_seq_save_bytes": [vp, i32, P(sz)],
            "kvq_seq_save": [vp, i32, vp, sz, vp],
            "kvq_seq_restore": [vp, i32, vp, sz, vp],
            "kvq_export": [vp, i32, i32, i32, i32, i64, vp, sz, vp],
            "kvq_import": [vp, i32, i32, i32, i32, i64, vp, sz, vp],
            "kvq_unit_bytes": [vp, i32, P(sz)],
            "kvq_profile_start": [vp, i32],
            "kvq_profile_stop": [vp, P(ctypes.c_float), P(i32)],
            "kvq_tbq4_tables": [P(ctypes.c_float), P(ctypes.c_float)],
            "kvq_tbq4_encode": [vp, i64, P(ctypes.c_uint64), vp, vp],
            "kvq_tbq4_decode": [vp, i64, P(ctypes.c_uint64), vp, vp],
            "kvq_tbq4_workspace_bytes": [i32, i32, i32, i32, i64, P(sz)],
            "kvq_tq_encode": [vp, i64, i32, P(ctypes.c_uint64), vp, vp],
            "kvq_tq_decode": [vp, i64, i32, P(ctypes.c_uint64), vp, vp],
            "kvq_read_probe": [vp, sz, vp, vp],
            "kvq_tbq4_attn_decode": [vp, vp, vp, i32, i32, i32, i32, i64, P(i64), P(ctypes.c_uint64),
                                     ctypes.c_float, vp, i32, vp, sz, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = i32
        L.kvq_status_string.argtypes = [i32]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def check(status: int) -> int:
    if status != OK:
        raise KVQError(status, lib().kvq_last_error().decode())
    return status


def make_config(n_layers, n_kv_heads, head_dim, n_q_heads, max_seqs, max_ctx, tail_min, tail_max,
                margin=512, k_bits=4, v_bits=4, passes=16, sign_words=(0, 0, 0, 0), flags=0,
                stage=STAGE_TQ6) -> Config:
    c = Config()
    c.stage_fmt = stage
    c.n_layers, c.n_kv_heads, c.head_dim, c.n_q_heads = n_layers, n_kv_heads, head_dim, n_q_heads
    c.max_seqs, c.max_ctx, c.tail_min, c.tail_max, c.margin = max_seqs, max_ctx, tail_min, tail_max, margin
    c.k_bits, c.v_bits, c.sinkhorn_passes, c.flags = k_bits, v_bits, passes, flags
    for i, w in enumerate(sign_words):
        c.rot_signs[i] = w
    return c


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ids(seq_ids):
    arr = (ctypes.c_int32 * len(seq_ids))(*[int(s) for s in seq_ids])
    return arr, len(seq_ids)


class Cache:
    """One cache on the current CUDA (HIP) device, arena owned by a torch tensor."""

    def __init__(self, cfg: Config, device="cuda", plan_only: bool = False):
        import torch
        self.cfg = cfg
        if plan_only:
            cfg.flags |= FLAG_PLAN_ONLY
        n = ctypes.c_size_t()
        check(lib().kvq_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)))
        self.arena_bytes = n.value
        self.arena = None
        if not plan_only:
            self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        check(lib().kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(_ptr(self.arena)), self.arena_bytes,
                                     ctypes.byref(h)))
        self.h = h
        self._ws = None

    def close(self):
        if self.h:
            lib().kvq_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- hot path
    def append(self, layer, seq_ids, k, v, stream=None):
        """k, v: fp16 device tensors [n_seqs][n_tok][H_kv][D] (contiguous)."""
        ids, n = _ids(seq_ids)
        n_tok = 0 if k is None else int(k.shape[1])
        if k is not None:
            assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
        st = _stream(stream) if self.arena is not None else ctypes.c_void_p(0)
        return check(lib().kvq_append(self.h, layer, ids, n, ctypes.c_void_p(_ptr(k)), ctypes.c_void_p(_ptr(v)),
                                      n_tok, st))

    def seal(self, layer=-1, mode=SEAL_IF_FULL, stream=None) -> int:
        g = ctypes.c_int32()
        st = _stream(stream) if self.arena is not None else ctypes.c_void_p(0)
        check(lib().kvq_seal(self.h, layer, mode, st, ctypes.byref(g)))
        return g.value

    def workspace_bytes(self, n_seqs) -> int:
        n = ctypes.c_size_t()
        check(lib().kvq_workspace_bytes(self.h, n_seqs, ctypes.byref(n)))
        return n.value

    def workspace(self, n_seqs):
        import torch
        need = self.workspace_bytes(n_seqs)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.arena.device)
        return self._ws

    def attn_decode(self, layer, seq_ids, q, out=None, scale=1.0, out_f16=False, workspace=None, stream=None):
        """q: fp16 device [n_seqs][H_q][D] -> out fp32 (or fp16) [n_seqs][H_q][D]."""
        import torch
        ids, n = _ids(seq_ids)
        assert q.is_contiguous() and q.dtype == torch.float16
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float16 if out_f16 else torch.float32, device=q.device)
        ws = workspace if workspace is not None else self.workspace(n)
        check(lib().kvq_attn_decode(self.h, layer, ids, n, ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), OUT_F16 if out_f16 else OUT_F32,
                                    float(scale), ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))
        return out

    def attn_decode_noalloc(self, layer, seq_ids, q, out=None, scale=1.0, out_f16=False, stream=None):
        """attn_decode with the split-K partials in the library's per-GPU scratch
        array (kvq_attn_decode_noalloc); out must be given by callers that
        cannot allocate."""
        import torch
        ids, n = _ids(seq_ids)
        assert q.is_contiguous() and q.dtype == torch.float16
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float16 if out_f16 else torch.float32, device=q.device)
        check(lib().kvq_attn_decode_noalloc(self.h, layer, ids, n, ctypes.c_void_p(q.data_ptr()),
                                            ctypes.c_void_p(out.data_ptr()), OUT_F16 if out_f16 else OUT_F32,
                                            float(scale), _stream(stream)))
        return out

    def prefill_workspace_bytes(self, n_seqs, n_q) -> int:
        n = ctypes.c_size_t()
        check(lib().kvq_prefill_workspace_bytes(self.h, n_seqs, n_q, ctypes.byref(n)))
        return n.value

    def attn_prefill(self, layer, seq_ids, q, out=None, scale=1.0, out_f16=False, workspace=None, stream=None):
        """Block attention of the newest n_q tokens of each sequence:
        q fp16 device [n_seqs][n_q][H_q][D] -> out fp32 (or fp16), same shape."""
        import torch
        ids, n = _ids(seq_ids)
        assert q.is_contiguous() and q.dtype == torch.float16 and q.dim() == 4 and q.shape[0] == n
        n_q = q.shape[1]
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float16 if out_f16 else torch.float32, device=q.device)
        if workspace is None:
            need = self.prefill_workspace_bytes(n, n_q)
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.arena.device)
            workspace = self._ws
        check(lib().kvq_attn_prefill(self.h, layer, ids, n, n_q, ctypes.c_void_p(q.data_ptr()),
                                     ctypes.c_void_p(out.data_ptr()), OUT_F16 if out_f16 else OUT_F32, float(scale),
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
        return out

    def decode_step(self, layer, seq_ids, k, v, q, out=None, scale=1.0, out_f16=False, workspace=None,
                    stream=None) -> tuple:
        """Append one token per sequence (k, v: fp16 device [n_seqs][H][D]), seal
        if full, decode q; returns (out, groups sealed)."""
        import torch
        ids, n = _ids(seq_ids)
        for t in (k, v, q):
            assert t.is_contiguous() and t.dtype == torch.float16
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float16 if out_f16 else torch.float32, device=q.device)
        ws = workspace if workspace is not None else self.workspace(n)
        g = ctypes.c_int32()
        check(lib().kvq_decode_step(self.h, layer, ids, n, ctypes.c_void_p(k.data_ptr()),
                                    ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), OUT_F16 if out_f16 else OUT_F32,
                                    float(scale), ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
                                    ctypes.byref(g)))
        return out, g.value

    def profile_start(self, max_calls: int):
        """Record the duration of the main decode kernel of the next max_calls
        attn_decode calls (HIP events on their stream)."""
        self._prof_n = int(max_calls)
        check(lib().kvq_profile_start(self.h, self._prof_n))

    def profile_stop(self):
        """Kernel durations in microseconds of the profiled calls."""
        buf = (ctypes.c_float * self._prof_n)()
        n = ctypes.c_int32()
        check(lib().kvq_profile_stop(self.h, buf, ctypes.byref(n)))
        return list(buf[:n.value])

    def set_decode_path(self, path: int):
        check(lib().kvq_set_decode_path(self.h, path))

    # ---- bookkeeping
    def info(self, seq, layer):
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        check(lib().kvq_seq_info(self.h, seq, layer, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return a.value, b.value, c.value

    def reset(self, seq):
        check(lib().kvq_seq_reset(self.h, seq))

    def truncate(self, seq, layer, n_tok):
        return lib().kvq_seq_truncate(self.h, seq, layer, n_tok)

    def save_bytes(self, seq) -> int:
        n = ctypes.c_size_t()
        check(lib().kvq_seq_save_bytes(self.h, seq, ctypes.byref(n)))
        return n.value

    def save(self, seq, stream=None, out=None):
        """The sequence's saved state as a numpy uint8 array (written into `out`,
        a contiguous uint8 array of save_bytes(seq) bytes, when given)."""
        import numpy as np
        if out is None:
            out = np.empty(self.save_bytes(seq), dtype=np.uint8)
        assert out.dtype == np.uint8 and out.flags["C_CONTIGUOUS"] and out.nbytes == self.save_bytes(seq)
        check(lib().kvq_seq_save(self.h, seq, out.ctypes.data, out.nbytes, _stream(stream)))
        return out

    def restore(self, seq, blob, stream=None) -> int:
        """Restore a saved sequence into slot seq; returns the status (not raised)."""
        import numpy as np
        b = np.ascontiguousarray(np.frombuffer(blob, dtype=np.uint8) if isinstance(blob, (bytes, bytearray)) else blob)
        return lib().kvq_seq_restore(self.h, seq, b.ctypes.data, b.nbytes, _stream(stream))

    def unit_bytes(self, region) -> int:
        n = ctypes.c_size_t()
        check(lib().kvq_unit_bytes(self.h, region, ctypes.byref(n)))
        return n.value

    def export(self, seq, layer, head, region, index, stream=None) -> bytes:
        n = self.unit_bytes(region)
        buf = ctypes.create_string_buffer(n)
        check(lib().kvq_export(self.h, seq, layer, head, region, index, buf, n, _stream(stream)))
        return buf.raw

    def import_(self, seq, layer, head, region, index, data: bytes, stream=None):
        n = self.unit_bytes(region)
        assert len(data) == n
        buf = ctypes.create_string_buffer(bytes(data), n)
        check(lib().kvq_import(self.h, seq, layer, head, region, index, buf, n, _stream(stream)))


def config_for(w, max_ctx=None, max_seqs=None, sign_words=(0, 0, 0, 0), flags=0) -> Config:
    """A Config from a configs.Workload."""
    return make_config(w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads,
                       max_seqs if max_seqs is not None else w.n_seqs,
                       max_ctx if max_ctx is not None else w.ctx, w.tail_min, w.tail_max, w.margin,
                       w.k_bits, w.v_bits, w.passes, sign_words, flags,
                       STAGE_F16 if getattr(w, "stage", "tq6") == "f16" else STAGE_TQ6)


# --- TBQ4 comparator codec ---------------------------------------------------

TBQ4_BLOCK_BYTES = 66


def _words(sign_words):
    w = (ctypes.c_uint64 * 4)(*[int(x) for x in sign_words])
    return w


def tbq4_tables():
    """(centroids[16], boundaries[15]) as float32 numpy arrays (host only)."""
    import numpy as np
    c = (ctypes.c_float * 16)()
    b = (ctypes.c_float * 15)()
    check(lib().kvq_tbq4_tables(c, b))
    return np.array(c, np.float32), np.array(b, np.float32)


def tbq4_encode(x, sign_words, out=None, stream=None):
    """x: fp16 device tensor (..., 128) -> uint8 device tensor (n, 66)."""
    import torch
    assert x.dtype == torch.float16 and x.is_contiguous() and x.shape[-1] == 128
    n = x.numel() // 128
    if out is None:
        out = torch.empty((n, TBQ4_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    assert out.dtype == torch.uint8 and out.is_contiguous() and out.numel() >= n * TBQ4_BLOCK_BYTES
    check(lib().kvq_tbq4_encode(_ptr(x), n, _words(sign_words), _ptr(out), _stream(stream)))
    return out


def tbq4_decode(blocks, sign_words, out=None, stream=None):
    """blocks: uint8 device tensor (n, 66) -> fp32 device tensor (n, 128)."""
    import torch
    assert blocks.dtype == torch.uint8 and blocks.is_contiguous() and blocks.numel() % TBQ4_BLOCK_BYTES == 0
    n = blocks.numel() // TBQ4_BLOCK_BYTES
    if out is None:
        out = torch.empty((n, 128), dtype=torch.float32, device=blocks.device)
    assert out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= n * 128
    check(lib().kvq_tbq4_decode(_ptr(blocks), n, _words(sign_words), _ptr(out), _stream(stream)))
    return out


def tbq4_workspace_bytes(n_seqs, n_q_heads, n_kv_heads, head_dim, max_len) -> int:
    b = ctypes.c_size_t()
    check(lib().kvq_tbq4_workspace_bytes(n_seqs, n_q_heads, n_kv_heads, head_dim, max_len, ctypes.byref(b)))
    return b.value


def tbq4_attn_decode(q, k_blocks, v_blocks, seq_len, sign_words, scale=1.0, out=None, out_f16=False,
                     workspace=None, stream=None):
    """q fp16 (n_seqs, Hq, D); k_blocks/v_blocks uint8 (n_seqs, H, cap, D // 128, 66)."""
    import torch
    n_seqs, hq, d = q.shape
    assert q.dtype == torch.float16 and q.is_contiguous()
    assert k_blocks.shape == v_blocks.shape and k_blocks.dtype == v_blocks.dtype == torch.uint8
    assert k_blocks.is_contiguous() and v_blocks.is_contiguous()
    _, h, cap, nb, bb = k_blocks.shape
    assert k_blocks.shape[0] == n_seqs and nb * 128 == d and bb == TBQ4_BLOCK_BYTES
    lens = (ctypes.c_int64 * n_seqs)(*[int(x) for x in seq_len])
    if workspace is None:
        workspace = torch.empty(max(1, tbq4_workspace_bytes(n_seqs, hq, h, d, max(int(x) for x in seq_len))),
                                dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((n_seqs, hq, d), dtype=torch.float16 if out_f16 else torch.float32, device=q.device)
    check(lib().kvq_tbq4_attn_decode(_ptr(q), _ptr(k_blocks), _ptr(v_blocks), n_seqs, hq, h, d, cap, lens,
                                     _words(sign_words), float(scale), _ptr(out), 1 if out_f16 else 0,
                                     _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def tq_block_bytes(bits: int) -> int:
    return 2 + 16 * bits


def tq_encode(x, bits, sign_words, out=None, stream=None):
    """x: fp16 device tensor (..., 128) -> uint8 device tensor (n, 2 + 16 bits)."""
    import torch
    assert x.dtype == torch.float16 and x.is_contiguous() and x.shape[-1] == 128
    n = x.numel() // 128
    if out is None:
        out = torch.empty((n, tq_block_bytes(bits)), dtype=torch.uint8, device=x.device)
    assert out.dtype == torch.uint8 and out.is_contiguous() and out.numel() >= n * tq_block_bytes(bits)
    check(lib().kvq_tq_encode(_ptr(x), n, bits, _words(sign_words), _ptr(out), _stream(stream)))
    return out


def tq_decode(blocks, bits, sign_words, out=None, stream=None):
    """blocks: uint8 device tensor (n, 2 + 16 bits) -> fp32 device tensor (n, 128)."""
    import torch
    nb = tq_block_bytes(bits)
    assert blocks.dtype == torch.uint8 and blocks.is_contiguous() and blocks.numel() % nb == 0
    n = blocks.numel() // nb
    if out is None:
        out = torch.empty((n, 128), dtype=torch.float32, device=blocks.device)
    assert out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= n * 128
    check(lib().kvq_tq_decode(_ptr(blocks), n, bits, _words(sign_words), _ptr(out), _stream(stream)))
    return out


READ_PROBE_OUT_BYTES = 262144


def read_probe(src, out=None, stream=None):
    """One streaming read of the device tensor src (contiguous, 16-byte
    aligned, a multiple of 16 bytes) by kvq_read_probe; out: uint8 device
    tensor of READ_PROBE_OUT_BYTES receiving the per-wave XOR words."""
    import torch
    assert src.is_cuda and src.is_contiguous()
    if out is None:
        out = torch.empty(READ_PROBE_OUT_BYTES, dtype=torch.uint8, device=src.device)
    assert out.dtype == torch.uint8 and out.numel() >= READ_PROBE_OUT_BYTES
    check(lib().kvq_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(out), _stream(stream)))
    return out
