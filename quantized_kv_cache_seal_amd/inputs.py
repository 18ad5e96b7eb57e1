"""Seeded synthetic inputs: the one module that both the HIP path's tests and the
oracle draw from.

It holds none of the method's arithmetic (no rotation, no quantiser, no
attention): only a counter-based random generator and the recipes that shape
its output like the workloads the pages measure (keys with outlier channels,
heavy-tailed keys, Gaussian values and queries).

Generator.  splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the finaliser as published by Vigna) applied
to a counter: ``word(seed, stream, i) = mix(mix(mix(seed) ^ stream) + i)``.
Uniforms take the top 53 bits, ``(w >> 11 + 0.5) / 2**53``, so they lie in
(0, 1).  Normals use the Box-Muller transform in float64 over consecutive
uniform pairs, then round to fp16 with round-to-nearest-even.  Every value is
a pure function of (seed, stream, index), so any slice can be regenerated
alone, on the host (numpy) or on a device (torch int64 arithmetic, which wraps
like uint64 and gives the same words).

The keys have outlier channels (KV cache math: "Keys have outlier channels");
the configurations scale a seeded set of key channels, chosen per (layer, KV
head) by a Fisher-Yates shuffle, in the original (unrotated) domain.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# purposes, folded into the stream id
P_K, P_V, P_Q, P_OUTLIER, P_SIGNS, P_T1, P_T2, P_T3 = range(8)


def mix64(x: int) -> int:
    """splitmix64 step on a Python int (host-side key derivation)."""
    x = (x + _GOLDEN) & MASK64
    x = ((x ^ (x >> 30)) * _M1) & MASK64
    x = ((x ^ (x >> 27)) * _M2) & MASK64
    return x ^ (x >> 31)


def stream_id(purpose: int, layer: int = 0, head: int = 0, extra: int = 0) -> int:
    """Pack the sub-stream coordinates into one 64-bit stream number."""
    return ((purpose & 0xFF) << 56) | ((layer & 0xFFFF) << 40) | ((head & 0xFFFF) << 24) | (extra & 0xFFFFFF)


def stream_key(seed: int, stream: int) -> int:
    return mix64(mix64(seed & MASK64) ^ (stream & MASK64))


# ---------------------------------------------------------------- numpy backend
def _mix_np(x: np.ndarray) -> np.ndarray:
    x = x + np.uint64(_GOLDEN)
    x = (x ^ (x >> np.uint64(30))) * np.uint64(_M1)
    x = (x ^ (x >> np.uint64(27))) * np.uint64(_M2)
    return x ^ (x >> np.uint64(31))


def words_np(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    key = np.uint64(stream_key(seed, stream))
    idx = np.arange(start, start + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix_np(idx + key)


def uniform_np(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    w = words_np(seed, stream, start, n)
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal_np(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    """Standard normals (float64) at indices start..start+n-1 of a stream.

    Normal k uses uniforms 2*(k//2) and 2*(k//2)+1: cos for even k, sin for odd k.
    """
    if n == 0:
        return np.zeros(0, np.float64)
    p0 = start // 2
    p1 = (start + n - 1) // 2 + 1
    u = uniform_np(seed, stream, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log(u[:, 0]))
    th = 2.0 * math.pi * u[:, 1]
    z = np.empty(2 * (p1 - p0), np.float64)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    off = start - 2 * p0
    return z[off:off + n]


# ---------------------------------------------------------------- torch backend
def _i64(c: int) -> int:
    """A uint64 constant as the int64 with the same bits."""
    return c - (1 << 64) if c >= (1 << 63) else c


def _srl_t(x, k):
    import torch
    return (x >> k) & ((1 << (64 - k)) - 1)


def _mix_t(x):
    x = x + _i64(_GOLDEN)
    x = (x ^ _srl_t(x, 30)) * _i64(_M1)
    x = (x ^ _srl_t(x, 27)) * _i64(_M2)
    return x ^ _srl_t(x, 31)


def words_t(seed: int, stream: int, start: int, n: int, device):
    import torch
    key = _i64(stream_key(seed, stream))
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    return _mix_t(idx + key)


def normal_t(seed: int, stream: int, start: int, n: int, device):
    """Same values as normal_np, computed on a torch device (float64)."""
    import torch
    if n == 0:
        return torch.zeros(0, dtype=torch.float64, device=device)
    p0 = start // 2
    p1 = (start + n - 1) // 2 + 1
    w = words_t(seed, stream, 2 * p0, 2 * (p1 - p0), device)
    u = ((_srl_t(w, 11)).to(torch.float64) + 0.5) * (1.0 / 9007199254740992.0)
    u = u.view(-1, 2)
    r = torch.sqrt(-2.0 * torch.log(u[:, 0]))
    th = 2.0 * math.pi * u[:, 1]
    z = torch.stack([r * torch.cos(th), r * torch.sin(th)], dim=1).reshape(-1)
    off = start - 2 * p0
    return z[off:off + n]


# ---------------------------------------------------------------- recipes
def shuffle_pick(seed: int, stream: int, n: int, k: int) -> np.ndarray:
    """The first k entries of a seeded Fisher-Yates shuffle of range(n), sorted."""
    perm = list(range(n))
    u = uniform_np(seed, stream, 0, n)
    for i in range(n - 1, 0, -1):
        j = int(u[n - 1 - i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return np.array(sorted(perm[n - k:]), dtype=np.int64)


def outlier_channels(seed: int, layer: int, head: int, head_dim: int, count: int) -> np.ndarray:
    if count <= 0:
        return np.zeros(0, np.int64)
    return shuffle_pick(seed, stream_id(P_OUTLIER, layer, head), head_dim, count)


def rotation_signs(seed: int, n: int = 128) -> np.ndarray:
    """Two seeded +-1 vectors (the sign flips of a randomized Walsh-Hadamard
    transform), returned as a (2, n) int8 array: row 0 before, row 1 after."""
    w = words_np(seed, stream_id(P_SIGNS), 0, 2 * n)
    bits = (w >> np.uint64(63)).astype(np.int8)
    return (1 - 2 * bits).reshape(2, n)


def signs_to_words(signs: np.ndarray) -> list:
    """Pack a (2, 128) sign array into four uint64 words: bit b of word w is set
    where entry 64*w+b of the flattened array is -1."""
    flat = (signs.reshape(-1) < 0).astype(np.uint64)
    out = []
    for w in range(len(flat) // 64):
        v = 0
        for b in range(64):
            v |= int(flat[64 * w + b]) << b
        out.append(v)
    return out


class KVSpec:
    """Distribution of one cache's synthetic keys and values.

    k_dist: "normal" or "student_t3"; outliers: number of key channels per
    (layer, KV head) multiplied by outlier_scale.
    """

    def __init__(self, n_layers, n_kv_heads, head_dim, seed, k_dist="normal",
                 outliers=0, outlier_scale=1.0):
        self.n_layers, self.n_kv_heads, self.head_dim = n_layers, n_kv_heads, head_dim
        self.seed, self.k_dist = seed, k_dist
        self.outliers, self.outlier_scale = outliers, outlier_scale
        self._scale = {}

    def channel_scale(self, layer: int, head: int) -> np.ndarray:
        key = (layer, head)
        if key not in self._scale:
            s = np.ones(self.head_dim, np.float64)
            s[outlier_channels(self.seed, layer, head, self.head_dim, self.outliers)] = self.outlier_scale
            self._scale[key] = s
        return self._scale[key]

    def _raw(self, purpose, layer, head, t0, n, backend, device):
        D = self.head_dim
        st = stream_id(purpose, layer, head)
        if backend == "numpy":
            return normal_np(self.seed, st, t0 * D, n * D).reshape(n, D)
        return normal_t(self.seed, st, t0 * D, n * D, device).view(n, D)

    def tokens(self, layer: int, kv: str, t0: int, n: int, backend="numpy", device=None):
        """fp16 array [n][H_kv][D] for tokens t0..t0+n-1 of one layer (kv 'k' or 'v')."""
        heads = []
        for h in range(self.n_kv_heads):
            if kv == "v":
                x = self._raw(P_V, layer, h, t0, n, backend, device)
            else:
                x = self._raw(P_K, layer, h, t0, n, backend, device)
                if self.k_dist == "student_t3":
                    c = [self._raw(p, layer, h, t0, n, backend, device) for p in (P_T1, P_T2, P_T3)]
                    chi = (c[0] * c[0] + c[1] * c[1] + c[2] * c[2]) / 3.0
                    x = x / (chi ** 0.5)
                if self.outliers:
                    s = self.channel_scale(layer, h)
                    if backend != "numpy":
                        import torch
                        s = torch.as_tensor(s, device=device)
                    x = x * s
            heads.append(x)
        if backend == "numpy":
            return np.stack(heads, axis=1).astype(np.float16)
        import torch
        return torch.stack(heads, dim=1).to(torch.float16)


def queries(seed: int, step: int, layer: int, n_seqs: int, n_q_heads: int, head_dim: int,
            backend="numpy", device=None):
    """Decode queries q ~ N(0, sigma = 1/sqrt(D)) as fp16 [n_seqs][H_q][D]."""
    n = n_seqs * n_q_heads * head_dim
    st = stream_id(P_Q, layer, 0, step)
    s = 1.0 / math.sqrt(head_dim)
    if backend == "numpy":
        return (normal_np(seed, st, 0, n) * s).astype(np.float16).reshape(n_seqs, n_q_heads, head_dim)
    import torch
    return (normal_t(seed, st, 0, n, device) * s).to(torch.float16).view(n_seqs, n_q_heads, head_dim)


def block_queries(seed: int, step: int, layer: int, n_seqs: int, n_q: int, n_q_heads: int, head_dim: int,
                  backend="numpy", device=None):
    """Queries of a block of n_q tokens per sequence (a prefill chunk or a verify
    block): the decode recipe over n_seqs * n_q rows, as fp16 [n_seqs][n_q][H_q][D]."""
    q = queries(seed, step, layer, n_seqs * n_q, n_q_heads, head_dim, backend, device)
    return q.reshape(n_seqs, n_q, n_q_heads, head_dim)
