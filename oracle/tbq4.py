"""TBQ4 (turbo4-style) block codec, the comparator format (oracle; test
infrastructure only).

KV cache math: the TBQ4 cache rotates each 128-value block with the
randomized Walsh-Hadamard transform (sign flip, transform, sign flip), stores
the block's norm and, per value, a 4-bit index into 16 centroids fitted to the
Gaussian the rotated, normalised values follow; 66 bytes per 128 values
(4.125 bits).  The pages print neither the centroids nor the byte layout.

Readings:
* y = R x (the 128-point rotation of the staging path: exact, rounded once to
  fp32); norm = fp16(sqrt(sum y^2)) with the sum in float64;
* v = fp32(y * fp32(1 / float(norm))) (0 when norm is 0); the 16 centroids are
  the Lloyd-Max quantiser of N(0, 1/128) (each the conditional mean of its
  cell, each cell boundary the midpoint of its centroids), iterated in float64
  to a fixed point; the index is the number of fp32 boundaries strictly below
  v (ties take the lower index);
* block = [fp16 norm, little-endian][64 bytes: index pairs, even value in the
  low nibble];
* decode: y^ = centroid[index] * norm, x^ = R^T y^ (float64).
Pinned by the Lloyd-Max table for the unit Gaussian at 16 levels (Max, 1960):
levels +-0.1284 .. +-2.733, mean squared error 0.009497.
"""
from __future__ import annotations

import math

import numpy as np

from . import rotation

LEVELS = 16
DIM = 128
BLOCK_BYTES = 2 + DIM // 2


def _phi(t):
    return math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _cdf(t):
    return 0.5 * (1.0 + math.erf(t / math.sqrt(2.0)))


def lloyd_gaussian(levels: int = LEVELS, sigma: float = 1.0, tol: float = 1e-15, max_iter: int = 100000):
    """Centroids (ascending, float64) of the Lloyd-Max quantiser of N(0, sigma^2)."""
    half = levels // 2
    c = [sigma * (k + 0.5) * 3.0 / half for k in range(half)]   # positive half; symmetric
    for _ in range(max_iter):
        full = [-x for x in reversed(c)] + c
        b = [-math.inf] + [(full[k] + full[k + 1]) / 2 for k in range(levels - 1)] + [math.inf]
        new = []
        for k in range(half, levels):
            lo, hi = b[k] / sigma, b[k + 1] / sigma
            mass = _cdf(hi) - _cdf(lo)
            new.append(sigma * (_phi(lo) - _phi(hi)) / mass)
        done = max(abs(x - y) for x, y in zip(new, c)) <= tol * sigma
        c = new
        if done:
            break
    return np.array([-x for x in reversed(c)] + c, np.float64)


def mse_gaussian(centroids, sigma: float = 1.0) -> float:
    """Mean squared error of a quantiser with these centroids (nearest-centroid cells) on N(0, sigma^2)."""
    c = np.asarray(centroids, np.float64)
    b = [-math.inf] + [(c[k] + c[k + 1]) / 2 for k in range(len(c) - 1)] + [math.inf]
    tot = 0.0
    for k in range(len(c)):
        lo, hi = b[k] / sigma, b[k + 1] / sigma
        # E[(X - c)^2; lo < X/sigma < hi] for X ~ N(0, sigma^2)
        m0 = _cdf(hi) - _cdf(lo)
        m1 = sigma * (_phi(lo) - _phi(hi))
        t2 = (lo * _phi(lo) if math.isfinite(lo) else 0.0) - (hi * _phi(hi) if math.isfinite(hi) else 0.0)
        m2 = sigma * sigma * (m0 + t2)
        tot += m2 - 2 * c[k] * m1 + c[k] * c[k] * m0
    return tot


def tables():
    """(centroids fp32[16], boundaries fp32[15]) for the rotated, normalised values."""
    c = lloyd_gaussian(LEVELS, 1.0 / math.sqrt(DIM))
    b = (c[:-1] + c[1:]) / 2
    return c.astype(np.float32), b.astype(np.float32)


def encode(x16, signs):
    """x16: fp16 (n, 128) -> (norm fp16 (n,), idx uint8 (n, 128))."""
    y = rotation.rotate(np.asarray(x16, np.float16), DIM, signs).astype(np.float32)
    with np.errstate(over="ignore"):  # a norm past the fp16 range is stored as infinity
        norm = np.sqrt((y.astype(np.float64) ** 2).sum(axis=-1)).astype(np.float16)
    nf = norm.astype(np.float32)
    inv = np.where(nf > 0, np.float32(1.0) / np.where(nf > 0, nf, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    v = (y * inv[:, None]).astype(np.float32)
    _, b = tables()
    idx = (v[..., None] > b).sum(axis=-1).astype(np.uint8)
    return norm, idx


def pack(norm, idx) -> np.ndarray:
    """(n,) fp16 norms and (n, 128) indices -> (n, 66) bytes."""
    n = idx.shape[0]
    out = np.zeros((n, BLOCK_BYTES), np.uint8)
    out[:, :2] = np.asarray(norm, np.float16).view(np.uint8).reshape(n, 2)
    out[:, 2:] = (idx[:, 0::2] & 0xF) | ((idx[:, 1::2] & 0xF) << 4)
    return out


def unpack(blocks):
    blocks = np.asarray(blocks, np.uint8)
    n = blocks.shape[0]
    norm = blocks[:, :2].copy().view(np.float16).reshape(n)
    idx = np.empty((n, DIM), np.uint8)
    idx[:, 0::2] = blocks[:, 2:] & 0xF
    idx[:, 1::2] = blocks[:, 2:] >> 4
    return norm, idx


def decode(blocks, signs) -> np.ndarray:
    """(n, 66) blocks -> float64 (n, 128) in the original domain."""
    norm, idx = unpack(blocks)
    c, _ = tables()
    y = c.astype(np.float64)[idx] * norm.astype(np.float64)[:, None]
    return rotation.inverse_exact(y, DIM, signs)
