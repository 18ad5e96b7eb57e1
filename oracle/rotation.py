"""Rotations of head vectors (oracle; test infrastructure only).

SJ-KVaRN, section 2.2 "Rotation": each 256-value head vector is multiplied by
a 256-point Hadamard matrix, an orthonormal matrix of +1 and -1 entries; the
queries get the same rotation, values are rotated too, and the attention
output is rotated back.  512-wide heads are rotated as two independent
256-point halves.

KV cache math, "rotate first": a randomized Walsh-Hadamard transform on a
128-value block is a sign flip, the transform, and another sign flip.

Readings where the pages are silent:
* ordering: the Sylvester (natural) ordering, H[i, j] = (-1)^popcount(i & j);
* normalisation: orthonormal, i.e. H/16 for 256 points and H/sqrt(128) for
  128 points;
* the two sign vectors of the 128-point transform are one pair per cache,
  shared by every layer and head, and are an input of the cache.

Precision.  Head vectors arrive as fp16.  A signed sum of at most 256 fp16
values is exact in float64 (every partial sum is a multiple of 2^-24 below
2^24 in magnitude, so it needs at most 48 significant bits), hence the
rotation is computed exactly in float64 and then rounded once:
* 256 points: y = fp32( (H x) / 16 )                       (the /16 is exact)
* 128 points: y = fp32( s2 * fl64( (H (s1 * x)) * c128 ) ),  c128 = 1/sqrt(128)
  correctly rounded to float64 (0x1.6a09e667f3bcdp-4)
"""
from __future__ import annotations

import numpy as np

# 1/sqrt(128) correctly rounded: sqrt(2) is correctly rounded and /16 is exact
# (1/sqrt(128) computed directly rounds twice and lands one ulp low).
C128 = np.sqrt(np.float64(2.0)) / np.float64(16.0)


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), int64 entries +-1."""
    h = np.ones((1, 1), np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n
    return h


_H = {}


def _h(n):
    if n not in _H:
        _H[n] = hadamard(n).astype(np.float64)
    return _H[n]


def _check_signs(signs):
    s = np.asarray(signs)
    assert s.shape == (2, 128) and np.all(np.abs(s) == 1)
    return s.astype(np.float64)


def rotate_exact(x, head_dim: int, signs=None) -> np.ndarray:
    """R x in float64, for x of shape (..., head_dim) (fp16 or wider input).

    For fp16 inputs the 256-point result is exact; the 128-point result is the
    exact signed sum times c128, rounded once in float64.
    """
    x = np.asarray(x, np.float64)
    if head_dim == 256:
        return (x @ _h(256)) / 16.0
    if head_dim == 512:
        return np.concatenate([rotate_exact(x[..., :256], 256), rotate_exact(x[..., 256:], 256)], axis=-1)
    if head_dim == 128:
        s = _check_signs(signs)
        return s[1] * (((s[0] * x) @ _h(128)) * C128)
    raise ValueError(head_dim)


def rotate(x16, head_dim: int, signs=None) -> np.ndarray:
    """The staged rotation: R x computed exactly, rounded once to fp32."""
    return rotate_exact(x16, head_dim, signs).astype(np.float32)


def inverse_exact(y, head_dim: int, signs=None) -> np.ndarray:
    """R^T y in float64 (R is orthonormal, so R^T is its inverse)."""
    y = np.asarray(y, np.float64)
    if head_dim == 256:
        return (y @ _h(256)) / 16.0
    if head_dim == 512:
        return np.concatenate([inverse_exact(y[..., :256], 256), inverse_exact(y[..., 256:], 256)], axis=-1)
    if head_dim == 128:
        s = _check_signs(signs)
        return s[0] * (((s[1] * y) @ _h(128)) * C128)
    raise ValueError(head_dim)


def matrix(head_dim: int, signs=None) -> np.ndarray:
    """R as an explicit float64 matrix (rows = output channels)."""
    return rotate_exact(np.eye(head_dim), head_dim, signs).T
