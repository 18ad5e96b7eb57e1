"""Per-row rounding of a balanced tile (oracle; test infrastructure only).

SJ-KVaRN, section 2.2 "Rounding": each row is rounded to the target bit width
with its own scale and zero point, and every scale factor is stored as fp16
next to the payload.  Section 2.3 "Scalar body": plain rounding.

Readings:
* a row is one token of the tile; the tile is first divided by its column
  scales: Y'_ij = X_ij * fp32(1 / float(C_j)) (one IEEE fp32 division per
  column, then a multiply);
* asymmetric quantiser with 2^b levels: mn, mx = min, max of the row;
  S = fp16(fp32((mx - mn) / (2^b - 1))), replaced by 1.0 if that is zero;
  Z = fp16(mn); inv = fp32(1 / float(S));
  code = clamp(rne(fp32(fp32(Y' - float(Z)) * inv)), 0, 2^b - 1);
* fp16 conversions saturate at +-65504 instead of overflowing to infinity;
* round to nearest, ties to even.
The arithmetic is IEEE fp32 (no fused multiply-add) so a GPU can take exactly
the same decisions given the same C.
Dequantised value: C_j * (S_i * code_ij + Z_i).
"""
from __future__ import annotations

import numpy as np

F16_MAX = np.float32(65504.0)


def sat_f16(x32) -> np.ndarray:
    return np.clip(np.asarray(x32, np.float32), -F16_MAX, F16_MAX).astype(np.float16)


def col_reciprocal(C16) -> np.ndarray:
    return (np.float32(1.0) / np.asarray(C16, np.float16).astype(np.float32)).astype(np.float32)


def round_rows(x32, C16, bits: int):
    """x32 fp32 (rows, cols), C16 fp16 (cols,) -> (codes uint8 (rows, cols), S fp16 (rows,), Z fp16 (rows,))."""
    x = np.asarray(x32, np.float32)
    y = (x * col_reciprocal(C16)[None, :]).astype(np.float32)
    mn = y.min(axis=1)
    mx = y.max(axis=1)
    levels = np.float32(2 ** bits - 1)
    S = sat_f16(((mx - mn).astype(np.float32) / levels).astype(np.float32))
    S = np.where(S == 0, np.float16(1.0), S).astype(np.float16)
    Z = sat_f16(mn)
    inv = (np.float32(1.0) / S.astype(np.float32)).astype(np.float32)
    t = ((y - Z.astype(np.float32)[:, None]).astype(np.float32) * inv[:, None]).astype(np.float32)
    codes = np.clip(np.rint(t), 0, 2 ** bits - 1).astype(np.uint8)
    return codes, S, Z


def pre_round_values(x32, C16, S16, Z16) -> np.ndarray:
    """The fp32 value t whose rounding gives each code (for boundary counting)."""
    y = (np.asarray(x32, np.float32) * col_reciprocal(C16)[None, :]).astype(np.float32)
    inv = (np.float32(1.0) / np.asarray(S16, np.float16).astype(np.float32)).astype(np.float32)
    return ((y - np.asarray(Z16, np.float16).astype(np.float32)[:, None]).astype(np.float32)
            * inv[:, None]).astype(np.float32)


def dequant(codes, C16, S16, Z16) -> np.ndarray:
    """float64 C_j * (S_i * code_ij + Z_i)."""
    c = np.asarray(codes, np.float64)
    return (np.asarray(C16, np.float64)[None, :]
            * (np.asarray(S16, np.float64)[:, None] * c + np.asarray(Z16, np.float64)[:, None]))
