"""tq5_0, the rotated 5-bit comparator block (oracle; test infrastructure only).

SJ-KVaRN section 6 compares against a rotated 5-bit format of 82 bytes per 128
values (5.125 bits) whose quantiser the pages do not print.  Reading, the same
as for the 6-bit staging format with one bit less:
* the block's 128 values are rotated by the 128-point randomized
  Walsh-Hadamard transform (KV cache math), exact and rounded once to fp32;
* symmetric uniform quantiser with 31 levels q in [-15, 15]:
  amax = max |y|, d = fp16(fp32(amax / 15)), inv = fp32(1 / float(d)),
  q = clamp(rne(fp32(y * inv)), -15, 15), u = q + 16 (all 16 when d = 0);
* block = [fp16 d, little-endian][80 bytes: LSB-first bitstream of the 128
  5-bit codes, value k in bits 5k .. 5k + 4];
* decode: y^ = d * (u - 16) (exact in fp32), x^ = R^T y^ (float64).
"""
from __future__ import annotations

import numpy as np

from . import rotation

DIM = 128
BITS = 5
LEVEL = 15
OFFSET = 16
PAYLOAD = DIM * BITS // 8   # 80
BLOCK_BYTES = 2 + PAYLOAD   # 82


def quantize(y32):
    """Rotated fp32 values (..., 128) -> (d fp16 (...), u uint8 (..., 128))."""
    y = np.asarray(y32, np.float32)
    amax = np.abs(y).max(axis=-1)
    d = (amax / np.float32(LEVEL)).astype(np.float32).astype(np.float16)
    df = d.astype(np.float32)
    inv = np.where(df > 0, np.float32(1.0) / np.where(df > 0, df, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    t = (y * inv[..., None]).astype(np.float32)
    u = (np.clip(np.rint(t), -LEVEL, LEVEL) + OFFSET).astype(np.uint8)
    u[df == 0] = OFFSET
    return d, u


def pack(d, u) -> np.ndarray:
    """(n,) fp16 scales and (n, 128) codes -> (n, 82) bytes (plain bit loop)."""
    d = np.asarray(d, np.float16).reshape(-1)
    u = np.asarray(u, np.uint8).reshape(-1, DIM)
    out = np.zeros((u.shape[0], BLOCK_BYTES), np.uint8)
    out[:, :2] = d.view(np.uint8).reshape(-1, 2)
    for k in range(DIM):
        for bit in range(BITS):
            pos = BITS * k + bit
            out[:, 2 + pos // 8] |= ((u[:, k] >> bit) & 1).astype(np.uint8) << (pos % 8)
    return out


def unpack(blocks):
    blocks = np.asarray(blocks, np.uint8).reshape(-1, BLOCK_BYTES)
    d = blocks[:, :2].copy().view(np.float16).reshape(-1)
    u = np.zeros((blocks.shape[0], DIM), np.uint8)
    for k in range(DIM):
        for bit in range(BITS):
            pos = BITS * k + bit
            u[:, k] |= ((blocks[:, 2 + pos // 8] >> (pos % 8)) & 1) << bit
    return d, u


def encode(x16, signs) -> np.ndarray:
    """fp16 (n, 128) original-domain values -> (n, 82) blocks."""
    y = rotation.rotate(np.asarray(x16, np.float16), DIM, signs)
    return pack(*quantize(y))


def decode_rotated(blocks) -> np.ndarray:
    d, u = unpack(blocks)
    return d.astype(np.float32)[:, None] * (u.astype(np.int32) - OFFSET).astype(np.float32)


def decode(blocks, signs) -> np.ndarray:
    """(n, 82) blocks -> float64 (n, 128) in the original domain."""
    return rotation.inverse_exact(decode_rotated(blocks).astype(np.float64), DIM, signs)
