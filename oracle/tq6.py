"""tq6_0: the rotated 6-bit staging format (oracle; test infrastructure only).

SJ-KVaRN, section 2.1 item 2 "Staging": a new token's key and value are
rotated and written to a ring buffer in a 6.125-bit format, 98 bytes per 128
values.  The "_0" suffix is read as in the block formats the same page lists
(q8_0, q4_0: one scale, no offset; q5_1 carries "a scale and an offset").

Readings (the pages give only the byte count):
* block = [fp16 d, little-endian][96 bytes]; the 96 bytes are an LSB-first
  bitstream of 128 6-bit unsigned codes u_k = q_k + 32 (value k occupies
  stream bits 6k..6k+5; stream bit b is bit b%8 of byte b//8);
* symmetric uniform quantiser with 63 levels q in [-31, 31]:
  amax = max |x|, d = fp16(fp32(amax / 31)), inv = fp32(1 / float(d)),
  q = clamp(rne(fp32(x * inv)), -31, 31); if d == 0 every u is 32;
* decode: d * (u - 32), exact in fp32.
The quantiser arithmetic is IEEE fp32 so that a GPU can take the same
decisions bit for bit.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
BLOCK_BYTES = 98          # 2 + 96
BITS_PER_VALUE = BLOCK_BYTES * 8 / BLOCK   # 6.125


def encode_blocks(x32):
    """x32: float32 (..., 128) rotated values -> (d fp16 (...), u uint8 (..., 128))."""
    x = np.asarray(x32, np.float32)
    assert x.shape[-1] == BLOCK
    amax = np.max(np.abs(x), axis=-1)
    d = (amax / np.float32(31.0)).astype(np.float32).astype(np.float16)
    df = d.astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(df > 0, np.float32(1.0) / np.where(df > 0, df, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    t = (x * inv[..., None]).astype(np.float32)
    q = np.clip(np.rint(t), -31, 31)
    u = (q + 32).astype(np.uint8)
    u[df == 0] = 32
    return d, u


def decode_blocks(d, u) -> np.ndarray:
    """d fp16 (...), u uint8 (..., 128) -> float32 (..., 128) = d * (u - 32)."""
    return (np.asarray(d, np.float16).astype(np.float32)[..., None]
            * (np.asarray(u, np.int32) - 32).astype(np.float32)).astype(np.float32)


def pack6(u) -> bytes:
    """128 six-bit codes -> 96 bytes, LSB-first bitstream (plain bit loop)."""
    u = [int(v) for v in np.asarray(u).reshape(-1)]
    assert len(u) == BLOCK and all(0 <= v < 64 for v in u)
    out = bytearray(96)
    for k, v in enumerate(u):
        for b in range(6):
            if (v >> b) & 1:
                bit = 6 * k + b
                out[bit // 8] |= 1 << (bit % 8)
    return bytes(out)


def unpack6(buf) -> np.ndarray:
    buf = bytes(buf)
    assert len(buf) == 96
    u = np.zeros(BLOCK, np.uint8)
    for k in range(BLOCK):
        v = 0
        for b in range(6):
            bit = 6 * k + b
            v |= ((buf[bit // 8] >> (bit % 8)) & 1) << b
        u[k] = v
    return u


def block_bytes(d, u) -> bytes:
    return np.asarray(d, np.float16).reshape(1).tobytes() + pack6(u)


def parse_block(buf):
    buf = bytes(buf)
    assert len(buf) == BLOCK_BYTES
    d = np.frombuffer(buf[:2], np.float16)[0]
    return d, unpack6(buf[2:])


def encode_vector(x32) -> bytes:
    """One rotated head vector (D values, D a multiple of 128) -> D/128 blocks."""
    x = np.asarray(x32, np.float32).reshape(-1, BLOCK)
    d, u = encode_blocks(x)
    return b"".join(block_bytes(d[i], u[i]) for i in range(x.shape[0]))


def decode_vector(buf) -> np.ndarray:
    buf = bytes(buf)
    n = len(buf) // BLOCK_BYTES
    out = []
    for i in range(n):
        d, u = parse_block(buf[i * BLOCK_BYTES:(i + 1) * BLOCK_BYTES])
        out.append(decode_blocks(d, u))
    return np.concatenate(out).astype(np.float32)
