"""Byte layout of one sealed body record (oracle; test infrastructure only).

SJ-KVaRN, section 2.1 item 4 "Seal" and section 3: keys and values are
compressed in groups of 128 tokens into body records, one per group per KV
head; "4/4" means 4-bit keys and 4-bit values; every scale is fp16 and sits
next to the payload.  The pages count 2,304 bytes of fp16 scales per record
per KV head but do not itemise them.

Layout fixed here (per 128-token group, per KV head, per sub-tile of
``sub`` channels: 256, or 128 for 128-wide heads; a 512-wide head has two
sub-tiles, one per rotation half, stored one after the other):

    [K codes][V codes][K C[sub] S[128] Z[128]][V C[sub] S[128] Z[128]]

* K codes: 128 rows (tokens) x sub channels, row-major; V codes: sub rows
  (channels) x 128 tokens, i.e. channel-major.  Each row is an LSB-first
  bitstream of b-bit codes: element k occupies stream bits b k .. b k + b - 1,
  stream bit i is bit i % 8 of byte i // 8.  At 4 bits this is two codes per
  byte with the even element in the low nibble, at 8 bits one per byte; at 3
  bits eight codes fill three bytes, and codes 2 and 5 of every eight straddle
  a byte boundary (SJ-KVaRN section 2.3: 4/4, 3/3 and 3/2 scalar bodies; KV
  cache math, "a packing bug in the 3-bit codec": the elements that cross a
  byte are where such a packer goes wrong).
* C: per-channel balance scale; S, Z: per-token scale and zero point; all
  fp16, little-endian.
This carries 2,048 bytes of scales per 256-channel record (the pages count
2,304); the difference is recorded as a reading.
"""
from __future__ import annotations

import numpy as np

TOKENS = 128


def sub_width(head_dim: int) -> int:
    return 128 if head_dim == 128 else 256


def n_sub(head_dim: int) -> int:
    return head_dim // sub_width(head_dim)


def sub_bytes(sub: int, k_bits: int, v_bits: int) -> int:
    return TOKENS * sub * k_bits // 8 + sub * TOKENS * v_bits // 8 + 2 * 2 * (sub + 2 * TOKENS)


def record_bytes(head_dim: int, k_bits: int, v_bits: int) -> int:
    return n_sub(head_dim) * sub_bytes(sub_width(head_dim), k_bits, v_bits)


BITS = (2, 3, 4, 8)


def pack_rows(codes, bits: int) -> bytes:
    """Each row an LSB-first bitstream of `bits`-bit codes (a plain bit loop)."""
    c = np.asarray(codes, np.uint8)
    assert bits in BITS and c.ndim == 2 and (c.shape[1] * bits) % 8 == 0
    assert int(c.max(initial=0)) < (1 << bits)
    rows, cols = c.shape
    out = np.zeros((rows, cols * bits // 8), np.uint8)
    for k in range(cols):
        for i in range(bits):
            bit = (c[:, k] >> i) & 1
            pos = bits * k + i
            out[:, pos // 8] |= (bit << (pos % 8)).astype(np.uint8)
    return out.tobytes()


def unpack_rows(buf, rows: int, cols: int, bits: int) -> np.ndarray:
    assert bits in BITS
    b = np.frombuffer(bytes(buf), np.uint8).reshape(rows, cols * bits // 8)
    out = np.zeros((rows, cols), np.uint8)
    for k in range(cols):
        for i in range(bits):
            pos = bits * k + i
            out[:, k] |= ((b[:, pos // 8] >> (pos % 8)) & 1) << i
    return out


def build_sub(k, v, k_bits: int, v_bits: int) -> bytes:
    """k, v: dicts with 'codes' (128 tokens x sub channels), 'C', 'S', 'Z'."""
    parts = [pack_rows(k["codes"], k_bits), pack_rows(np.asarray(v["codes"]).T, v_bits)]
    for side in (k, v):
        parts += [np.asarray(side[n], np.float16).tobytes() for n in ("C", "S", "Z")]
    return b"".join(parts)


def parse_sub(buf, sub: int, k_bits: int, v_bits: int):
    buf = bytes(buf)
    assert len(buf) == sub_bytes(sub, k_bits, v_bits)
    o = 0
    kc = unpack_rows(buf[o:o + TOKENS * sub * k_bits // 8], TOKENS, sub, k_bits)
    o += TOKENS * sub * k_bits // 8
    vc = unpack_rows(buf[o:o + sub * TOKENS * v_bits // 8], sub, TOKENS, v_bits).T.copy()
    o += sub * TOKENS * v_bits // 8
    out = []
    for codes in (kc, vc):
        side = {"codes": codes}
        for n, cnt in (("C", sub), ("S", TOKENS), ("Z", TOKENS)):
            side[n] = np.frombuffer(buf[o:o + 2 * cnt], np.float16).copy()
            o += 2 * cnt
        out.append(side)
    return out[0], out[1]


def parse_record(buf, head_dim: int, k_bits: int, v_bits: int):
    """-> list (one per sub-tile) of (k, v) dicts."""
    sub = sub_width(head_dim)
    sb = sub_bytes(sub, k_bits, v_bits)
    buf = bytes(buf)
    assert len(buf) == n_sub(head_dim) * sb
    return [parse_sub(buf[i * sb:(i + 1) * sb], sub, k_bits, v_bits) for i in range(n_sub(head_dim))]
