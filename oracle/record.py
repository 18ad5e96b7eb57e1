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

* K codes: 128 rows (tokens) x sub channels, row-major; 4-bit codes pack two
  per byte, the even channel in the low nibble; 8-bit codes one per byte.
* V codes: sub rows (channels) x 128 tokens, i.e. channel-major; 4-bit codes
  pack two tokens per byte, the even token in the low nibble.
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


def pack_rows(codes, bits: int) -> bytes:
    """Row-major packing; 4-bit: element 2b in the low nibble of byte b."""
    c = np.asarray(codes, np.uint8)
    if bits == 8:
        return c.tobytes()
    assert bits == 4 and c.shape[-1] % 2 == 0 and int(c.max(initial=0)) < 16
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8).tobytes()


def unpack_rows(buf, rows: int, cols: int, bits: int) -> np.ndarray:
    b = np.frombuffer(bytes(buf), np.uint8)
    if bits == 8:
        return b.reshape(rows, cols).copy()
    b = b.reshape(rows, cols // 2)
    out = np.empty((rows, cols), np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
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
