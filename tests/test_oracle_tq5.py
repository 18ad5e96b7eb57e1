"""Pins of the tq5_0 comparator oracle (SJ-KVaRN section 6: rotated 5-bit, 82 bytes per 128)."""
import json
import pathlib

import numpy as np

from oracle import rotation, tq5
from quantized_kv_cache_seal_amd import inputs

PRINTED = json.loads((pathlib.Path(__file__).parent / "golden" / "printed_numbers.json").read_text())


def _y(seed, n):
    z = inputs.normal_np(seed, 201, 0, n * 128).reshape(n, 128)
    return (z * 2.0 ** (-8 + 12 * inputs.uniform_np(seed, 202, 0, n))[:, None]).astype(np.float32)


def test_block_bytes_match_printed():
    assert tq5.BLOCK_BYTES == PRINTED["tq5_0_block_bytes_per_128"]["value"] == 82


def test_nearest_level_and_error_bound():
    y = _y(1, 300)
    d, u = tq5.quantize(y)
    df = d.astype(np.float64)
    q = u.astype(np.int64) - 16
    # brute force: the code is the nearest of the 31 levels of d * inv-scaled grid
    inv = (np.float32(1) / d.astype(np.float32)).astype(np.float32)
    t = (y * inv[:, None]).astype(np.float32).astype(np.float64)
    lv = np.arange(-15, 16)
    want = lv[np.argmin(np.abs(t[..., None] - lv), axis=-1)]
    assert np.array_equal(q, want)
    assert np.all(np.abs(y - df[:, None] * q) <= df[:, None] * 0.5 * (1 + 1e-3) + 1e-12)
    assert np.all(np.abs(q).max(axis=1) == 15)


def test_requantize_round_trip_and_zero_block():
    y = _y(2, 200)
    b = tq5.pack(*tq5.quantize(y))
    assert np.array_equal(tq5.pack(*tq5.quantize(tq5.decode_rotated(b))), b)
    d, u = tq5.quantize(np.zeros((1, 128), np.float32))
    assert d[0] == 0 and np.all(u == 16)


def test_bitstream_every_position_and_value():
    ks, vs = np.meshgrid(np.arange(128), np.arange(32), indexing="ij")
    ks, vs = ks.reshape(-1), vs.reshape(-1)
    u = np.zeros((ks.size, 128), np.uint8)
    u[np.arange(ks.size), ks] = vs
    blk = tq5.pack(np.full(ks.size, 0.5, np.float16), u)
    bits = np.unpackbits(blk[:, 2:], axis=1, bitorder="little")
    assert np.array_equal(bits.sum(1), [bin(v).count("1") for v in vs])
    got = sum(bits[np.arange(ks.size), 5 * ks + i].astype(np.int64) << i for i in range(5))
    assert np.array_equal(got, vs)
    assert np.array_equal(tq5.unpack(blk)[1], u)


def test_decode_inverts_the_rotation():
    s = inputs.rotation_signs(3)
    x = (inputs.normal_np(4, 203, 0, 64 * 128).reshape(64, 128)).astype(np.float16)
    xh = tq5.decode(tq5.encode(x, s), s)
    y = rotation.rotate_exact(x, 128, s)
    # orthonormal rotation: the error in the original domain equals the rotated one
    d, u = tq5.unpack(tq5.encode(x, s))
    yh = d.astype(np.float64)[:, None] * (u.astype(np.float64) - 16)
    assert np.allclose(((xh - x) ** 2).sum(1), ((yh - y) ** 2).sum(1), rtol=1e-9, atol=1e-12)
    # uniform rounding error: d^2 / 12 per value
    rel = ((xh - x) ** 2).sum() / (x.astype(np.float64) ** 2).sum()
    model = (128 * (d.astype(np.float64) ** 2) / 12).sum() / (x.astype(np.float64) ** 2).sum()
    assert abs(rel / model - 1) < 0.1
