"""Pins for the oracle's balancing and row rounding (SJ-KVaRN section 2.2
"Balancing" and "Rounding"; section 2.3 "Scalar body").

The closed form: for X_ij = a_i b_j (-1)^(i+j) with b_(2k) = b_(2k+1) > 0, every
row and column of X has mean zero, the first row pass leaves
y_ij = b_j (-1)^(i+j) / rms(b), the first column pass makes every entry +-1,
and every later pass changes nothing; centring gives
C_j = fp16(b_j / geomean(b)) and the codes are 2^b - 1 where X > 0 and 0 where X < 0."""
import numpy as np
import pytest

from oracle import record, rounding, sinkhorn
from quantized_kv_cache_seal_amd import inputs


def _checker(a, b):
    i = np.arange(len(a))[:, None]
    j = np.arange(len(b))[None, :]
    return np.outer(a, b) * np.where((i + j) % 2 == 0, 1.0, -1.0)


def _pairs(seed, cols):
    half = np.exp(inputs.normal_np(seed, 2, 0, cols // 2) * 0.7)
    return np.repeat(half, 2)


@pytest.mark.parametrize("passes", [2, 3, 8, 16])
@pytest.mark.parametrize("cols", [128, 256])
def test_checkerboard_closed_form(passes, cols):
    a = np.exp(inputs.normal_np(1, 1, 0, 128))
    b = _pairs(2, cols)
    x = _checker(a, b)
    bal = sinkhorn.balance(x, passes)
    gm = np.exp(np.mean(np.log(b)))
    assert np.array_equal(bal["C"], (b / gm).astype(np.float16))
    for bits in (2, 3, 4, 8):
        codes, S, Z = rounding.round_rows(x.astype(np.float32), bal["C"], bits)
        assert np.array_equal(codes, np.where(x > 0, 2 ** bits - 1, 0).astype(np.uint8))


def test_single_row_pass_leaves_unit_columns():
    x = _checker(np.exp(inputs.normal_np(1, 1, 0, 128)), _pairs(2, 256))
    assert np.all(sinkhorn.balance(x, 1)["C"] == np.float16(1.0))
    assert np.all(sinkhorn.balance(x, 0)["C"] == np.float16(1.0))


def _tile(seed, cols=256):
    x = inputs.normal_np(seed, 3, 0, 128 * cols).reshape(128, cols)
    x *= np.exp(inputs.normal_np(seed, 4, 0, cols))[None, :]      # uneven columns
    x *= np.exp(0.5 * inputs.normal_np(seed, 5, 0, 128))[:, None]  # uneven rows
    return x.astype(np.float16).astype(np.float32)


def test_final_column_pass_gives_unit_column_spread():
    x = _tile(9).astype(np.float64)
    for passes in (2, 8, 16):
        bal = sinkhorn.balance(x, passes)
        y = x * np.exp(-bal["lr"][:, None] - bal["lc_raw"][None, :])
        assert np.max(np.abs(y.std(axis=0) - 1.0)) < 1e-12
        assert abs(np.mean(bal["lc"])) < 1e-12
    # more passes make the row spreads more even
    y2 = x * np.exp(-sinkhorn.balance(x, 2)["lr"][:, None] - sinkhorn.balance(x, 2)["lc_raw"][None, :])
    b16 = sinkhorn.balance(x, 16)
    y16 = x * np.exp(-b16["lr"][:, None] - b16["lc_raw"][None, :])
    assert np.std(y16.std(axis=1)) < np.std(y2.std(axis=1))


def test_power_of_two_row_scaling_invariance():
    x = _tile(10)
    k = (inputs.uniform_np(10, 6, 0, 128) * 8).astype(int) - 4
    xs = (x * np.exp2(k)[:, None].astype(np.float32)).astype(np.float32)
    c1 = sinkhorn.balance(x.astype(np.float64), 16)["C"]
    c2 = sinkhorn.balance(xs.astype(np.float64), 16)["C"]
    ulps = np.abs(c1.view(np.int16).astype(int) - c2.view(np.int16).astype(int))
    assert ulps.max() <= 1
    # codes are unchanged where the column scales are identical
    if np.array_equal(c1, c2):
        a, _, _ = rounding.round_rows(x, c1, 4)
        b, _, _ = rounding.round_rows(xs, c2, 4)
        assert np.array_equal(a, b)


def test_column_scaling_equivariance():
    x = _tile(11).astype(np.float64)
    c = np.exp(inputs.normal_np(11, 7, 0, 256))
    b1 = sinkhorn.balance(x, 16)
    b2 = sinkhorn.balance(x * c[None, :], 16)
    gm = np.exp(np.mean(np.log(c)))
    assert np.allclose(b2["lc"], b1["lc"] + np.log(c / gm), atol=1e-9)


def test_round_rows_brute_force_nearest_level():
    x = _tile(12)
    C = sinkhorn.balance(x.astype(np.float64), 16)["C"]
    for bits in (2, 3, 4, 8):
        codes, S, Z = rounding.round_rows(x, C, bits)
        t = rounding.pre_round_values(x, C, S, Z).astype(np.float64)
        lv = np.arange(2 ** bits)
        best = np.argmin(np.abs(t[..., None] - lv), axis=-1)
        tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-12
        assert np.array_equal(codes[~tie], best[~tie])
        # bound on the dequantised error: C_j (S_i / 2 + |Z_i - mn_i|), plus fp32 slack
        y = x.astype(np.float64) / C.astype(np.float64)[None, :]
        mn = y.min(axis=1)
        deq = rounding.dequant(codes, C, S, Z)
        bound = C.astype(np.float64)[None, :] * (S.astype(np.float64)[:, None] / 2 * (1 + 1e-5)
                                                 + np.abs(Z.astype(np.float64) - mn)[:, None]
                                                 + 1e-6 * np.abs(y).max(axis=1)[:, None])
        assert np.all(np.abs(deq - x) <= bound)


def test_round_rows_exact_grid():
    # a row already on its grid (values Z + k S, C = 1) comes back with codes k
    S = np.float16(0.25)
    Z = np.float16(-1.5)
    k = (inputs.uniform_np(13, 1, 0, 256) * 16).astype(np.int64)
    k[0], k[1] = 0, 15
    row = (np.float32(Z) + k.astype(np.float32) * np.float32(S)).astype(np.float32)
    codes, S2, Z2 = rounding.round_rows(row[None, :], np.ones(256, np.float16), 4)
    assert S2[0] == S and Z2[0] == Z and np.array_equal(codes[0], k)


def test_constant_row_scale_one():
    x = np.full((128, 256), 3.0, np.float32)
    codes, S, Z = rounding.round_rows(x, np.ones(256, np.float16), 4)
    assert np.all(S == np.float16(1.0)) and np.all(Z == np.float16(3.0)) and np.all(codes == 0)


def test_zero_tile_keeps_unit_scales():
    """An all-zero tile (every token zero, e.g. padding) has zero spread in
    every row and column: nothing is balanced, the log scales stay 0, C = 1,
    and the rounding gives S = 1 (the zero-range rule), Z = 0 and code 0."""
    for cols in (128, 256):
        r = sinkhorn.balance(np.zeros((128, cols)), 16)
        assert np.all(r["lr"] == 0.0) and np.all(r["lc_raw"] == 0.0)
        assert np.all(r["C"] == np.float16(1.0))
        codes, S, Z = rounding.round_rows(np.zeros((128, cols), np.float32), r["C"], 4)
        assert np.all(S == np.float16(1.0)) and np.all(Z == np.float16(0.0)) and np.all(codes == 0)


def test_zero_column_keeps_its_scale():
    """A column that is zero in every row keeps lc = 0 through every pass; the
    other columns are balanced as usual (finite, final column spreads 1)."""
    x = inputs.normal_np(11, 3, 0, 128 * 256).reshape(128, 256)
    x[:, 37] = 0.0
    r = sinkhorn.balance(x, 16)
    assert r["lc_raw"][37] == 0.0
    assert np.all(np.isfinite(r["lc_raw"])) and np.all(np.isfinite(r["C"].astype(np.float64)))
    y = x * np.exp(-r["lr"][:, None] - r["lc_raw"][None, :])
    sd = y.std(axis=0)
    assert abs(sd[37]) == 0.0 and np.allclose(np.delete(sd, 37), 1.0, atol=1e-12)


def test_identical_rows_keep_column_scales():
    """A tile of identical rows (repeated tokens) has constant columns: their
    spread about the first element is exactly zero, so they keep lc = 0 and
    C = 1; the rows (all alike) are balanced."""
    row = inputs.normal_np(12, 3, 0, 256)
    r = sinkhorn.balance(np.tile(row, (128, 1)), 16)
    assert np.all(r["lc_raw"] == 0.0) and np.all(r["C"] == np.float16(1.0))
    assert np.allclose(r["lr"], np.log(row.std()), atol=1e-12)
    # the same rows with one column perturbed by +-2^-10 of its value: a real
    # spread in that column, and the even and odd rows now have slightly
    # different spreads, so after the first row pass every column is a
    # constant plus a small real spread: every column is balanced
    alt = np.where(np.arange(128) % 2 == 0, 1.0, -1.0)
    x = np.tile(row, (128, 1))
    x[:, 10] = row[10] * (1.0 + 2.0 ** -10 * alt)
    lc = sinkhorn.balance(x, 16)["lc_raw"]
    assert np.all(np.isfinite(lc)) and np.all(lc < -5.0)


# ---------------------------------------------------------------------------
# An independent high-precision reference: the same passes in 60-digit decimal
# arithmetic (the spread taken about the mean, no shift), the inputs converted
# exactly from binary64.  At 60 digits a row or column that is constant in
# exact arithmetic comes out with a spread of ~1e-58 of its RMS; 1e-45 tells
# it from zero with a wide margin on both sides.

def _balance_decimal(x, passes):
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 60
        rows, cols = x.shape
        X = [[Decimal(float(v)) for v in r] for r in x]
        lr = [Decimal(0)] * rows
        lc = [Decimal(0)] * cols
        zero = Decimal("1e-45")
        for p in range(passes):
            if p % 2 == 0:
                for i in range(rows):
                    y = [X[i][j] * (-(lr[i] + lc[j])).exp() for j in range(cols)]
                    mean = sum(y) / cols
                    var = sum((v - mean) ** 2 for v in y) / cols
                    ms = sum(v * v for v in y) / cols
                    if var > zero * zero * ms:
                        lr[i] += var.sqrt().ln()
            else:
                for j in range(cols):
                    y = [X[i][j] * (-(lr[i] + lc[j])).exp() for i in range(rows)]
                    mean = sum(y) / rows
                    var = sum((v - mean) ** 2 for v in y) / rows
                    ms = sum(v * v for v in y) / rows
                    if var > zero * zero * ms:
                        lc[j] += var.sqrt().ln()
        m = sum(lc) / cols
        return np.array([float(min(max(v - m, Decimal(-9)), Decimal(9))) for v in lc])


def _small(seed, rows=16, cols=8):
    x = inputs.normal_np(seed, 3, 0, rows * cols).reshape(rows, cols)
    return x * np.exp(inputs.normal_np(seed, 4, 0, cols))[None, :]


@pytest.mark.parametrize("passes", [2, 7, 16])
def test_balance_matches_decimal_reference(passes):
    x = _small(31)
    assert np.max(np.abs(sinkhorn.balance(x, passes)["lc"] - _balance_decimal(x, passes))) < 1e-12


@pytest.mark.parametrize("rel", [1e-3, 1e-5, 1e-8])
def test_near_constant_columns_match_decimal_reference(rel):
    """Every column a constant offset plus a spread of `rel` of it (rows =
    one base row plus rel x noise): the spreads are real and are balanced
    exactly as 60-digit arithmetic balances them."""
    base = 1.0 + np.abs(inputs.normal_np(32, 1, 0, 8))
    x = base[None, :] * (1.0 + rel * inputs.normal_np(32, 2, 0, 16 * 8).reshape(16, 8))
    got = sinkhorn.balance(x, 16)
    want = _balance_decimal(x, 16)
    assert np.max(np.abs(got["lc"] - want)) < 1e-12 / rel
    assert np.max(np.abs(got["lc"])) > 0.1          # the columns were balanced


def test_exactly_constant_columns_keep_scales_like_the_decimal_reference():
    """Rows that are power-of-two multiples of one row: after the first row
    pass every column is constant in exact arithmetic, so its spread is zero
    and its scale is kept (C = 1, as at 60 digits); float64 rounds exp(-lr_i)
    differently per row, leaving a spread of ~1e-16 of the RMS that the
    2^-40 floor reads as zero.  Without the floor the log scales would jump
    by ~ln(1e-16) = -37."""
    row = 1.0 + np.abs(inputs.normal_np(33, 1, 0, 8))
    x = row[None, :] * np.exp2(np.arange(16) % 7 - 3.0)[:, None]
    want = _balance_decimal(x, 16)
    assert np.all(want == 0.0)
    got = sinkhorn.balance(x, 16)
    assert np.all(got["lc"] == 0.0) and np.all(got["C"] == np.float16(1.0))
    old = sinkhorn.ZERO_SPREAD_REL
    try:
        sinkhorn.ZERO_SPREAD_REL = 0.0
        wild = sinkhorn.balance(x, 16)["lc_raw"]
    finally:
        sinkhorn.ZERO_SPREAD_REL = old
    assert np.max(np.abs(wild)) > 20.0


def test_spread_is_taken_about_the_first_element():
    y = 1e8 + np.array([[0.0, 1.0, 2.0, 3.0], [5.0, 5.0, 5.0, 5.0]])
    sigma, rms = sinkhorn.spread(y, 1)
    assert sigma[0] == np.std([0.0, 1.0, 2.0, 3.0]) and sigma[1] == 0.0
    assert np.allclose(rms, 1e8 + np.array([1.5, 5.0]), rtol=1e-15)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("cols", [128, 256])
def test_row_packing_every_position_and_value(bits, cols):
    """Every element position of a row holds every code value in some row;
    the packed bytes, read as numpy's little-endian bit order, give back
    element k in stream bits bits k .. bits k + bits - 1."""
    n = 1 << bits
    c = ((np.arange(n)[:, None] + np.arange(cols)[None, :]) % n).astype(np.uint8)
    buf = record.pack_rows(c, bits)
    assert len(buf) == n * cols * bits // 8
    stream = np.unpackbits(np.frombuffer(buf, np.uint8).reshape(n, -1), axis=1, bitorder="little")
    ref = (stream.reshape(n, cols, bits) * (1 << np.arange(bits))).sum(axis=2)
    assert np.array_equal(ref, c)
    assert np.array_equal(record.unpack_rows(buf, n, cols, bits), c)


def test_three_bit_group_bytes():
    """Eight 3-bit codes in three bytes, written out: codes 2 and 5 straddle
    a byte boundary (the codes a wrong shift corrupts)."""
    for v in range(8 ** 2):
        cc = [(v + 3 * k) % 8 for k in range(8)]
        cc[2], cc[5] = v % 8, (v // 8) % 8
        b = record.pack_rows(np.array([cc], np.uint8), 3)
        want = bytes([cc[0] | cc[1] << 3 | (cc[2] & 3) << 6,
                      cc[2] >> 2 | cc[3] << 1 | cc[4] << 4 | (cc[5] & 1) << 7,
                      cc[5] >> 1 | cc[6] << 2 | cc[7] << 5])
        assert b == want, (cc, b, want)


@pytest.mark.parametrize("kb,vb", [(3, 3), (3, 2), (2, 2), (8, 3)])
def test_low_bit_record_round_trip(kb, vb):
    """A record at 3 and 2 bits: the sizes, and every field back unchanged."""
    assert record.record_bytes(256, kb, vb) == 128 * 256 * (kb + vb) // 8 + 2048
    x = _tile(15)
    sides = []
    for bits in (kb, vb):
        C = sinkhorn.balance(x.astype(np.float64), 8)["C"]
        codes, S, Z = rounding.round_rows(x, C, bits)
        assert int(codes.max()) == 2 ** bits - 1
        sides.append({"codes": codes, "C": C, "S": S, "Z": Z})
    k, v = record.parse_sub(record.build_sub(sides[0], sides[1], kb, vb), 256, kb, vb)
    for a, b in ((k, sides[0]), (v, sides[1])):
        for n in ("codes", "C", "S", "Z"):
            assert np.array_equal(a[n], b[n])


def test_record_sizes_and_round_trip():
    assert record.record_bytes(256, 4, 4) == 34816
    assert record.record_bytes(512, 4, 4) == 2 * 34816
    assert record.record_bytes(128, 8, 4) == 128 * 128 + 128 * 64 + 2 * 2 * (128 + 256)
    x = _tile(14)
    rng = np.random.default_rng(2)
    sides = []
    for bits in (4, 4):
        C = sinkhorn.balance(x.astype(np.float64), 8)["C"]
        codes, S, Z = rounding.round_rows(x, C, bits)
        sides.append({"codes": codes, "C": C, "S": S, "Z": Z})
    buf = record.build_sub(sides[0], sides[1], 4, 4)
    assert len(buf) == 34816
    k, v = record.parse_sub(buf, 256, 4, 4)
    for a, b in ((k, sides[0]), (v, sides[1])):
        for n in ("codes", "C", "S", "Z"):
            assert np.array_equal(a[n], b[n])
    # V codes are stored channel-major: byte b of channel row j holds tokens 2b, 2b+1
    raw = np.frombuffer(buf, np.uint8)
    j, t = 37, 91
    byte = raw[16384 + j * 64 + t // 2]
    assert ((byte >> (4 * (t % 2))) & 15) == sides[1]["codes"][t, j]
