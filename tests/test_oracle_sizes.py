"""The size model against every number the pages print (tests/golden)."""
import json
import os

import pytest

from oracle import sizes

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_numbers.json")))
GIB, MIB, KIB = sizes.GIB, sizes.MIB, sizes.KIB


def _printed(key, got):
    e = G[key]
    if "digits" in e:
        assert round(got, e["digits"]) == e["value"], (key, got)
    else:
        assert got == e["value"], (key, got)


def test_sjkvarn_section1():
    per_tok = sizes.kv_bytes_per_token(16, 4, 256, 16)
    _printed("f16_bytes_per_token_qwen27b", per_tok)
    _printed("f16_cache_gb_at_110592", per_tok * 110_592 / GIB)
    _printed("q8_0_cache_gb_at_110592", sizes.kv_bytes_per_token(16, 4, 256, sizes.FORMAT_BITS["q8_0"]) * 110_592 / GIB)


def test_record_scale_overhead():
    _printed("record_scale_bytes", sizes.PAGE_SCALE_BYTES)
    _printed("record_scale_bits_per_value", sizes.body_bits_per_value(4, 4) - 4)
    _printed("body_bits_44", sizes.body_bits_per_value(4, 4))
    assert sizes.page_record_bytes(4, 4) == 35072
    assert sizes.body_bytes_per_token(4, 4, 16, 4) == 17536
    assert sizes.body_bytes_per_token(3, 3, 16, 4) == 13440
    assert sizes.body_bytes_per_token(3, 2, 16, 4) == 11392


def test_allocation_rule():
    def rule(kb, vb, ctx):
        return sizes.allocated_bytes(sizes.body_bytes_per_token(kb, vb, 16, 4), ctx)
    _printed("sj44_allocated_gb_at_110592", rule(4, 4, 110_592) / GIB)
    for (kb, vb), key in (((4, 4), "allocated_bits_44_at_110592"), ((3, 3), "allocated_bits_33_at_110592"),
                          ((3, 2), "allocated_bits_32_at_110592")):
        _printed(key, sizes.allocated_bits(rule(kb, vb, 110_592), 110_592, 16, 4, 256))
    _printed("allocated_bits_44_at_204800", sizes.allocated_bits(rule(4, 4, 204_800), 204_800, 16, 4, 256))
    _printed("allocated_bits_33_at_204800", sizes.allocated_bits(rule(3, 3, 204_800), 204_800, 16, 4, 256))
    _printed("rule_gb_32_at_204800", rule(3, 2, 204_800) / GIB)


def test_format_sizes_section6():
    vpt = sizes.values_per_token(16, 4, 256)
    _printed("q8_0_q5_1_gb_at_110592", sizes.format_bytes("q8_0", 110_592, vpt, "q5_1") / GIB)
    _printed("q8_0_q5_1_bits", (sizes.FORMAT_BITS["q8_0"] + sizes.FORMAT_BITS["q5_1"]) / 2)
    _printed("tq5_0_block_bytes_per_128", sizes.FORMAT_BITS["tq5_0"] * 128 / 8)
    _printed("tbq4_block_bytes_per_128", sizes.FORMAT_BITS["tbq4"] * 128 / 8)


def test_kv_cache_math_worked_example_and_table():
    per_tok = G["tbq4_mib_at_262144"]["value"] * MIB / 262_144
    _printed("tbq4_bytes_per_token", per_tok)
    _printed("tbq4_values_per_token", per_tok / 66 * 128)
    vpt = 32_768
    t = G["kvmath_table"]
    for fmt, row in t["rows"].items():
        assert sizes.FORMAT_BITS[fmt] == row["bits"]
        assert sizes.format_bytes(fmt, 1, vpt) / KIB == row["per_token_kib"]
        for n, mib in zip(t["tokens"], row["sizes_mib"]):
            assert sizes.format_bytes(fmt, n, vpt) / MIB == mib
    p = t["printed_gib"]
    assert round(sizes.format_bytes("q8_0", 32_768, vpt) / GIB, 2) == p["q8_0_32k"]
    assert round(sizes.format_bytes("q8_0", 131_072, vpt) / GIB, 2) == p["q8_0_128k"]
    assert round(sizes.format_bytes("tbq4", 131_072, vpt) / GIB, 2) == p["tbq4_128k"]
    assert round(sizes.format_bytes("turbo3", 131_072, vpt) / GIB, 2) == p["turbo3_128k"]


def test_hal582_size_model():
    f16 = sizes.kv_bytes_per_token(48, 8, 128, 16)
    _printed("hal582_f16_kib_per_token", f16 / KIB)
    assert G["hal582_cells_mib"]["cells"] * f16 / MIB == G["hal582_cells_mib"]["mib"]
    fb = sizes.FORMAT_BITS
    for name, (kib, pct) in G["hal582_kib_per_token"]["rows"].items():
        k, v = name.split("/")
        got = sizes.kv_bytes_per_token(48, 8, 128, fb[k], fb[v]) / KIB
        assert got == kib and round(100 * got / (f16 / KIB), 1) == pct
    _printed("hal582_1m_f16_gib", f16 * 2 ** 20 / GIB)
    q84 = sizes.kv_bytes_per_token(48, 8, 128, fb["q8_0"], fb["q4_0"])
    _printed("hal582_1m_q8k_q4v_gib", q84 * 2 ** 20 / GIB)
    _printed("hal582_sessions_q8k_q4v", f16 / q84)
