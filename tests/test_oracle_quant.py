"""Pins of the oracle's quantizer and paged layout against things other than itself.

Quantizer rule: "INT8 KV and INT8 MMAC attention on a gfx936 DCU", §2.1.
Byte accounting: same article, §1.1.
"""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import paged, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pad(row, n=256):
    out = np.zeros(n, dtype=np.float32)
    out[: len(row)] = row
    return out


def _fp64_then_round(x):
    """Independent evaluation: IEEE fp32 divisions done in fp64 and rounded once to fp32.

    For a quotient of two fp32 values, fp64 division followed by one rounding to fp32
    equals the correctly rounded fp32 quotient (53 >= 2*24 + 2 bits).
    """
    x = np.asarray(x, np.float32)
    amax = float(np.max(np.abs(x)))
    scale = np.float32(np.float64(amax) / 127.0)
    if scale == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    q = np.array([np.float32(np.float64(v) / np.float64(scale)) for v in x.tolist()],
                 dtype=np.float32)
    return np.clip(np.rint(q), -127, 127).astype(np.int8), scale


def test_golden_tie_cases():
    with open(os.path.join(GOLDEN, "quant_ties.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = _pad(np.array(c["x"], np.float32))
        codes, scale = quant.quantize_rows(x[None])
        assert float(scale[0]) == c["scale"], c["name"]
        exp = np.zeros(256, np.int8)
        exp[: len(c["codes"])] = c["codes"]
        assert np.array_equal(codes[0], exp), c["name"]


def test_matches_fp64_then_round_random_and_near_ties():
    rows = np.concatenate([
        np.random.default_rng(11).standard_normal((64, 256), dtype=np.float32) * np.float32(3.7),
        workloads.near_tie_rows(12, 64),
    ])
    codes, scales = quant.quantize_rows(rows)
    for i in range(rows.shape[0]):
        c2, s2 = _fp64_then_round(rows[i])
        assert scales[i] == s2
        assert np.array_equal(codes[i], c2), i


def test_near_tie_rows_separate_division_from_reciprocal():
    # The near-tie generator must actually exercise the x/scale vs x*(1/scale) choice,
    # otherwise the previous test would not pin the division.
    rows = workloads.near_tie_rows(12, 64)
    codes, scales = quant.quantize_rows(rows)
    recip = np.float32(1.0) / scales
    alt = np.clip(np.rint((rows * recip[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    assert np.count_nonzero(alt != codes) > 0


def test_properties():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 256)) * np.exp(rng.uniform(-20, 20, (200, 1)))).astype(np.float32)
    codes, scales = quant.quantize_rows(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float32
    assert codes.min() >= -127
    amax_idx = np.argmax(np.abs(x), axis=1)
    picked = codes[np.arange(200), amax_idx]
    assert np.all(np.abs(picked) == 127)
    assert np.all(np.sign(picked) == np.sign(x[np.arange(200), amax_idx]))
    err = np.abs(x.astype(np.float64) - quant.dequantize(codes, scales))
    assert np.all(err <= scales[:, None].astype(np.float64) * (0.5 + 2.0 ** -20))


def test_zero_and_underflow_rows_are_all_zero():
    x = np.zeros((3, 256), np.float32)
    x[1, 7] = np.float32(1e-45)          # smallest denormal: amax/127 rounds to 0
    x[2, :] = np.float32(-0.0)
    codes, scales = quant.quantize_rows(x)
    assert np.all(codes == 0) and np.all(scales == 0)


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    f = quant.bf16_bits_to_f32(bits)
    assert f.tolist()[:4] == [1.0, -1.0, 0.0, -0.0]
    assert f[4] == np.float32(3.3895313892515355e38)
    assert workloads.f32_to_bf16_bits(f).tolist() == bits.tolist()


# ---- planted mistakes: each wrong variant must fail at least one pin above ----

def _variant_recip(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127)).astype(np.float32)
    r = np.float32(1) / np.where(s > 0, s, 1).astype(np.float32)
    c = np.clip(np.rint((x * r[..., None]).astype(np.float32)), -127, 127)
    return np.where(s[..., None] > 0, c, 0).astype(np.int8), s


def _variant_half_away(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127)).astype(np.float32)
    q = (x / np.where(s > 0, s, 1)[..., None]).astype(np.float32)
    c = np.clip(np.sign(q) * np.floor(np.abs(q) + 0.5), -127, 127)
    return np.where(s[..., None] > 0, c, 0).astype(np.int8), s


def _variant_scale_128(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(128)).astype(np.float32)
    q = (x / np.where(s > 0, s, 1)[..., None]).astype(np.float32)
    c = np.clip(np.rint(q), -128, 127)
    return np.where(s[..., None] > 0, c, 0).astype(np.int8), s


@pytest.mark.parametrize("variant", [_variant_recip, _variant_half_away, _variant_scale_128])
def test_planted_quantizer_mistakes_are_caught(variant, monkeypatch):
    monkeypatch.setattr(quant, "quantize_rows", variant)
    failures = 0
    for pin in (test_golden_tie_cases, test_matches_fp64_then_round_random_and_near_ties):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0


# ---- paged layout ----

def test_byte_accounting_matches_article():
    with open(os.path.join(GOLDEN, "byte_accounting.json")) as f:
        g = json.load(f)
    H = g["n_kv_heads"]
    cache = paged.alloc_cache(num_pages=3, n_kv_heads=H)
    per_page = sum(a.nbytes for a in cache) / 3
    assert per_page / paged.PAGE == g["int8_total_bytes_per_token"]
    assert sum(a.nbytes for a in cache[:2]) / 3 / paged.PAGE == g["int8_code_bytes_per_token"]
    assert round(100 * g["int8_total_bytes_per_token"] / g["bf16_bytes_per_token"], 2) == g["ratio_percent_printed"]


def test_layout_formulas_are_bijections_on_a_block():
    o, d = np.meshgrid(np.arange(16), np.arange(256), indexing="ij")
    for fn in (paged.k_offset, paged.v_offset):
        offs = fn(2, 1, o, d, 4)
        base = (2 * 4 + 1) * 4096
        assert offs.min() == base and offs.max() == base + 4095
        assert np.unique(offs).size == 4096


def test_layout_16_byte_runs():
    # K: 16 consecutive dims (aligned) of one token are one 16-byte run.
    o = np.arange(16)[:, None]; d = np.arange(256)[None, :]
    k = paged.k_offset(0, 0, o, d, 1)
    assert np.all(np.diff(k.reshape(16, 16, 16), axis=2) == 1)
    # V: the 16 tokens of one dim are one 16-byte run, dims in order.
    v = paged.v_offset(0, 0, o, d, 1)
    assert np.all(np.diff(v, axis=0) == 1) and np.all(v[0] == 16 * np.arange(256))


def test_write_gather_round_trip_with_permuted_pages():
    case = workloads.make_decode_case(21, [37, 16, 1], pages="random", extra_pages=3)
    k, v, _, slots = case.all_data()
    kc, ks = quant.quantize_rows(k)
    vc, vs = quant.quantize_rows(v)
    cache = paged.alloc_cache(case.num_pages, 4, fill_code=5, fill_scale=-1.0)
    paged.write_rows(cache, slots, kc, ks, vc, vs)
    off = 0
    for s, ctx in enumerate(case.context_lens):
        g = paged.gather_seq(cache, case.block_table[s], int(ctx), 4)
        assert np.array_equal(g[0], kc[off:off + ctx]) and np.array_equal(g[1], ks[off:off + ctx])
        assert np.array_equal(g[2], vc[off:off + ctx]) and np.array_equal(g[3], vs[off:off + ctx])
        off += int(ctx)
    # untouched slots keep their fill (3 extra pages + tail of partial pages)
    used = np.zeros(case.num_pages * 16, bool); used[slots] = True
    assert np.count_nonzero(cache[2] == -1.0) == 4 * np.count_nonzero(~used)


def test_negative_slot_skips_row():
    cache = paged.alloc_cache(1, 1)
    kc = np.ones((2, 1, 256), np.int8); s = np.ones((2, 1), np.float32)
    paged.write_rows(cache, np.array([-1, 3]), kc, s, kc, s)
    assert np.count_nonzero(cache[0]) == 256 and cache[2][3] == 1.0 and cache[2][0] == 0.0


def test_bf16_rounding_closed_forms():
    cases = {
        1.0: 0x3F80, -2.5: 0xC020,                        # exactly representable
        1.0 + 2.0 ** -8: 0x3F80,                          # halfway 1 .. 1+2^-7: to even (1)
        1.0 + 3 * 2.0 ** -8: 0x3F82,                      # halfway 1+2^-7 .. 1+2^-6: to even
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,             # just above halfway: up
        3.0e-38: 0x0123,                                  # near the bottom of the normals
    }
    for x, bits in cases.items():
        got = int(quant.f32_to_bf16_rne(np.array([x], np.float32))[0])
        assert got == bits, (x, hex(got), hex(bits))


def test_bf16_rounding_agrees_with_the_bit_trick():
    """The input generators round with an integer-add trick; the two agree on normals."""
    x = np.random.default_rng(13).standard_normal(100000).astype(np.float32) * np.float32(50.0)
    assert np.array_equal(quant.f32_to_bf16_rne(x), workloads.f32_to_bf16_bits(x))
