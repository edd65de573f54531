"""Pins of the oracle's E4M3 table and encoder against what the pages fix.

Sources: wangyu.me "大语言模型量化技术（五）：FP8", section "FP8 是什么" (format table,
grid steps, saturation) and section "什么是 FP8 量化" (round to the nearest
representable value, ties to even, saturate). The brute-force checks use a
different algorithm (argmin over all finite values) from the oracle's
midpoint search.
"""

import math

import numpy as np
import pytest

from conftest import read_golden
from oracle import e4m3


def golden():
    return {k: float(v) for k, v in read_golden("e4m3_format_table.txt")}


def test_format_table_extremes():
    g = golden()
    finite = e4m3.DECODE[np.isfinite(e4m3.DECODE)]
    assert finite.max() == g["max_value"] == 448.0
    assert -finite.min() == g["max_value"]
    pos = finite[finite > 0]
    assert pos.min() == g["min_subnormal"]
    # smallest normal: exponent field 1, mantissa 0
    assert e4m3.DECODE[0x08] == g["min_normal"]
    assert e4m3.DECODE[0x7E] == 448.0
    assert e4m3.DECODE[0x01] == 2.0 ** -9
    # 1 + 4 + 3 bits
    assert int(g["sign_bits"] + g["exponent_bits"] + g["mantissa_bits"]) == 8


def test_steps_per_interval():
    g = golden()
    grid = e4m3.GRID

    def steps_in(lo, hi):
        sel = grid[(grid >= lo) & (grid < hi)]
        return set(np.diff(np.append(sel, hi)))

    assert steps_in(1, 2) == {g["step_in_1_2"]}
    assert steps_in(2, 4) == {g["step_in_2_4"]}
    assert steps_in(16, 32) == {g["step_in_16_32"]}
    # at scale 0.1 the dequantized steps are 0.1 times these
    assert 0.1 * g["step_in_1_2"] == pytest.approx(g["scaled_step_in_1_2_at_scale_0.1"])
    assert 0.1 * g["step_in_2_4"] == pytest.approx(g["scaled_step_in_2_4_at_scale_0.1"])
    assert 0.1 * g["step_in_16_32"] == pytest.approx(g["scaled_step_in_16_32_at_scale_0.1"])


def test_relative_half_step_is_one_sixteenth():
    g = golden()
    grid = e4m3.GRID
    normal = grid[grid >= 2.0 ** -6]
    half_rel = (np.diff(normal) / 2) / normal[:-1]
    assert half_rel.max() == g["relative_error_about"] == 1 / 16


def test_code_structure():
    finite = e4m3.finite_codes()
    assert finite.size == 254
    vals = e4m3.DECODE[finite]
    assert np.unique(vals).size == 253            # +0 and -0 coincide
    assert np.all(np.diff(e4m3.GRID) > 0)          # 0x00..0x7E strictly increasing
    for c in e4m3.NAN_CODES:
        assert math.isnan(e4m3.DECODE[c])
    # sign bit mirrors the value
    for c in range(0x7F):
        assert e4m3.DECODE[c | 0x80] == -e4m3.DECODE[c]


def test_encode_decode_roundtrip_all_finite_codes():
    codes = e4m3.finite_codes()
    back = e4m3.encode(e4m3.DECODE[codes])
    # -0.0 keeps its sign bit, so every finite code comes back unchanged
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("v,code", [
    (1.0625, 0x38),          # halfway 1.0 / 1.125: mantissa 000 is even
    (1.1875, 0x3A),          # halfway 1.125 / 1.25: 1.25 (mantissa 010) is even
    (2.0 ** -10, 0x00),      # halfway 0 / 2^-9: zero is even
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 / 2^-8: 2^-8 (m = 2) is even
    (432.0, 0x7E),           # halfway 416 / 448: 448 (mantissa 110) is even
    (0.9375 * 2.0 ** -6, 0x08),  # halfway largest subnormal / smallest normal
])
def test_ties_go_to_even(v, code):
    assert e4m3.encode(np.float32(v)) == code
    assert e4m3.encode(np.float32(-v)) == code | 0x80


@pytest.mark.parametrize("v", [448.0, 448.0001, 463.9, 464.0, 480.0, 1e30, 3.0e38])
def test_saturation(v):
    assert e4m3.encode(np.float32(v)) == 0x7E
    assert e4m3.encode(np.float32(-v)) == 0xFE


def test_signed_zero_results():
    assert e4m3.encode(np.float32(-0.0)) == 0x80
    assert e4m3.encode(np.float32(0.0)) == 0x00
    assert e4m3.encode(np.float32(-1e-30)) == 0x80
    with pytest.raises(ValueError):
        e4m3.encode(np.float32(np.inf))
    with pytest.raises(ValueError):
        e4m3.encode(np.float32(np.nan))


def _argmin_encode(values):
    """Brute force: nearest of the 254 finite values, ties to an even mantissa,
    magnitude >= 448 saturates, sign copied. Independent of the midpoint table."""
    codes = np.arange(0x7F)
    grid = e4m3.DECODE[codes]
    a = np.abs(values.astype(np.float64))[:, None]
    d = np.abs(a - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among the (at most two) nearest codes prefer an even code
    even_ok = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even_ok.any(axis=1), even_ok.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a[:, 0] >= 448.0, 0x7E, pick)
    return (pick | (np.signbit(values).astype(np.int64) << 7)).astype(np.uint8)


def test_bruteforce_all_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(e4m3.encode(vals), _argmin_encode(vals))


def test_bruteforce_dense_fp32_sweep():
    rng = np.random.default_rng(7)
    # uniform over the magnitude range that matters, plus values on and next to
    # every midpoint and grid point
    mags = np.exp2(rng.uniform(-12, 9.2, size=200_000)).astype(np.float32)
    pts = np.concatenate([e4m3.MIDPOINTS, e4m3.GRID]).astype(np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    vals = np.concatenate([mags, near]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(e4m3.encode(vals), _argmin_encode(vals))
