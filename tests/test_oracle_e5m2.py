"""Pins of the oracle's E5M2 table and encoder against what the pages fix.

Sources: wangyu.me "大语言模型量化技术（五）：FP8", section "FP8 是什么" (format table
row E5M2: 1-5-2 bits, largest value 57344, smallest normal 2^-14, smallest
subnormal 2^-16) and section "什么是 FP8 量化" (round to the nearest
representable value, ties to even, saturate); api.makesence.top "LLM推理量化：FP8
versus INT8", section 1 (E5M2 range +-57344) and section 2 (E5M2 KV cache).

Independent checks: E5M2 shares sign, exponent width and bias with IEEE
binary16, so every code is the upper byte of a binary16 value (NumPy's float16
decodes it), and rounding a binary16 bit pattern to its upper byte with
round-half-even on the integer is a correctly rounded conversion; that integer
rule is checked against the oracle's midpoint search for every finite
binary16 value. Brute force (argmin over the grid) covers fp32 inputs.
"""

import math

import numpy as np
import pytest

from conftest import read_golden
from oracle import e5m2, quant


def golden():
    return {k: float(v) for k, v in read_golden("e5m2_format_table.txt")}


def test_format_table_extremes():
    g = golden()
    finite = e5m2.DECODE[np.isfinite(e5m2.DECODE)]
    assert finite.max() == g["max_value"] == 57344.0
    assert -finite.min() == g["max_value"]
    pos = finite[finite > 0]
    assert pos.min() == g["min_subnormal"] == 2.0 ** -16
    assert e5m2.DECODE[0x04] == g["min_normal"] == 2.0 ** -14
    assert e5m2.DECODE[0x7B] == 57344.0
    assert int(g["sign_bits"] + g["exponent_bits"] + g["mantissa_bits"]) == 8


def test_steps_per_interval():
    g = golden()
    grid = e5m2.GRID
    for e in range(-14, 15):
        lo, hi = 2.0 ** e, 2.0 ** (e + 1)
        sel = grid[(grid >= lo) & (grid < hi)]
        assert sel.size == g["steps_per_interval"]
        assert set(np.diff(np.append(sel, hi))) == {lo / g["steps_per_interval"]}


def test_code_structure():
    finite = e5m2.finite_codes()
    assert finite.size == 248
    vals = e5m2.DECODE[finite]
    assert np.unique(vals).size == 247            # +0 and -0 coincide
    assert np.all(np.diff(e5m2.GRID) > 0)
    assert e5m2.DECODE[0x7C] == math.inf and e5m2.DECODE[0xFC] == -math.inf
    for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF):
        assert math.isnan(e5m2.DECODE[c])
    for c in range(0x7C):
        assert e5m2.DECODE[c | 0x80] == -e5m2.DECODE[c]


def test_every_code_is_the_upper_byte_of_binary16():
    codes = np.arange(256, dtype=np.uint16)
    half = (codes << 8).view(np.float16).astype(np.float64)
    ours = e5m2.DECODE
    both_nan = np.isnan(half) & np.isnan(ours)
    assert np.all(both_nan | (half == ours))
    assert np.array_equal(np.isnan(half), np.isnan(ours))


def _rne_upper_byte(bits16):
    """Correctly rounded binary16 -> E5M2 by integer round-half-even on the low
    byte of the magnitude's bit pattern, then saturation at 0x7B."""
    mag = bits16 & 0x7FFF
    q = (mag + 0x7F + ((mag >> 8) & 1)) >> 8
    q = np.minimum(q, 0x7B)
    return (q | ((bits16 >> 8) & 0x80)).astype(np.uint8)


def test_encoder_matches_binary16_rounding_exhaustively():
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals16 = bits.astype(np.uint16).view(np.float16)
    keep = np.isfinite(vals16)
    vals = vals16[keep].astype(np.float32)          # exact widening
    assert np.array_equal(e5m2.encode(vals), _rne_upper_byte(bits[keep]))


def test_encode_decode_roundtrip_all_finite_codes():
    codes = e5m2.finite_codes()
    assert np.array_equal(e5m2.encode(e5m2.DECODE[codes]), codes)


@pytest.mark.parametrize("v,code", [
    (1.125, 0x3C),           # halfway 1.0 / 1.25: mantissa 00 is even
    (1.375, 0x3E),           # halfway 1.25 / 1.5: 1.5 (mantissa 10) is even
    (2.0 ** -17, 0x00),      # halfway 0 / 2^-16: zero is even
    (3 * 2.0 ** -17, 0x02),  # halfway 2^-16 / 2^-15: 2^-15 (m = 2) is even
    (53248.0, 0x7A),         # halfway 49152 / 57344: 49152 (mantissa 10) is even
    (0.875 * 2.0 ** -14, 0x04),  # halfway largest subnormal / smallest normal
])
def test_ties_go_to_even(v, code):
    assert e5m2.encode(np.float32(v)) == code
    assert e5m2.encode(np.float32(-v)) == code | 0x80


@pytest.mark.parametrize("v", [57344.0, 57344.01, 61439.0, 61440.0, 65504.0, 1e30, 3.0e38])
def test_saturation(v):
    assert e5m2.encode(np.float32(v)) == 0x7B
    assert e5m2.encode(np.float32(-v)) == 0xFB


def test_signed_zero_results():
    assert e5m2.encode(np.float32(-0.0)) == 0x80
    assert e5m2.encode(np.float32(-1e-30)) == 0x80
    with pytest.raises(ValueError):
        e5m2.encode(np.float32(np.inf))


def _argmin_encode(values):
    codes = np.arange(0x7C)
    grid = e5m2.DECODE[codes]
    a = np.abs(values.astype(np.float64))[:, None]
    d = np.abs(a - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even_ok = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even_ok.any(axis=1), even_ok.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a[:, 0] >= 57344.0, 0x7B, pick)
    return (pick | (np.signbit(values).astype(np.int64) << 7)).astype(np.uint8)


def test_bruteforce_dense_fp32_sweep():
    rng = np.random.default_rng(8)
    mags = np.exp2(rng.uniform(-20, 16.5, size=200_000)).astype(np.float32)
    pts = np.concatenate([e5m2.MIDPOINTS, e5m2.GRID]).astype(np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    vals = np.concatenate([mags, near]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(e5m2.encode(vals), _argmin_encode(vals))


# ---- the quantizer with E5M2 ------------------------------------------------

def test_scale_is_amax_over_57344_and_amax_maps_to_max_code():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 512)) * np.exp2(rng.integers(-8, 8, size=(16, 1)))).astype(np.float32)
    q, s = quant.quantize_group_1x128(x, fmt="e5m2")
    amax = np.abs(x).reshape(16, 4, 128).max(axis=2)
    assert np.array_equal(s, (amax / np.float32(57344.0)).astype(np.float32))
    # the element that holds the group max encodes as +-57344 (code 0x7B)
    idx = np.abs(x).reshape(16, 4, 128).argmax(axis=2)
    qq = q.reshape(16, 4, 128)
    for r in range(16):
        for g in range(4):
            assert qq[r, g, idx[r, g]] & 0x7F == 0x7B


def test_e5m2_relative_error_bound():
    """Normal-range values come back within half a step: relative error <= 2^-3."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    q, s = quant.quantize_group_1x128(x, fmt="e5m2")
    xh = quant.dequantize_grid(q, s, 1, 128, fmt="e5m2")
    s_full = np.repeat(s, 128, axis=1).astype(np.float64)
    normal = np.abs(x) >= s_full * 2.0 ** -14
    rel = np.abs(xh - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -3 * (1 + 1e-6)


def test_e5m2_is_coarser_than_e4m3_on_the_same_group():
    """Same data: the E5M2 grid has 2 mantissa bits against E4M3's 3, so its
    mean relative error is larger (the pages' range/precision trade-off)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    err = {}
    for fmt in ("e4m3", "e5m2"):
        q, s = quant.quantize_group_1x128(x, fmt=fmt)
        xh = quant.dequantize_grid(q, s, 1, 128, fmt=fmt)
        err[fmt] = np.mean(np.abs(xh - x) / np.maximum(np.abs(x), 1e-3))
    assert err["e5m2"] > 1.5 * err["e4m3"]


def test_e5m2_kv_round_trip():
    rng = np.random.default_rng(12)
    kv = (rng.standard_normal((2, 300, 64)) * 3).astype(np.float32)
    q, s = quant.kv_quantize(kv, 128, fmt="e5m2")
    assert s.shape == (2, 3)
    bits = quant.kv_dequantize(q, s, 128, fmt="e5m2")
    back = quant.bf16_bits_to_f32(bits).astype(np.float64)
    ref = e5m2.decode(q) * np.repeat(s, 128, axis=1)[:, :300, None].astype(np.float64)
    # one fp32 rounding and one bf16 rounding of the exact product
    assert np.all(np.abs(back - ref) <= np.abs(ref) * 2.0 ** -8 * 1.0001)
