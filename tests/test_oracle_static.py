"""Pins of the oracle's static / delayed scaling (a caller-supplied scale).

Sources: charles2530.github.io "量化：FP8 与混合精度推理", section "scale 是控制面"
(the scale may come from recorded amax history instead of the current batch);
api.makesence.top "LLM推理量化:FP8 versus INT8", section 2 (delayed scaling);
wangyu.me "大语言模型量化技术（五）：FP8", section "什么是 FP8 量化" (divide by the
scale, round to nearest even, saturate).

Independent checks: the scale s = amax / MAX reproduces the dynamic per-tensor
codes; a power-of-two scale makes the division exact, so the codes are the
encoder's codes of x * 2^-k; a scale far below amax / MAX saturates every large
element to the largest code with its sign while small elements keep their
codes; the dequantization error bound of the format for in-range values; the
recorded amax is the largest magnitude; the history scale of closed-form
windows, and of any window equals the dynamic scale of its largest entry.
"""

import numpy as np
import pytest

from oracle import e4m3, e5m2, quant

MAX_CODE = {"e4m3": 0x7E, "e5m2": 0x7B}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_amax_scale_reproduces_dynamic_codes(fmt):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((37, 300)) * 3.7).astype(np.float32)
    qd, sd = quant.quantize_per_tensor(x, fmt)
    qs, amax = quant.quantize_static(x, sd[0], fmt)
    assert np.array_equal(qs, qd)
    assert amax == np.float32(np.abs(x).max())


@pytest.mark.parametrize("fmt,mod", [("e4m3", e4m3), ("e5m2", e5m2)])
def test_power_of_two_scale_is_an_exact_shift(fmt, mod):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 256)) * 50).astype(np.float32)
    for k in (-6, 0, 3):
        q, _ = quant.quantize_static(x, np.float32(2.0 ** k), fmt)
        assert np.array_equal(q, mod.encode(x.astype(np.float64) * 2.0 ** -k))


@pytest.mark.parametrize("fmt,mod", [("e4m3", e4m3), ("e5m2", e5m2)])
def test_small_scale_saturates_with_sign(fmt, mod):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((8, 512)) * 1000).astype(np.float32)
    k = -2 if fmt == "e4m3" else -8
    q, _ = quant.quantize_static(x, np.float32(2.0 ** k), fmt)
    big = np.abs(x) * 2.0 ** -k >= quant.FORMAT_MAX[fmt] * 1.2
    assert big.any() and (~big).any()
    assert np.all(q[big] == (MAX_CODE[fmt] | (np.signbit(x[big]).astype(np.uint8) << 7)))
    assert np.array_equal(q[~big], mod.encode(x[~big].astype(np.float64) * 2.0 ** -k))


@pytest.mark.parametrize("fmt,rel", [("e4m3", 2.0 ** -4), ("e5m2", 2.0 ** -3)])
def test_dequant_error_bound_in_range(fmt, rel):
    rng = np.random.default_rng(4)
    x = rng.standard_normal(20000).astype(np.float32)
    s = np.float32(np.abs(x).max() / quant.FORMAT_MAX[fmt] * 1.5)        # headroom: nothing saturates
    q, _ = quant.quantize_static(x, s, fmt)
    xh = quant.fmt_module(fmt).decode(q) * np.float64(s)
    smallest_normal = {"e4m3": 2.0 ** -6, "e5m2": 2.0 ** -14}[fmt]
    normal = np.abs(x) / np.float64(s) >= smallest_normal
    assert np.all(np.abs(xh - x)[normal] <= rel * np.abs(x)[normal] * (1 + 1e-12))


def test_recorded_amax_and_empty_tensor():
    x = np.array([[1.5, -7.25, 0.0], [3.0, -0.0, 7.0]], np.float32)
    _, amax = quant.quantize_static(x, np.float32(1.0))
    assert amax == np.float32(7.25)
    q, amax = quant.quantize_static(np.zeros((0, 4), np.float32), np.float32(1.0))
    assert q.shape == (0, 4) and amax == 0


def test_zero_scale_gives_signed_zeros():
    x = np.array([[1.0, -2.0, 0.0, -0.0]], np.float32)
    q, _ = quant.quantize_static(x, np.float32(0.0))
    assert list(q[0]) == [0x00, 0x80, 0x00, 0x80]


@pytest.mark.parametrize("fmt,window,expect", [("e4m3", [448.0, 100.0, 3.0], 1.0), ("e4m3", [0.0], 0.0),
                                               ("e4m3", [1.0, 896.0], 2.0), ("e5m2", [57344.0, 1.0], 1.0),
                                               ("e5m2", [7168.0], 0.125)])
def test_history_scale_closed_forms(fmt, window, expect):
    assert quant.scale_from_history(np.array(window, np.float32), fmt) == np.float32(expect)


def test_history_scale_is_the_dynamic_scale_of_the_window_max():
    rng = np.random.default_rng(5)
    for n in (1, 5, 1024):
        h = np.abs(rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, size=n))).astype(np.float32)
        i = int(np.argmax(h))
        x = np.zeros((1, 3), np.float32)
        x[0, 1] = -h[i]
        for fmt in ("e4m3", "e5m2"):
            assert quant.scale_from_history(h, fmt) == quant.quantize_per_tensor(x, fmt)[1][0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_overflowing_quotient_saturates(fmt):
    """x / s beyond the largest fp32 number is still beyond the format's range."""
    x = np.array([[3.0e38, -3.0e38, 1.0, -1e-30]], np.float32)
    q, _ = quant.quantize_static(x, np.float32(2.0 ** -10), fmt)
    m = MAX_CODE[fmt]
    assert list(q[0][:3]) == [m, m | 0x80, quant.fmt_module(fmt).encode(np.array([1024.0]))[0]]
