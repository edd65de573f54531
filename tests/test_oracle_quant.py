"""Pins of the oracle's quantizer and KV dequantizer.

Sources: wangyu.me "大语言模型量化技术（五）：FP8": section "什么是 FP8 量化" (scale
max|x|/448, divide, round, saturate, keep codes and scale), section "FP8 与 INT8
量化精度对比" (the worked outlier example), section "权重量化：128×128 分块 FP8"
(block amax, s = a/448, per-element division, fp32 scales, ceil-sized grid).
charles2530.github.io "量化：FP8 与混合精度推理", section "E4M3 和 E5M2 是范围与格点的取舍"
(dequantization multiplies the code by s). pwwt.cn Llama-3 FP8 notes, sections
1 and 3 (K and V get separate scales; per-head, per-128-token KV blocks).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import e4m3, quant


def golden():
    return {r[0]: (float(r[1]), float(r[2])) for r in read_golden("worked_outlier_example.txt")}


# ----------------------------------------------------------------------------
# the page's worked example
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("bf16_inputs", [False, True])
def test_worked_outlier_example(bf16_inputs):
    g = golden()
    rng = np.random.default_rng(3)
    body = rng.uniform(-0.1, 0.1, size=125).astype(np.float32)
    x = np.concatenate([[g["outlier"][0], g["x1"][0], g["x2"][0]], body]).astype(np.float32)
    if bf16_inputs:
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    q, s = quant.quantize_per_tensor(x)
    s = float(s[0])
    assert s == pytest.approx(g["scale"][0], abs=g["scale"][1])
    assert s == float(np.float32(10) / np.float32(448))
    for key in ("x1", "x2"):
        i = 1 if key == "x1" else 2
        xi = float(x[i])
        assert xi / s == pytest.approx(g[key + "_over_s"][0], abs=g[key + "_over_s"][1])
        v = e4m3.DECODE[q[i]]
        assert v == g[key + "_quantized"][0]
        # the step of the interval the quotient lies in
        lo = e4m3.GRID[e4m3.GRID <= v].max()
        hi = e4m3.GRID[e4m3.GRID > v].min()
        assert hi - lo == g[key + "_step"][0]
        if not bf16_inputs:
            assert abs(v * s - xi) == pytest.approx(g[key + "_error"][0], abs=g[key + "_error"][1])
    # the outlier itself lands on the largest code
    assert q[0] == 0x7E
    # more than 100 distinct levels within [-0.1, 0.1] at this scale
    vals = np.unique(e4m3.DECODE[e4m3.finite_codes()])
    levels = vals[np.abs(vals * s) <= 0.1]
    assert levels.size > g["levels_in_pm_0.1_more_than"][0]
    assert levels.size == 145


# ----------------------------------------------------------------------------
# correctly rounded fp32 quotient, pinned with exact rational arithmetic
# ----------------------------------------------------------------------------

def _round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Nearest fp32 to an exact rational, ties to even (normal range)."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_scale_is_amax_over_448():
    # s is the fp32 nearest to the exact amax / 448 (normal and subnormal s)
    for amax in [10.0, 1.0, 448.0, 3.3e38, 2.0 ** -133, 0.0234375, 1e-40]:
        x = np.array([amax, -amax / 3, 0.0], dtype=np.float32)
        _, s = quant.quantize_per_tensor(x)
        exact = Fraction(float(np.float32(amax))) / 448
        assert s[0] == _round_fraction_to_f32(exact)


def test_cast_uses_correctly_rounded_fp32_quotient():
    rng = np.random.default_rng(11)
    # scales with many significant bits and inputs placed next to quotient midpoints
    xs, ss = [], []
    for _ in range(400):
        s = np.float32(rng.uniform(1e-3, 1.0))
        m = rng.choice(e4m3.MIDPOINTS[8:])
        for k in (-2, -1, 0, 1, 2):
            x = np.float32(float(m) * float(s))
            for _ in range(abs(k)):
                x = np.nextafter(x, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
            xs.append(x)
            ss.append(s)
    xs = np.array(xs, dtype=np.float32)
    ss = np.array(ss, dtype=np.float32)
    got = quant.cast(xs, ss)
    ref = np.array([e4m3.encode(_round_fraction_to_f32(Fraction(float(x)) / Fraction(float(s))))
                    for x, s in zip(xs, ss)], dtype=np.uint8)
    assert np.array_equal(got, ref)
    # the reciprocal shortcut would differ somewhere in this set
    approx = e4m3.encode(xs * (np.float32(1) / ss))
    assert not np.array_equal(approx, ref)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def _random_groups(seed, n=64):
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-20, 20, size=(n, 1))).astype(np.float32)
    x = (rng.standard_normal((n, 128)).astype(np.float32) * mags)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def test_amax_element_maps_to_448():
    x = _random_groups(1)
    q, s = quant.quantize_group_1x128(x)
    idx = np.abs(x).argmax(axis=1)
    top = q[np.arange(x.shape[0]), idx]
    assert np.all((top & 0x7F) == 0x7E)


def test_relative_error_bound():
    x = _random_groups(2)
    q, s = quant.quantize_group_1x128(x)
    quot = x / s.astype(np.float32)
    dec = e4m3.decode(q)
    err = np.abs(quot.astype(np.float64) - dec)
    a = np.abs(quot.astype(np.float64))
    normal = a >= 2.0 ** -6
    assert np.all(err[normal] <= a[normal] / 16)
    assert np.all(err[~normal] <= 2.0 ** -10)


def test_sign_symmetry():
    x = _random_groups(3)
    q, s = quant.quantize_group_1x128(x)
    qn, sn = quant.quantize_group_1x128(-x)
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ 0x80)


@pytest.mark.parametrize("k", [-7, -1, 1, 5])
def test_power_of_two_scale_equivariance(k):
    x = _random_groups(4)
    x = x[(np.abs(x).max(axis=1) > 2.0 ** -100) & (np.abs(x).max(axis=1) < 2.0 ** 100)]
    q, s = quant.quantize_group_1x128(x)
    q2, s2 = quant.quantize_group_1x128(x * np.float32(2.0 ** k))
    assert np.array_equal(q, q2)
    assert np.array_equal(s2, s * np.float32(2.0 ** k))


def test_requantizing_the_dequantized_group_keeps_codes():
    x = _random_groups(5)
    q, s = quant.quantize_group_1x128(x)
    back = quant.bf16_bits_to_f32(quant.f32_to_bf16_bits(
        (e4m3.decode(q) * np.repeat(s, 128, axis=1).astype(np.float64)).astype(np.float32)))
    q2, _ = quant.quantize_group_1x128(back)
    assert np.array_equal(q, q2)


def test_zero_group():
    x = np.zeros((2, 256), dtype=np.float32)
    x[0, :128] = -0.0
    x[1, 128:] = 1.5
    q, s = quant.quantize_group_1x128(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(q[0, :128] == 0x80) and np.all(q[0, 128:] == 0x00)
    assert np.all(q[1, :128] == 0x00) and np.all(q[1, 128:] == 0x7E)


# ----------------------------------------------------------------------------
# group shapes: each granularity equals per-tensor quantization of every group
# taken on its own (brute-force loop, small sizes, ragged tails)
# ----------------------------------------------------------------------------

def _bf16_normal(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) * np.exp2(rng.uniform(-3, 3, size=shape[:1] + (1,) * (len(shape) - 1))).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def test_group_1x128_is_per_tensor_per_group():
    x = _bf16_normal((5, 300), 6)
    q, s = quant.quantize_group_1x128(x)
    assert s.shape == (5, 3)
    for r in range(5):
        for j in range(3):
            qq, ss = quant.quantize_per_tensor(x[r, 128 * j:128 * (j + 1)])
            assert np.array_equal(q[r, 128 * j:128 * (j + 1)], qq)
            assert s[r, j] == ss[0]


def test_block_128x128_is_per_tensor_per_block():
    x = _bf16_normal((300, 200), 7)
    q, s = quant.quantize_block_128x128(x)
    assert s.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            blk = x[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            qq, ss = quant.quantize_per_tensor(blk)
            assert np.array_equal(q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)], qq)
            assert s[i, j] == ss[0]


def test_kv_is_per_tensor_per_head_token_block():
    kv = _bf16_normal((3, 300, 64), 8)
    q, s = quant.kv_quantize(kv, 128)
    assert s.shape == (3, 3)
    for h in range(3):
        for b in range(3):
            blk = kv[h, 128 * b:128 * (b + 1)]
            qq, ss = quant.quantize_per_tensor(blk)
            assert np.array_equal(q[h, 128 * b:128 * (b + 1)], qq)
            assert s[h, b] == ss[0]


def test_special_case_reductions():
    x = _bf16_normal((1, 128), 9)
    qa, sa = quant.quantize_per_tensor(x)
    qb, sb = quant.quantize_group_1x128(x)
    assert np.array_equal(qa, qb) and sa[0] == sb[0, 0]
    kv = _bf16_normal((2, 256, 128), 10)
    qk, sk = quant.kv_quantize(kv, 128)
    qw, sw = quant.quantize_block_128x128(kv.reshape(512, 128))
    assert np.array_equal(qk.reshape(512, 128), qw)
    assert np.array_equal(sk.reshape(-1), sw.reshape(-1))


# ----------------------------------------------------------------------------
# dequantizer and bf16 rounding
# ----------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-60, 60, 100_000))).astype(np.float32)
    # exact halfway cases: low 16 bits == 0x8000, both parities of the kept bits
    hi = rng.integers(0x0080, 0x7F00, 4000, dtype=np.uint32)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = quant.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_kv_dequantize_round_trip():
    kv = _bf16_normal((2, 384, 128), 13)
    q, s = quant.kv_quantize(kv, 128)
    out = quant.bf16_bits_to_f32(quant.kv_dequantize(q, s, 128)).astype(np.float64)
    s_full = np.repeat(s, 128, axis=1)[:, :, None].astype(np.float64)
    dec = e4m3.decode(q)
    # exact product decode * s, then one fp32 and one bf16 rounding
    prod = dec * s_full
    assert np.all(np.abs(out - prod) <= np.abs(prod) * (2.0 ** -8 + 2.0 ** -23))
    # reconstruction error: at most half an E4M3 step (relative 1/16 in the
    # normal range, 2^-10 * s below it) plus the two roundings
    x = kv.astype(np.float64)
    bound = np.maximum(np.abs(x) / 16, 2.0 ** -10 * s_full) * (1 + 2.0 ** -8) + np.abs(prod) * 2.0 ** -8
    assert np.all(np.abs(out - x) <= bound)


def test_kv_decay_per_block_beats_per_tensor():
    """Diagnostic from the long-context page: late (small) keys lose precision
    under a single scale and keep it under per-(head, 128-token) scales."""
    rng = np.random.default_rng(14)
    t = 4096
    k = rng.standard_normal((1, t, 128)).astype(np.float32) * np.exp2(-16 * np.arange(t) / t)[None, :, None].astype(np.float32)
    k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
    q, s = quant.kv_quantize(k, 128)
    blk = quant.bf16_bits_to_f32(quant.kv_dequantize(q, s, 128))
    qt, st = quant.quantize_per_tensor(k)
    tens = e4m3.decode(qt) * float(st[0])
    late = slice(t - 128, t)
    rel_blk = np.abs(blk[0, late] - k[0, late]).sum() / np.abs(k[0, late]).sum()
    rel_ten = np.abs(tens[0, late] - k[0, late]).sum() / np.abs(k[0, late]).sum()
    assert rel_blk < 1 / 16
    assert rel_ten > 4 * rel_blk
