"""Pins of the oracle's MX (block-32, power-of-two scale) quantizer and GEMM.

Sources: api.makesence.top "LLM推理量化:FP8 versus INT8", section 3 (Microscaling,
block size 32); wangyu.me "大语言模型量化技术（五）：FP8", section "什么是 FP8 量化"
(scale into the format's range, round to nearest even, saturate).

Independent checks: closed-form exponents for chosen block maxima; the
defining property (smallest power of two that keeps the block max in range)
checked with exact float64 arithmetic against the oracle's search; reduction
to the per-group quantizer when the block max is MAX times a power of two
(then s = amax / MAX is that power of two); exact rational sums for the GEMM,
unit scales reducing it to the per-tensor block GEMM, and exact doubling of
one block's contribution when its scale byte grows by one.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm, mx, quant


@pytest.mark.parametrize("amax,k", [(448.0, 0), (448.0001, 1), (224.0, -1), (1.0, -8), (0.875, -9),
                                    (57344.0 / 128, 0), (0.0, -127), (1e-40, -127), (3.0e38, 120)])
def test_shared_exponent_closed_forms(amax, k):
    assert int(mx.shared_exponent(np.array([amax]))[0]) == k


def test_shared_exponent_e5m2():
    assert int(mx.shared_exponent(np.array([57344.0]), "e5m2")[0]) == 0
    assert int(mx.shared_exponent(np.array([57345.0]), "e5m2")[0]) == 1
    assert int(mx.shared_exponent(np.array([1.0]), "e5m2")[0]) == -15


def test_shared_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(1)
    a = np.exp2(rng.uniform(-130, 127, size=4000)).astype(np.float32).astype(np.float64)
    k = mx.shared_exponent(a)
    for ai, ki in zip(a, k):
        assert 448.0 * 2.0 ** int(ki) >= ai
        if ki > -127:
            assert 448.0 * 2.0 ** (int(ki) - 1) < ai


def test_block_max_never_saturates_and_uses_the_top_binade():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, size=(64, 8)).repeat(32, axis=1))).astype(np.float32)
    q, sb = mx.quantize_mx(x)
    assert q.shape == x.shape and sb.shape == (64, 8)
    xb = np.abs(x).reshape(64, 8, 32)
    qb = e4m3.decode(q).reshape(64, 8, 32)
    idx = xb.argmax(axis=2)
    top = np.take_along_axis(np.abs(qb), idx[..., None], axis=2)[..., 0]
    assert np.all(top <= 448.0) and np.all(top >= 224.0)


def test_reduces_to_the_group_quantizer_at_power_of_two_maxima():
    """With the block max equal to 448 * 2^k, s = amax / 448 = 2^k exactly, so
    the MX codes equal the per-group quantizer's codes on each 32-wide block."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 32 * 6)).astype(np.float32)
    for b in range(6):
        blk = x[:, 32 * b:32 * (b + 1)]
        blk /= np.abs(blk).max(axis=1, keepdims=True)
        blk *= np.float32(448.0) * np.exp2(np.float32(rng.integers(-20, 20)))
    q, sb = mx.quantize_mx(x)
    for b in range(6):
        qr, sr = quant.quantize_per_tensor(x[0:1, 32 * b:32 * (b + 1)])
        assert np.array_equal(q[0:1, 32 * b:32 * (b + 1)], qr)
        assert float(sr[0]) == 2.0 ** (int(sb[0, b]) - 127)


def test_dequant_error_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    q, sb = mx.quantize_mx(x)
    xh = mx.dequantize_mx(q, sb)
    scale = np.repeat(np.exp2(sb.astype(np.float64) - 127), 32, axis=1)
    normal = np.abs(x) >= scale * 2.0 ** -6
    rel = np.abs(xh - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-9)


def test_ragged_last_block():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 70)).astype(np.float32)
    q, sb = mx.quantize_mx(x)
    assert sb.shape == (3, 3)
    q2, sb2 = mx.quantize_mx(x[:, 64:])
    assert np.array_equal(q[:, 64:], q2) and np.array_equal(sb[:, 2], sb2[:, 0])


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


def test_gemm_exact_rational():
    rng = np.random.default_rng(6)
    M, N, K = 3, 4, 128
    qa, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    sw = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    y, t = mx.mx_gemm(qa, sa, qw, sw)
    da, dw = e4m3.decode(qa), e4m3.decode(qw)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                tot += (Fraction(float(da[m, k])) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                        * Fraction(float(dw[n, k])) * Fraction(2) ** (int(sw[n, k // 32]) - 127))
            assert abs(Fraction(float(y[m, n])) - tot) <= Fraction(float(t[m, n])) * Fraction(1, 1 << 45)


def test_unit_scales_reduce_to_the_block_gemm():
    rng = np.random.default_rng(7)
    qa, qw = _codes(rng, (5, 256)), _codes(rng, (6, 256))
    one_a = np.full((5, 8), 127, np.uint8)
    one_w = np.full((6, 8), 127, np.uint8)
    y, _ = mx.mx_gemm(qa, one_a, qw, one_w)
    yb, _ = gemm.block_gemm(qa, np.ones(1, np.float32), gemm.PER_TENSOR, qw, np.ones(1, np.float32), gemm.PER_TENSOR)
    assert np.array_equal(y, yb)


def test_one_scale_byte_doubles_its_block():
    rng = np.random.default_rng(8)
    qa, qw = _codes(rng, (2, 128)), _codes(rng, (3, 128))
    sa = np.full((2, 4), 127, np.uint8)
    sw = np.full((3, 4), 127, np.uint8)
    y0, _ = mx.mx_gemm(qa, sa, qw, sw)
    sa2 = sa.copy()
    sa2[0, 2] += 1
    y1, _ = mx.mx_gemm(qa, sa2, qw, sw)
    blk = e4m3.decode(qa)[0, 64:96] @ e4m3.decode(qw)[:, 64:96].T
    assert np.array_equal(y1[0], y0[0] + blk)
    assert np.array_equal(y1[1], y0[1])
