"""Pins of the oracle's block-scaled GEMM.

Source: wangyu.me "大语言模型量化技术（五）：FP8", section "激活动态量化" (the product
as a sum over 128-wide K blocks of activation scale x weight-block scale x FP8
block product) and section "FP8 矩阵乘" (128x128 weight blocks, 1x128 activation
groups, FP8 products, fp32 accumulation, partial results multiplied by their
scales). The pins are exact rational sums (Python fractions), a closed form for
one K block, an identity weight that reproduces the dequantized activations,
and symmetries (scale equivalence, sign, power-of-two linearity). Shapes are
non-square so that a transposed operand fails.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, c ^ 0x01, c)   # avoid the NaN codes
    return c.astype(np.uint8)


def _rand_scales(rng, shape):
    return (rng.uniform(0.5, 2.0, size=shape) * np.exp2(rng.integers(-12, 4, size=shape))).astype(np.float32)


def _exact_y(qa, sa, qw, sw, gran_a, gran_w):
    """Exact rational y[m, n] = sum_j s_a s_w sum_{k in block j} dec(qa) dec(qw)."""
    M, K = qa.shape
    N = qw.shape[0]
    # decoded values times 2^9 are integers, so the block sums are exact integers / 2^18
    ia = (e4m3.decode(qa) * 512).astype(np.int64)
    iw = (e4m3.decode(qw) * 512).astype(np.int64)
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for j in range(K // 128):
                p = int(np.dot(ia[m, 128 * j:128 * (j + 1)], iw[n, 128 * j:128 * (j + 1)]))
                s_a = float(sa[0]) if gran_a == gemm.PER_TENSOR else float(sa[m, j])
                s_w = float(sw[0]) if gran_w == gemm.PER_TENSOR else float(sw[n // 128, j])
                tot += Fraction(s_a) * Fraction(s_w) * Fraction(p, 1 << 18)
            out[m][n] = tot
    return out


@pytest.mark.parametrize("gran_a,gran_w", [
    (gemm.GROUP_1x128, gemm.BLOCK_128x128),
    (gemm.PER_TENSOR, gemm.PER_TENSOR),
    (gemm.GROUP_1x128, gemm.PER_TENSOR),
])
def test_bruteforce_exact_rational(gran_a, gran_w):
    rng = np.random.default_rng(21)
    M, N, K = 3, 5, 384
    qa = _rand_codes(rng, (M, K))
    qw = _rand_codes(rng, (N, K))
    # only rows 0..4 of W are used, but the scale grid follows N
    sa = _rand_scales(rng, (1,)) if gran_a == gemm.PER_TENSOR else _rand_scales(rng, (M, K // 128))
    sw = _rand_scales(rng, (1,)) if gran_w == gemm.PER_TENSOR else _rand_scales(rng, (1, K // 128))
    y, t = gemm.block_gemm(qa, sa, gran_a, qw, sw, gran_w)
    assert y.shape == (M, N)
    ex = _exact_y(qa, sa, qw, sw, gran_a, gran_w)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - ex[m][n]) <= Fraction(float(t[m, n])) * Fraction(1, 1 << 45)


def test_bruteforce_several_weight_blocks():
    rng = np.random.default_rng(22)
    M, N, K = 2, 260, 256          # N spans three 128-row weight blocks (ragged)
    qa = _rand_codes(rng, (M, K))
    qw = _rand_codes(rng, (N, K))
    sa = _rand_scales(rng, (M, 2))
    sw = _rand_scales(rng, (3, 2))
    y, t = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128)
    cols = [0, 127, 128, 255, 256, 259]
    # exact sums with the right weight-block row of the scale grid
    ia = (e4m3.decode(qa) * 512).astype(np.int64)
    iw = (e4m3.decode(qw) * 512).astype(np.int64)
    for m in range(M):
        for n in cols:
            tot = Fraction(0)
            for j in range(2):
                p = int(np.dot(ia[m, 128 * j:128 * (j + 1)], iw[n, 128 * j:128 * (j + 1)]))
                tot += Fraction(float(sa[m, j])) * Fraction(float(sw[n // 128, j])) * Fraction(p, 1 << 18)
            assert abs(Fraction(float(y[m, n])) - tot) <= Fraction(float(t[m, n])) * Fraction(1, 1 << 45)


def test_single_block_closed_form():
    """K = 128: y = s_a * s_w * (an integer-grid dot product)."""
    rng = np.random.default_rng(23)
    qa = _rand_codes(rng, (4, 128))
    qw = _rand_codes(rng, (6, 128))
    sa = np.array([0.75], dtype=np.float32)
    sw = np.array([2.0 ** -5], dtype=np.float32)
    y, _ = gemm.block_gemm(qa, sa, gemm.PER_TENSOR, qw, sw, gemm.PER_TENSOR)
    ia = (e4m3.decode(qa) * 512).astype(np.int64)
    iw = (e4m3.decode(qw) * 512).astype(np.int64)
    dots = ia @ iw.T
    assert np.array_equal(y, dots.astype(np.float64) * (0.75 * 2.0 ** -5) / (1 << 18))


def test_identity_weight_reproduces_activations_for_every_code():
    """W = identity (code 0x38 = 1.0) with s_w = 1: y is A_hat exactly. The rows
    of A hold every finite code, which pins the decode of all 254 of them."""
    codes = e4m3.finite_codes()
    K = 256
    qa = np.zeros((2, K), dtype=np.uint8)
    qa[0, :127] = codes[:127]
    qa[1, :127] = codes[127:]
    sa = np.ones((2, 2), dtype=np.float32)
    sa[1, 0] = 3.0
    qw = np.zeros((K, K), dtype=np.uint8)
    qw[np.arange(K), np.arange(K)] = 0x38
    sw = np.ones((2, 2), dtype=np.float32)
    y, _ = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128)
    expect = e4m3.decode(qa) * np.repeat(sa, 128, axis=1)
    assert np.array_equal(y, expect)
    assert y[0, 126] == 448.0 and y[1, 126] == -448.0 * 3.0


def test_per_tensor_equals_blocks_with_equal_scales():
    rng = np.random.default_rng(24)
    qa = _rand_codes(rng, (7, 256))
    qw = _rand_codes(rng, (256, 256))
    y1, _ = gemm.block_gemm(qa, np.array([0.5], np.float32), gemm.PER_TENSOR,
                            qw, np.array([0.125], np.float32), gemm.PER_TENSOR)
    y2, _ = gemm.block_gemm(qa, np.full((7, 2), 0.5, np.float32), gemm.GROUP_1x128,
                            qw, np.full((2, 2), 0.125, np.float32), gemm.BLOCK_128x128)
    assert np.array_equal(y1, y2)


def test_sign_flip_negates():
    rng = np.random.default_rng(25)
    qa = _rand_codes(rng, (5, 256))
    qw = _rand_codes(rng, (128, 256))
    sa = _rand_scales(rng, (5, 2))
    sw = _rand_scales(rng, (1, 2))
    y, _ = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128)
    yn, _ = gemm.block_gemm(qa ^ 0x80, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128)
    assert np.array_equal(yn, -y)


def test_power_of_two_block_scale_linearity():
    rng = np.random.default_rng(26)
    qa = _rand_codes(rng, (4, 256))
    qw = _rand_codes(rng, (128, 256))
    sa = np.ones((4, 2), np.float32)
    sw = np.array([[1.0, 1.0]], np.float32)
    y, _ = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128)
    only1, _ = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, np.array([[0.0, 1.0]], np.float32), gemm.BLOCK_128x128)
    y8, _ = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, np.array([[1.0, 8.0]], np.float32), gemm.BLOCK_128x128)
    assert np.array_equal(y8, y + 7 * only1)


def test_tolerance_base_dominates():
    rng = np.random.default_rng(27)
    qa = _rand_codes(rng, (6, 256))
    qw = _rand_codes(rng, (130, 256))
    sa = _rand_scales(rng, (6, 2))
    sw = _rand_scales(rng, (2, 2))
    y, t = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128)
    assert np.all(np.abs(y) <= t)
    sub_y, sub_t = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128,
                                   rows=[5, 0], cols=[129, 3])
    # same definition on a subset; BLAS may order the sums differently
    ref_t = t[np.ix_([5, 0], [129, 3])]
    assert np.all(np.abs(sub_y - y[np.ix_([5, 0], [129, 3])]) <= 1e-13 * ref_t)
    assert np.all(np.abs(sub_t - ref_t) <= 1e-13 * ref_t)


def _rand_codes_fmt(rng, shape, fmt):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    if fmt == "e4m3":
        c = np.where((c & 0x7F) == 0x7F, c ^ 0x01, c)
    else:
        c = np.where((c & 0x7F) >= 0x7C, c & 0xBB, c)   # no inf / NaN codes
    return c.astype(np.uint8)


@pytest.mark.parametrize("fmt_a,fmt_w", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_bruteforce_exact_rational_e5m2_operands(fmt_a, fmt_w):
    """E5M2 operands ([FP8] section "FP8 是什么", format table): the same block sum
    with each operand decoded from its own format, against exact fractions."""
    from oracle import quant
    rng = np.random.default_rng(24)
    M, N, K = 3, 4, 256
    qa = _rand_codes_fmt(rng, (M, K), fmt_a)
    qw = _rand_codes_fmt(rng, (N, K), fmt_w)
    sa = _rand_scales(rng, (M, 2))
    sw = _rand_scales(rng, (1, 2))
    y, t = gemm.block_gemm(qa, sa, gemm.GROUP_1x128, qw, sw, gemm.BLOCK_128x128, fmt_a=fmt_a, fmt_w=fmt_w)
    da = quant.fmt_module(fmt_a).decode(qa)
    dw = quant.fmt_module(fmt_w).decode(qw)
    assert np.all(np.isfinite(da)) and np.all(np.isfinite(dw))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for j in range(2):
                p = sum((Fraction(float(da[m, k])) * Fraction(float(dw[n, k])) for k in range(128 * j, 128 * (j + 1))),
                        Fraction(0))
                tot += Fraction(float(sa[m, j])) * Fraction(float(sw[0, j])) * p
            assert abs(Fraction(float(y[m, n])) - tot) <= Fraction(float(t[m, n])) * Fraction(1, 1 << 45)


def test_identity_weight_reproduces_every_e5m2_code():
    """E4M3 identity weight (0x38 = 1.0) times E5M2 activations holding all 248
    finite codes reproduces their decoded values exactly."""
    from oracle import e5m2
    codes = e5m2.finite_codes()
    K = 256
    qa = np.zeros((1, K), dtype=np.uint8)
    qa[0, :codes.size] = codes
    qw = np.zeros((K, K), dtype=np.uint8)
    np.fill_diagonal(qw, 0x38)
    one = np.ones(1, dtype=np.float32)
    y, _ = gemm.block_gemm(qa, one, gemm.PER_TENSOR, qw, one, gemm.PER_TENSOR, fmt_a="e5m2", fmt_w="e4m3")
    assert np.array_equal(y[0, :codes.size], e5m2.DECODE[codes])
