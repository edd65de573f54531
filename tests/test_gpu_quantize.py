"""GPU parity of fp8_quantize against the CPU oracle: codes and scales bit-exact.

Covers: every fp32 value in [-448, 448] through the encoder (groups whose scale
is exactly 1), fp32 quotients placed next to every kind of E4M3 midpoint,
random bf16 groups over the whole bf16 range (subnormal to max), all three
granularities on ragged shapes with padded leading dimensions, both input
dtypes, both scale layouts, and the activation / weight tensors of every
configuration at full size, and every bf16 value under every bf16 amax whose
scale takes the reciprocal fast path.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, assert_scales_equal, f32_of, pmap
from oracle import e4m3, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_code_boundaries():
    """For c = 1..126: the smallest non-negative fp32 bit pattern the oracle
    encodes to a code >= c (the oracle is monotone in the magnitude)."""
    out = []
    for c in range(1, 127):
        lo, hi = 0, 0x43E00000
        while lo < hi:
            mid = (lo + hi) // 2
            v = np.array([mid], dtype=np.uint32).view(np.float32)
            if e4m3.encode(v)[0] >= c:
                hi = mid
            else:
                lo = mid + 1
        out.append(lo)
    return np.array(out, dtype=np.int64)


def test_encoder_every_fp32_value_up_to_448(gpu_lib):
    """Every fp32 bit pattern with |x| <= 448 (and its negation) in groups of
    127 next to one 448.0, so s == 1 and x / s == x. Expected codes come from
    the oracle's own boundaries between consecutive codes."""
    bounds = torch.tensor(_oracle_code_boundaries(), device=DEV)
    total = 0x43E00000 + 1
    per = 127
    chunk_groups = 1 << 21
    start = 0
    while start < total:
        ng = min(chunk_groups, (total - start + per - 1) // per)
        pats = torch.arange(start, start + ng * per, device=DEV, dtype=torch.int64).clamp_(max=total - 1)
        expect = torch.searchsorted(bounds, pats, right=True).to(torch.uint8).view(ng, per)
        x = torch.empty((ng, 128), dtype=torch.float32, device=DEV)
        x[:, 0] = 448.0
        x[:, 1:] = pats.to(torch.int32).view(torch.float32).view(ng, per)
        for sign in (1.0, -1.0):
            q, s = gpu_lib.fp8_quantize(x * sign, "group_1x128")
            assert bool(torch.all(s == 1.0))
            want = expect if sign > 0 else (expect | 0x80)
            bad = q[:, 1:] != want
            if bool(bad.any()):
                i = int(torch.nonzero(bad.view(-1))[0])
                p = int(pats[i])
                raise AssertionError(f"pattern 0x{p:08x} sign {sign}: gpu 0x{int(q[:, 1:].reshape(-1)[i]):02x} "
                                     f"oracle 0x{int(want.reshape(-1)[i]):02x}")
            assert bool(torch.all(q[:, 0] == (0x7E if sign > 0 else 0xFE)))
        start += ng * per
        del pats, expect, x
    torch.cuda.synchronize()


def test_fp32_quotients_next_to_midpoints(gpu_lib):
    """x = fl32(m * s) nudged by -3..3 ulps for E4M3 midpoints m (normal and
    subnormal range), under scales with full 24-bit mantissas."""
    rng = np.random.default_rng(202)
    G = 4096
    # three quarters with normal scales, one quarter with fp32-subnormal scales
    amax = np.exp2(np.concatenate([rng.uniform(-100, 100, size=3 * G // 4),
                                   rng.uniform(-140, -118, size=G // 4)])).astype(np.float32)
    s = quant.scale_of(amax)
    mids = np.concatenate([e4m3.MIDPOINTS, e4m3.GRID[1:126]])
    m = rng.choice(mids, size=(G, 127))
    x = (m * s[:, None].astype(np.float64)).astype(np.float32)
    k = rng.integers(-3, 4, size=(G, 127))
    xi = np.maximum(x.view(np.int32) + k.astype(np.int32), 0)
    x = xi.view(np.float32)
    x = np.where(np.abs(x) <= amax[:, None], x, x * np.float32(0.5))
    x *= np.where(rng.random((G, 127)) < 0.5, np.float32(-1), np.float32(1))
    full = np.concatenate([amax[:, None], x], axis=1).astype(np.float32)
    perm = rng.permuted(np.tile(np.arange(128), (G, 1)), axis=1)
    full = np.take_along_axis(full, perm, axis=1)
    qr, sr = quant.quantize_group_1x128(full)
    qg, sg = gpu_lib.fp8_quantize(torch.from_numpy(full).to(DEV), "group_1x128")
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, full, "codes")


def _random_bf16_groups(rng, G):
    """bf16 groups: one amax pattern per group; the rest have |x| <= amax,
    half spread over every pattern below it, half within 16 binades of it."""
    amax_bits = rng.integers(0x0001, 0x7F80, size=G).astype(np.int64)
    u = rng.random((G, 127))
    near = np.maximum(amax_bits[:, None] - (u * 2048).astype(np.int64), 0)
    spread = (u * (amax_bits[:, None] + 1)).astype(np.int64)
    mag = np.where((np.arange(G) % 2 == 0)[:, None], near, spread)
    sign = (rng.random((G, 127)) < 0.5).astype(np.int64) << 15
    bits = np.concatenate([amax_bits[:, None] | ((rng.random((G, 1)) < 0.5).astype(np.int64) << 15),
                           mag | sign], axis=1).astype(np.uint16)
    perm = rng.permuted(np.tile(np.arange(128), (G, 1)), axis=1)
    bits = np.take_along_axis(bits, perm, axis=1)
    return quant.bf16_bits_to_f32(bits)


def test_bf16_groups_across_the_range(gpu_lib):
    rng = np.random.default_rng(203)
    x = _random_bf16_groups(rng, 1 << 15)
    qr, sr = quant.quantize_group_1x128(x)
    xt = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    qg, sg = gpu_lib.fp8_quantize(xt, "group_1x128")
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, "codes")


def test_bf16_every_value_below_sampled_amax(gpu_lib):
    """For sampled bf16 amax patterns A, every bf16 pattern |x| <= A (both
    signs, and -0) appears in a 1x128 group whose amax is A. The samples include
    the patterns whose scale amax / 448 sits at either side of 2^-64 and 2^64
    and the smallest and largest finite ones."""
    rng = np.random.default_rng(211)
    edges = []
    for e in (-64.0, 64.0):
        a = np.float32(np.ldexp(448.0, int(e)))
        b = int(np.array([a], np.float32).view(np.uint32)[0] >> 16)
        edges += [b - 2, b - 1, b, b + 1, b + 2]
    amax_bits = np.unique(np.concatenate([
        np.array(edges + [0x0001, 0x0002, 0x0080, 0x3F80, 0x43E0, 0x7F7F], np.int64),
        rng.integers(0x0001, 0x7F80, size=200)]))
    rows = []
    for A in amax_bits:
        mags = np.arange(A + 1, dtype=np.int64)
        sign = (np.arange(A + 1) & 1).astype(np.int64) << 15
        pat = np.concatenate([mags | sign, [0x8000]])
        pad = (-len(pat)) % 127
        pat = np.concatenate([pat, np.zeros(pad, np.int64)]).reshape(-1, 127)
        head = np.full((pat.shape[0], 1), A, np.int64)
        rows.append(np.concatenate([head, pat], axis=1))
    bits = np.concatenate(rows).astype(np.uint16)
    x = quant.bf16_bits_to_f32(bits)
    qr, sr = quant.quantize_group_1x128(x)
    xt = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    qg, sg = gpu_lib.fp8_quantize(xt, "group_1x128")
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, "codes")


def _fast_path_amax_patterns(fmt="e4m3"):
    """Every positive finite bf16 pattern A whose scale fl32(A / MAX) lies in
    [2^-64, 2^64]: the groups whose bf16 elements the 1x128 quantizer divides
    through its Newton reciprocal and one residual correction."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    s = quant.scale_of(quant.bf16_bits_to_f32(bits), fmt)
    keep = (s >= np.float32(2.0 ** -64)) & (s <= np.float32(2.0 ** 64))
    return bits[keep].astype(np.int64)


def _sweep_groups(amax):
    """1x128 groups holding, for each amax pattern A, every bf16 pattern with
    |x| <= A in both signs (-0 included), 127 per group after one A; the last
    group of each A is padded with +0. Returns uint16 bits [groups, 128]."""
    n = 2 * (amax + 1)
    rows_per = -(-n // 127)
    starts = np.cumsum(rows_per) - rows_per
    r_in = np.arange(rows_per.sum()) - np.repeat(starts, rows_per)
    i = r_in[:, None] * 127 + np.arange(127)[None, :]
    valid = i < np.repeat(n, rows_per)[:, None]
    pat = np.where(valid, (i >> 1) | ((i & 1) << 15), 0)
    return np.concatenate([np.repeat(amax, rows_per)[:, None], pat], axis=1).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_bf16_fast_path_exhaustive(gpu_lib, fmt):
    """Every bf16 amax whose scale lies in [2^-64, 2^64] (16385 patterns for
    either format) and, under each, every bf16 |x| <= amax in both signs:
    5.7e8 (E4M3) and 6.0e8 (E5M2) elements in 4.5e6 and 4.7e6 groups, codes
    and scales against the oracle, in chunks of 256 amax patterns."""
    amax = _fast_path_amax_patterns(fmt)
    assert amax.size == 16385
    checked = 0
    for c0 in range(0, amax.size, 256):
        bits = _sweep_groups(amax[c0:c0 + 256])
        qg, sg = gpu_lib.fp8_quantize(torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16),
                                      "group_1x128", fmt=fmt)
        qg, sg = qg.cpu().numpy(), sg.cpu().numpy()
        x = quant.bf16_bits_to_f32(bits)
        parts = pmap(lambda r: quant.quantize_group_1x128(x[r:r + 8192], fmt), range(0, x.shape[0], 8192))
        assert_scales_equal(sg, np.concatenate([p[1] for p in parts]), f"{fmt} amax chunk {c0} scales")
        assert_codes_equal(qg, np.concatenate([p[0] for p in parts]), x, f"{fmt} amax chunk {c0} codes")
        checked += x.shape[0] * 127
    print(f"bf16 fast path ({fmt}): {checked} element slots under {amax.size} amax patterns match the oracle")


def _padded(x32: np.ndarray, dtype, ld: int) -> torch.Tensor:
    rows, cols = x32.shape
    buf = torch.full((rows, ld), float("nan"), dtype=dtype)
    buf[:, :cols] = torch.from_numpy(x32).to(dtype)
    return buf.to(DEV)[:, :cols]


ORACLE = {"per_tensor": quant.quantize_per_tensor, "group_1x128": quant.quantize_group_1x128,
          "block_128x128": quant.quantize_block_128x128}


@pytest.mark.parametrize("gran", ["per_tensor", "group_1x128", "block_128x128"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols,ld", [(1, 1, 8), (7, 3, 16), (300, 2, 16), (3, 8, 8), (5, 300, 304),
                                          (129, 131, 136), (257, 1000, 1024), (130, 128, 128), (1, 4096, 4096)])
def test_ragged_shapes(gpu_lib, gran, dtype, rows, cols, ld):
    rng = np.random.default_rng(rows * 7919 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-8, 8, size=(rows, 1)))).astype(np.float32)
    x = torch.from_numpy(x).to(dtype).float().numpy()
    xt = _padded(x, dtype, ld)
    qr, sr = ORACLE[gran](x)
    qg, sg = gpu_lib.fp8_quantize(xt, gran)
    assert_scales_equal(sg.cpu().numpy(), sr, f"{gran} scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, f"{gran} codes")


@pytest.mark.parametrize("gran", ["per_tensor", "group_1x128", "block_128x128"])
def test_special_values(gpu_lib, gran):
    """Zero groups, negative zeros, bf16 subnormals, the largest bf16 values,
    and groups mixing 2^-133 with 2^127."""
    rows, cols = 256, 384
    x = np.zeros((rows, cols), dtype=np.float32)
    x[0:128, 0:128] = -0.0
    sub = quant.bf16_bits_to_f32(np.arange(1, 129, dtype=np.uint16))
    x[128:256, 0:128] = np.tile(sub, (128, 1)) * np.where(np.arange(128) % 2, -1, 1)[:, None]
    big = quant.bf16_bits_to_f32(np.arange(0x7F00, 0x7F80, dtype=np.uint16))
    x[0:128, 128:256] = np.tile(big, (128, 1))
    x[128:256, 128:256] = np.where(np.arange(128)[None, :] % 2, 2.0 ** 127, 2.0 ** -133)
    x[:, 256:] = np.linspace(-1, 1, 128)[None, :]
    x[5, 300] = -0.0
    xt = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    x = f32_of(xt)
    qr, sr = ORACLE[gran](x)
    qg, sg = gpu_lib.fp8_quantize(xt, gran)
    assert_scales_equal(sg.cpu().numpy(), sr, f"{gran} scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, f"{gran} codes")


def test_kmajor_scale_layout(gpu_lib):
    x = syn.activations(2, M=300, K=1024)
    qr, sr = quant.quantize_group_1x128(f32_of(x))
    qg, sg = gpu_lib.fp8_quantize(x.to(DEV), "group_1x128", scale_layout="kmajor")
    assert sg.stride(0) == 1 and sg.stride(1) == 300
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, None, "codes")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 300), (7, 129), (33, 1000), (257, 256), (1000, 4096)])
def test_kmajor_ragged(gpu_lib, fmt, dtype, rows, cols):
    """K-block-major scales (workgroups then walk a column of groups down the
    rows) on ragged shapes, both input dtypes and formats."""
    rng = np.random.default_rng(rows * 13 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-10, 10, size=(rows, 1)))).astype(np.float32)
    ld = (cols + 15) // 16 * 16
    xt = _padded(torch.from_numpy(x).to(dtype).float().numpy(), dtype, ld)
    xr = f32_of(xt)
    qr, sr = quant.quantize_group_1x128(xr, fmt)
    qg, sg = gpu_lib.fp8_quantize(xt, "group_1x128", fmt=fmt, scale_layout="kmajor")
    assert_scales_equal(sg.cpu().numpy(), sr, f"{rows}x{cols} kmajor scales")
    assert_codes_equal(qg.cpu().numpy(), qr, xr, f"{rows}x{cols} kmajor codes")


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_config_activations_full_size(gpu_lib, config):
    c = syn.CONFIGS[config]
    x = syn.activations(config)
    x32 = f32_of(x)
    qr, sr = ORACLE[c["gran_a"]](x32)
    qg, sg = gpu_lib.fp8_quantize(x.to(DEV), c["gran_a"])
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, None, "codes")


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_config_weights_full_size(gpu_lib, config):
    """Every code and scale of each configuration's weights (up to 28672 x
    8192), the oracle run on 128-row slabs in parallel host threads."""
    c = syn.CONFIGS[config]
    w = syn.weights(config)
    qg, sg = gpu_lib.fp8_quantize(w.to(DEV), c["gran_w"])
    qg, sg = qg.cpu().numpy(), sg.cpu().numpy()
    w32 = f32_of(w)
    del w
    if c["gran_w"] == "per_tensor":
        qr, sr = quant.quantize_per_tensor(w32)
        assert_scales_equal(sg, sr, "scales")
        assert_codes_equal(qg, qr, None, "codes")
        return
    slabs = pmap(lambda sl: quant.quantize_block_128x128(w32[sl * 128:(sl + 1) * 128]),
                 range((w32.shape[0] + 127) // 128))
    assert_scales_equal(sg, np.concatenate([s for _, s in slabs]), "scales")
    assert_codes_equal(qg, np.concatenate([q for q, _ in slabs]), None, "codes")


def test_repeated_calls_and_scale_buffer_reuse(gpu_lib):
    """The per-tensor scale slot doubles as the amax accumulator: a second call
    with smaller values must not keep the first call's maximum."""
    a = torch.full((64, 512), 3.0, dtype=torch.bfloat16, device=DEV)
    b = torch.full((64, 512), 0.5, dtype=torch.bfloat16, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    gpu_lib.fp8_quantize(a, "per_tensor", scales=s)
    q, s = gpu_lib.fp8_quantize(b, "per_tensor", scales=s)
    assert float(s[0]) == float(np.float32(0.5) / np.float32(448))
    assert bool(torch.all(q == 0x7E))


@pytest.mark.parametrize("ngroups", [5, 7, 13, 33, 64, 65, 127])
def test_group_index_division(gpu_lib, ngroups):
    """Row / group decomposition of the flat group index for many group counts
    (the kernel divides by the group count with a multiply and shift)."""
    rng = np.random.default_rng(ngroups)
    rows, cols = 67, 128 * ngroups - 40
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-4, 4, size=(rows, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    x = xt.float().numpy()
    qr, sr = quant.quantize_group_1x128(x)
    qg, sg = gpu_lib.fp8_quantize(xt.to(DEV), "group_1x128")
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, "codes")


def test_per_tensor_and_static_grid_stride(gpu_lib):
    """A [16384, 8192] tensor: more chunks than the capped grids of the amax
    and cast passes cover in one round, so every thread loops. The per-tensor
    scale and the static pass's recorded amax are exact; codes are compared on
    sampled rows, including the row that holds the single largest element."""
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(16384, 8192, generator=g) * 3).to(torch.bfloat16)
    x[12345, 777] = -300.0
    x32 = x.float().numpy()
    amax = np.float32(np.abs(x32).max())
    assert amax == np.float32(300.0)
    xd = x.to(DEV)
    rows = np.unique(np.concatenate([np.random.default_rng(6).choice(16384, 40, replace=False), [0, 12345, 16383]]))
    qg, sg = gpu_lib.fp8_quantize(xd, "per_tensor")
    s_ref = quant.scale_of(amax)
    assert_scales_equal(sg.cpu().numpy(), np.array([s_ref], np.float32), "per-tensor scale")
    assert_codes_equal(qg.cpu().numpy()[rows], quant.cast(x32[rows], s_ref), x32[rows], "per-tensor codes")
    s_static = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    qs, am = gpu_lib.fp8_quantize_static(xd, s_static, record_amax=True)
    assert float(am.item()) == 300.0
    qr, _ = quant.quantize_static(x32[rows], np.float32(0.5))
    assert_codes_equal(qs.cpu().numpy()[rows], qr, x32[rows], "static codes")


def test_past_2_31_chunks(gpu_lib):
    """A [2^21 + 64, 8192] bf16 tensor (34 GB) has more than 2^31 chunks of 8
    elements, so the per-tensor and static passes take their 64-bit chunk
    indexing. Built on the device (small N(0, 0.01^2) values and one planted
    maximum of -300 beyond chunk 2^31): the scale and the recorded amax are
    known exactly; codes are compared on sampled rows on both sides of the
    boundary, for per tensor, static and 1 x 128."""
    rows, cols = (1 << 21) + 64, 8192
    torch.manual_seed(7)
    x = torch.randn((rows, cols), dtype=torch.bfloat16, device=DEV)
    x.mul_(0.01)
    x[rows - 10, 4000] = -300.0
    assert (rows - 10) * (cols // 8) > (1 << 31)
    sample = np.array([0, 5, (1 << 21) - 1, 1 << 21, (1 << 21) + 3, rows - 10, rows - 1])
    xs = f32_of(x[torch.from_numpy(sample).to(DEV)])
    try:
        qg, sg = gpu_lib.fp8_quantize(x, "per_tensor")
        s_ref = quant.scale_of(np.float32(300.0))
        assert_scales_equal(sg.cpu().numpy(), np.array([s_ref], np.float32), "per-tensor scale")
        assert_codes_equal(qg[torch.from_numpy(sample).to(DEV)].cpu().numpy(), quant.cast(xs, s_ref), xs,
                           "per-tensor codes")
        s_static = torch.tensor([0.25], dtype=torch.float32, device=DEV)
        qs, am = gpu_lib.fp8_quantize_static(x, s_static, record_amax=True, out=qg)
        assert float(am.item()) == 300.0
        assert_codes_equal(qs[torch.from_numpy(sample).to(DEV)].cpu().numpy(),
                           quant.quantize_static(xs, np.float32(0.25))[0], xs, "static codes")
        del qs, qg
        q1, s1 = gpu_lib.fp8_quantize(x, "group_1x128")
        qr, sr = quant.quantize_group_1x128(xs)
        idx = torch.from_numpy(sample).to(DEV)
        assert_scales_equal(s1[idx].cpu().numpy(), sr, "1x128 scales")
        assert_codes_equal(q1[idx].cpu().numpy(), qr, xs, "1x128 codes")
    finally:
        del x
        torch.cuda.empty_cache()
