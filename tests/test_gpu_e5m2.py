"""GPU parity of the E5M2 format through every entry point, against the CPU oracle.

E5M2 ([FP8] section "FP8 是什么", format table: largest value 57344; [VS]
api.makesence.top section 2: the KV cache in E5M2) runs the same per-group
method with s = amax / 57344. Codes, scales and dequantized values are compared bit for
bit; the GEMM with E5M2 operands (alone or mixed with E4M3) is held to the same
tolerance as the E4M3 GEMM.

Covers: every fp32 value in [-57344, 57344] through the encoder (groups with
s == 1), fp32 quotients next to every E5M2 midpoint, random bf16 groups over
the whole range, every bf16 value below sampled amax patterns, all
granularities on ragged shapes for both input dtypes, the KV quantizer and
dequantizer on ragged caches and the full [8, 131072, 128] V tensor, and the
GEMM's decoding of every finite E5M2 code as either operand in the prefill
and decode kernels; the GEMM's fp32 outputs are also held to the model of the
matrix instruction's block sum (tests/mfma_model.py).
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, assert_scales_equal, bf16_round_f32, check_gemm_tolerance, f32_of, pmap
from mfma_model import check_against_model
from oracle import e4m3, e5m2, gemm as ogemm, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"
F = "e5m2"


def _oracle_code_boundaries():
    """For c = 1..123: the smallest non-negative fp32 bit pattern the oracle
    encodes to an E5M2 code >= c."""
    out = []
    top = int(np.array([57344.0], np.float32).view(np.uint32)[0])
    for c in range(1, 0x7C):
        lo, hi = 0, top
        while lo < hi:
            mid = (lo + hi) // 2
            v = np.array([mid], dtype=np.uint32).view(np.float32)
            if e5m2.encode(v)[0] >= c:
                hi = mid
            else:
                lo = mid + 1
        out.append(lo)
    return np.array(out, dtype=np.int64), top


def test_encoder_every_fp32_value_up_to_57344(gpu_lib):
    """Every fp32 bit pattern with |x| <= 57344 (and its negation) in groups of
    127 next to one 57344.0, so s == 1 and x / s == x."""
    b, top = _oracle_code_boundaries()
    bounds = torch.tensor(b, device=DEV)
    total = top + 1
    per = 127
    chunk_groups = 1 << 21
    start = 0
    while start < total:
        ng = min(chunk_groups, (total - start + per - 1) // per)
        pats = torch.arange(start, start + ng * per, device=DEV, dtype=torch.int64).clamp_(max=total - 1)
        expect = torch.searchsorted(bounds, pats, right=True).to(torch.uint8).view(ng, per)
        x = torch.empty((ng, 128), dtype=torch.float32, device=DEV)
        x[:, 0] = 57344.0
        x[:, 1:] = pats.to(torch.int32).view(torch.float32).view(ng, per)
        for sign in (1.0, -1.0):
            q, s = gpu_lib.fp8_quantize(x * sign, "group_1x128", fmt=F)
            assert bool(torch.all(s == 1.0))
            want = expect if sign > 0 else (expect | 0x80)
            bad = q[:, 1:] != want
            if bool(bad.any()):
                i = int(torch.nonzero(bad.view(-1))[0])
                p = int(pats[i])
                raise AssertionError(f"pattern 0x{p:08x} sign {sign}: gpu 0x{int(q[:, 1:].reshape(-1)[i]):02x} "
                                     f"oracle 0x{int(want.reshape(-1)[i]):02x}")
            assert bool(torch.all(q[:, 0] == (0x7B if sign > 0 else 0xFB)))
        start += ng * per
        del pats, expect, x
    torch.cuda.synchronize()


def test_fp32_quotients_next_to_midpoints(gpu_lib):
    """x = fl32(m * s) nudged by -3..3 ulps for E5M2 midpoints and grid values
    m, under scales with full 24-bit mantissas (normal and subnormal)."""
    rng = np.random.default_rng(502)
    G = 4096
    amax = np.exp2(np.concatenate([rng.uniform(-100, 100, size=3 * G // 4),
                                   rng.uniform(-140, -112, size=G // 4)])).astype(np.float32)
    s = quant.scale_of(amax, F)
    mids = np.concatenate([e5m2.MIDPOINTS, e5m2.GRID[1:0x7B]])
    m = rng.choice(mids, size=(G, 127))
    x = (m * s[:, None].astype(np.float64)).astype(np.float32)
    k = rng.integers(-3, 4, size=(G, 127))
    x = np.maximum(x.view(np.int32) + k.astype(np.int32), 0).view(np.float32)
    x = np.where(np.abs(x) <= amax[:, None], x, x * np.float32(0.5))
    x *= np.where(rng.random((G, 127)) < 0.5, np.float32(-1), np.float32(1))
    full = np.concatenate([amax[:, None], x], axis=1).astype(np.float32)
    full = np.take_along_axis(full, rng.permuted(np.tile(np.arange(128), (G, 1)), axis=1), axis=1)
    qr, sr = quant.quantize_group_1x128(full, F)
    qg, sg = gpu_lib.fp8_quantize(torch.from_numpy(full).to(DEV), "group_1x128", fmt=F)
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, full, "codes")


def test_bf16_groups_across_the_range(gpu_lib):
    rng = np.random.default_rng(503)
    G = 1 << 15
    amax_bits = rng.integers(0x0001, 0x7F80, size=G).astype(np.int64)
    u = rng.random((G, 127))
    near = np.maximum(amax_bits[:, None] - (u * 2048).astype(np.int64), 0)
    spread = (u * (amax_bits[:, None] + 1)).astype(np.int64)
    mag = np.where((np.arange(G) % 2 == 0)[:, None], near, spread)
    sign = (rng.random((G, 127)) < 0.5).astype(np.int64) << 15
    bits = np.concatenate([amax_bits[:, None], mag | sign], axis=1).astype(np.uint16)
    bits = np.take_along_axis(bits, rng.permuted(np.tile(np.arange(128), (G, 1)), axis=1), axis=1)
    x = quant.bf16_bits_to_f32(bits)
    qr, sr = quant.quantize_group_1x128(x, F)
    xt = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    qg, sg = gpu_lib.fp8_quantize(xt, "group_1x128", fmt=F)
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, "codes")


def test_bf16_every_value_below_sampled_amax(gpu_lib):
    """For sampled bf16 amax patterns A, every bf16 |x| <= A (both signs, and
    -0) in 1x128 groups whose amax is A; the samples include amax values whose
    scale is a power of two (x / s then lands exactly on E5M2 midpoints)."""
    rng = np.random.default_rng(511)
    pow2 = [int(np.array([np.ldexp(57344.0, e)], np.float32).view(np.uint32)[0] >> 16) for e in (-20, 0, 5)]
    amax_bits = np.unique(np.concatenate([
        np.array(pow2 + [0x0001, 0x0080, 0x3F80, 0x4760, 0x7F7F], np.int64),
        rng.integers(0x0001, 0x7F80, size=120)]))
    rows = []
    for A in amax_bits:
        mags = np.arange(A + 1, dtype=np.int64)
        sign = (np.arange(A + 1) & 1).astype(np.int64) << 15
        pat = np.concatenate([mags | sign, [0x8000]])
        pat = np.concatenate([pat, np.zeros((-len(pat)) % 127, np.int64)]).reshape(-1, 127)
        rows.append(np.concatenate([np.full((pat.shape[0], 1), A, np.int64), pat], axis=1))
    bits = np.concatenate(rows).astype(np.uint16)
    x = quant.bf16_bits_to_f32(bits)
    qr, sr = quant.quantize_group_1x128(x, F)
    xt = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    qg, sg = gpu_lib.fp8_quantize(xt, "group_1x128", fmt=F)
    assert_scales_equal(sg.cpu().numpy(), sr, "scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x, "codes")


ORACLE = {"per_tensor": quant.quantize_per_tensor, "group_1x128": quant.quantize_group_1x128,
          "block_128x128": quant.quantize_block_128x128}


@pytest.mark.parametrize("gran", ["per_tensor", "group_1x128", "block_128x128"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 1), (5, 300), (129, 131), (257, 1000)])
def test_ragged_shapes(gpu_lib, gran, dtype, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(dtype)
    x32 = xt.float().numpy()
    qr, sr = ORACLE[gran](x32, F)
    ld = (cols + 15) // 16 * 16          # row stride: a multiple of 16 bytes for both dtypes
    buf = torch.full((rows, ld), float("nan"), dtype=dtype)
    buf[:, :cols] = xt
    qg, sg = gpu_lib.fp8_quantize(buf.to(DEV)[:, :cols], gran, fmt=F)
    assert_scales_equal(sg.cpu().numpy().reshape(sr.shape), sr, f"{gran} scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x32, f"{gran} codes")


def _check_kv(gpu_lib, kv: torch.Tensor, token_block: int):
    x32 = f32_of(kv)
    qr, sr = quant.kv_quantize(x32, token_block, F)
    qg, sg = gpu_lib.fp8_kv_quantize(kv, token_block, fmt=F)
    assert_scales_equal(sg.cpu().numpy(), sr, "kv scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x32, "kv codes")
    out = gpu_lib.fp8_kv_dequantize(qg, sg, token_block, fmt=F)
    ref = quant.kv_dequantize(qr, sr, token_block, F)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"dequant mismatch at {tuple(bad[0])}: gpu 0x{got[tuple(bad[0])]:04x} oracle 0x{ref[tuple(bad[0])]:04x}"


@pytest.mark.parametrize("heads,tokens,head_dim,token_block", [(1, 1, 8, 128), (3, 1000, 128, 128),
                                                               (2, 777, 64, 128), (4, 300, 128, 32)])
def test_kv_small_caches(gpu_lib, heads, tokens, head_dim, token_block):
    k, v = syn.kv_pair(heads=heads, tokens=tokens, head_dim=head_dim, variant=3)
    _check_kv(gpu_lib, k.to(DEV), token_block)
    _check_kv(gpu_lib, v.to(DEV), token_block)


def test_kv_dequantize_every_code(gpu_lib):
    """Every finite E5M2 code under scales 1, 2^-20 and 3.7 (decode exactness
    and the fp32 product's rounding)."""
    codes = e5m2.finite_codes()
    q = np.zeros((3, 128, 8), dtype=np.uint8)
    for h in range(3):
        q[h].reshape(-1)[:codes.size] = codes
    s = np.array([[1.0], [2.0 ** -20], [3.7]], dtype=np.float32)
    out = gpu_lib.fp8_kv_dequantize(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), 128, fmt=F)
    ref = quant.kv_dequantize(q, s, 128, F)
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), ref)


def test_kv_full_size_v(gpu_lib):
    """Every code, scale and dequantized value of the full [8, 131072, 128] V
    tensor in E5M2 (the oracle on one head per host thread)."""
    _, v = syn.kv_pair(5)
    tb = 128
    qg, sg = gpu_lib.fp8_kv_quantize(v.to(DEV), tb, fmt=F)
    out = gpu_lib.fp8_kv_dequantize(qg, sg, tb, fmt=F)
    qg, sg = qg.cpu().numpy(), sg.cpu().numpy()
    out = out.cpu().view(torch.int16).numpy().view(np.uint16)
    v32 = f32_of(v)
    del v

    def head(h):
        qr, sr = quant.kv_quantize(v32[h:h + 1], tb, F)
        return qr, sr, quant.kv_dequantize(qr, sr, tb, F)

    for h, (qr, sr, dr) in enumerate(pmap(head, range(v32.shape[0]))):
        assert_scales_equal(sg[h:h + 1], sr, f"V scales, head {h}")
        assert_codes_equal(qg[h:h + 1], qr, v32[h:h + 1], f"V codes, head {h}")
        assert np.array_equal(out[h:h + 1], dr), f"V dequant, head {h}"


# ---- GEMM with E5M2 operands --------------------------------------------------

def _gemm_compare(gpu_lib, qa, sa, ga, qw, sw, gw, fa, fw, what):
    args = (qa, sa, ga, qw, sw, gw)
    y32 = gpu_lib.fp8_block_gemm(*args, out_dtype=torch.float32, fmt_a=fa, fmt_w=fw).cpu().numpy()
    y16 = f32_of(gpu_lib.fp8_block_gemm(*args, out_dtype=torch.bfloat16, fmt_a=fa, fmt_w=fw))
    assert np.array_equal(y16.view(np.uint32), bf16_round_f32(y32).view(np.uint32)), what + ": bf16 != bf16(fp32)"
    y64, t = ogemm.block_gemm(qa.cpu().numpy(), sa.cpu().numpy(), ga, qw.cpu().numpy(), sw.cpu().numpy(), gw,
                              fmt_a=fa, fmt_w=fw)
    check_gemm_tolerance(y32, y64, t, bf16=False, what=what + " fp32")
    check_gemm_tolerance(y16, y64, t, bf16=True, what=what + " bf16")
    M, N = y32.shape
    worst = check_against_model(y32, qa.cpu().numpy(), sa.cpu().numpy(), ga, qw.cpu().numpy(), sw.cpu().numpy(),
                                gw, np.arange(M), np.arange(N), fa, fw, what=what)
    print(f"{what}: max |y32 - y_model| / T = {worst:.3e}")


@pytest.mark.parametrize("fa,fw", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("M", [16, 48, 300])
def test_gemm_quantized_operands(gpu_lib, fa, fw, M):
    """Activations and weights quantized on the GPU in the given formats;
    M = 16 and 48 run the decode kernel, 300 the prefill kernel."""
    N, K = 512, 640
    a = syn.activations(2, M=M, K=K, variant=11).to(DEV)
    w = syn.weights(2, N=N, K=K, variant=11).to(DEV)
    qa, sa = gpu_lib.fp8_quantize(a, "group_1x128", fmt=fa)
    qw, sw = gpu_lib.fp8_quantize(w, "block_128x128", fmt=fw)
    _gemm_compare(gpu_lib, qa, sa, "group_1x128", qw, sw, "block_128x128", fa, fw, f"{fa}x{fw} M={M}")


@pytest.mark.parametrize("M", [8, 256])
@pytest.mark.parametrize("side", ["a", "w"])
def test_gemm_decodes_every_e5m2_code(gpu_lib, M, side):
    """One operand holds every finite E5M2 code, the other is an E4M3 identity
    (0x38 = 1.0) with unit scales: the fp32 output reproduces the decoded E5M2
    values exactly, in the decode (M = 8) and prefill (M = 256) kernels."""
    codes = e5m2.finite_codes()
    K = N = 256
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    ones_a = np.ones((M, 2), np.float32)
    ones_w = np.ones((2, 2), np.float32)
    if side == "a":
        # A [M, K] holds the codes; W = identity, so C = A
        qa = np.zeros((M, K), dtype=np.uint8)
        for r in range(M):
            qa[r, :codes.size] = np.roll(codes, 31 * r)
        qw = np.zeros((N, K), dtype=np.uint8)
        qw[np.arange(N), np.arange(K)] = 0x38
        expect = e5m2.decode(qa)
        fa, fw = "e5m2", "e4m3"
    else:
        # A = the first M rows of the identity, W [N, K] holds the codes in
        # its first M columns, so C[m, n] = W[n, m]
        qa = np.zeros((M, K), dtype=np.uint8)
        qa[np.arange(M), np.arange(M)] = 0x38
        qw = np.zeros((N, K), dtype=np.uint8)
        for m in range(M):
            qw[:codes.size, m] = np.roll(codes, 31 * m)
        expect = e5m2.decode(qw[:, :M]).T
        fa, fw = "e4m3", "e5m2"
    y = gpu_lib.fp8_block_gemm(t(qa), t(ones_a), "group_1x128", t(qw), t(ones_w), "block_128x128",
                               out_dtype=torch.float32, fmt_a=fa, fmt_w=fw).cpu().numpy()
    bad = np.argwhere(y != expect)
    assert bad.size == 0, f"first mismatch at {tuple(bad[0])}: gpu {y[tuple(bad[0])]} expect {expect[tuple(bad[0])]}"


def test_gemm_random_e5m2_codes(gpu_lib):
    """Uniformly random finite E5M2 codes against E4M3 codes, scales spread
    over 2^-12 .. 2^3, prefill kernel with a ragged M."""
    rng = np.random.default_rng(521)
    M, N, K = 330, 384, 512
    ca = rng.integers(0, 256, size=(M, K))
    ca = np.where((ca & 0x7F) >= 0x7C, ca & 0xBB, ca).astype(np.uint8)
    cw = rng.integers(0, 256, size=(N, K))
    cw = np.where((cw & 0x7F) == 0x7F, cw ^ 1, cw).astype(np.uint8)
    sa = (rng.uniform(0.5, 2, (M, K // 128)) * np.exp2(rng.integers(-12, 4, (M, K // 128)))).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N // 128, K // 128)) * np.exp2(rng.integers(-12, 4, (N // 128, K // 128)))).astype(np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    _gemm_compare(gpu_lib, t(ca), t(sa), "group_1x128", t(cw), t(sw), "block_128x128", "e5m2", "e4m3", "random e5m2")
