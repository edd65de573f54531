"""GPU parity of the MX path (block-32 power-of-two scales) against the CPU oracle.

fp8_quantize_mx: codes and E8M0 scale bytes bit-exact against oracle.mx
([VS] api.makesence.top section 3: Microscaling, blocks of 32). fp8_mx_gemm:
|y - y64| <= 1e-3 * T in fp32 mode, the bf16 output equal to bf16(fp32 output)
and within 1e-3 * T + half a bf16 ulp, as the block-scaled GEMM. The random
scale bytes differ per (row, 32-block), so a wrong scale-to-block mapping in
the scaled MFMA fails the comparison.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, bf16_round_f32, check_gemm_tolerance, f32_of
from oracle import e4m3, e5m2, mx, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _padded(x32, dtype, rows, cols):
    ld = (cols + 15) // 16 * 16
    buf = torch.full((rows, ld), float("nan"), dtype=dtype)
    buf[:, :cols] = torch.from_numpy(x32).to(dtype)
    return buf.to(DEV)[:, :cols]


def _check_quant(gpu_lib, x32, dtype, fmt, what):
    rows, cols = x32.shape
    xt = _padded(x32, dtype, rows, cols)
    xr = xt.float().cpu().numpy()
    qr, sr = mx.quantize_mx(xr, fmt)
    qg, sg = gpu_lib.fp8_quantize_mx(xt, fmt)
    sg = sg.cpu().numpy()
    bad = np.argwhere(sg != sr)
    assert bad.size == 0, f"{what}: scale byte mismatch at {tuple(bad[0])}: gpu {sg[tuple(bad[0])]} oracle {sr[tuple(bad[0])]}"
    assert_codes_equal(qg.cpu().numpy(), qr, xr, what + " codes")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 31), (5, 33), (64, 300), (129, 1024)])
def test_quantize_shapes(gpu_lib, fmt, dtype, rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-40, 40, size=(rows, 1)))).astype(np.float32)
    _check_quant(gpu_lib, x, dtype, fmt, f"{rows}x{cols} {fmt}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_across_the_range(gpu_lib, fmt):
    """Blocks whose maxima sweep the whole fp32 range (subnormal to huge,
    including exact MAX * 2^k maxima and zero blocks)."""
    rng = np.random.default_rng(31)
    G = 8192
    mag = np.exp2(rng.uniform(-148, 127, size=G)).astype(np.float32)
    mx_ = np.float32(quant.FORMAT_MAX[fmt])
    mag[::7] = (mx_ * np.exp2(rng.integers(-120, 100, size=mag[::7].size))).astype(np.float32)
    mag[::11] = 0.0
    x = (rng.uniform(-1, 1, size=(G, 32)) * mag[:, None]).astype(np.float32)
    x[np.arange(G), rng.integers(0, 32, size=G)] = mag * np.where(rng.random(G) < 0.5, -1, 1)
    _check_quant(gpu_lib, x.reshape(G // 4, 128), torch.float32, fmt, f"range {fmt}")


def test_quantize_every_bf16_below_sampled_amax(gpu_lib):
    rng = np.random.default_rng(32)
    rows = []
    for A in np.unique(np.concatenate([[0x0001, 0x0080, 0x3F80, 0x43E0, 0x7F7F], rng.integers(1, 0x7F80, 60)])):
        mags = np.arange(A + 1, dtype=np.int64)
        pat = mags | ((mags & 1) << 15)
        pat = np.concatenate([pat, np.zeros((-len(pat)) % 31, np.int64)]).reshape(-1, 31)
        rows.append(np.concatenate([np.full((pat.shape[0], 1), A, np.int64), pat], axis=1))
    bits = np.concatenate(rows).astype(np.uint16)
    x = quant.bf16_bits_to_f32(bits)
    _check_quant(gpu_lib, x, torch.bfloat16, "e4m3", "every bf16 value")


def test_quantize_full_size_activations(gpu_lib):
    a = syn.activations(2)
    rows = np.random.default_rng(33).choice(a.shape[0], 64, replace=False)
    qg, sg = gpu_lib.fp8_quantize_mx(a.to(DEV))
    qr, sr = mx.quantize_mx(a[rows].float().numpy())
    assert np.array_equal(sg.cpu().numpy()[rows], sr)
    assert_codes_equal(qg.cpu().numpy()[rows], qr, a[rows].float().numpy(), "full-size MX codes")


def _gemm_compare(gpu_lib, qa, sa, qw, sw, fa, fw, what, rows=None, cols=None):
    y32 = gpu_lib.fp8_mx_gemm(qa, sa, qw, sw, out_dtype=torch.float32, fmt_a=fa, fmt_w=fw).cpu().numpy()
    y16 = f32_of(gpu_lib.fp8_mx_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16, fmt_a=fa, fmt_w=fw))
    assert np.array_equal(y16.view(np.uint32), bf16_round_f32(y32).view(np.uint32)), what + ": bf16 != bf16(fp32)"
    if rows is not None:
        y32, y16 = y32[np.ix_(rows, cols)], y16[np.ix_(rows, cols)]
    y64, t = mx.mx_gemm(qa.cpu().numpy(), sa.cpu().numpy(), qw.cpu().numpy(), sw.cpu().numpy(), fa, fw,
                        rows=rows, cols=cols)
    check_gemm_tolerance(y32, y64, t, bf16=False, what=what + " fp32")
    check_gemm_tolerance(y16, y64, t, bf16=True, what=what + " bf16")


def _rand_codes(rng, shape, fmt):
    c = rng.integers(0, 256, size=shape)
    if fmt == "e4m3":
        c = np.where((c & 0x7F) == 0x7F, c ^ 1, c)
    else:
        c = np.where((c & 0x7F) >= 0x7C, c & 0xBB, c)
    return c.astype(np.uint8)


@pytest.mark.parametrize("fa,fw", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("M", [8, 300])
def test_gemm_random_codes_and_scales(gpu_lib, fa, fw, M):
    rng = np.random.default_rng(M + len(fa + fw))
    N, K = 384, 512
    qa, qw = _rand_codes(rng, (M, K), fa), _rand_codes(rng, (N, K), fw)
    sa = rng.integers(112, 142, size=(M, K // 32)).astype(np.uint8)
    sw = rng.integers(112, 142, size=(N, K // 32)).astype(np.uint8)
    t = lambda x: torch.from_numpy(x).to(DEV)
    _gemm_compare(gpu_lib, t(qa), t(sa), t(qw), t(sw), fa, fw, f"random {fa}x{fw} M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (65, 256, 384), (513, 640, 256)])
def test_gemm_quantized_operands(gpu_lib, M, N, K):
    a = syn.activations(2, M=M, K=K, variant=M).to(DEV)
    w = syn.weights(2, N=N, K=K, variant=M).to(DEV)
    qa, sa = gpu_lib.fp8_quantize_mx(a)
    qw, sw = gpu_lib.fp8_quantize_mx(w)
    _gemm_compare(gpu_lib, qa, sa, qw, sw, "e4m3", "e4m3", f"{M}x{N}x{K}")


def test_gemm_decodes_every_code(gpu_lib):
    """A holds every finite E4M3 code (rows 0-1) and every finite E5M2 code
    (rows 2-3 of a second call); W is the identity with unit scales."""
    K = 256
    ident = np.zeros((K, K), np.uint8)
    ident[np.arange(K), np.arange(K)] = 0x38
    ones = np.full((K, K // 32), 127, np.uint8)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    for mod, fmt in ((e4m3, "e4m3"), (e5m2, "e5m2")):
        codes = mod.finite_codes()
        qa = np.zeros((2, K), np.uint8)
        qa.reshape(-1)[:codes.size] = codes
        sa = np.full((2, K // 32), 127, np.uint8)
        sa[1, 3] = 130                      # one block scaled by 8
        y = gpu_lib.fp8_mx_gemm(t(qa), t(sa), t(ident), t(ones), out_dtype=torch.float32, fmt_a=fmt).cpu().numpy()
        expect = mod.decode(qa) * np.repeat(np.exp2(sa.astype(np.float64) - 127), 32, axis=1)
        assert np.array_equal(y, expect), fmt


def test_gemm_full_size_sampled(gpu_lib):
    c = syn.CONFIGS[2]
    M, N, K = c["M"], c["N"], c["K"]
    qa, sa = gpu_lib.fp8_quantize_mx(syn.activations(2).to(DEV))
    qw, sw = gpu_lib.fp8_quantize_mx(syn.weights(2).to(DEV))
    rng = np.random.default_rng(34)
    rows = np.unique(np.concatenate([rng.choice(M, 64, replace=False), [0, 255, 256, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 64, replace=False), [0, 127, 128, 255, 256, N - 1]]))
    _gemm_compare(gpu_lib, qa, sa, qw, sw, "e4m3", "e4m3", "4096x14336x4096", rows=rows, cols=cols)
