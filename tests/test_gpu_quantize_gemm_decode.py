"""GPU parity of fp8_quantize_gemm_decode: the activations quantized (per
tensor or 1x128) inside the decode GEMM, one launch.

Its output, codes and scales must equal, bit for bit, those of the two calls
it fuses: fp8_quantize(x, gran_a) followed by fp8_block_gemm, or
fp8_block_gemm_packed on decode-packed weights (whose parity with the oracle
the other GPU tests establish). Two configurations are also compared with the
oracle directly, codes and scales exactly and C within the GEMM tolerance:
per-tensor 64x512x512, and the one decode step 16x28672x8192 with 1x128
activations and 128x128 weights (sampled output columns).
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, assert_scales_equal, check_gemm_tolerance, f32_of
from oracle import gemm as ogemm
from oracle import quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _weights(gpu_lib, N, K, gran_w, fmt_w, seed, config=1):
    w = syn.weights(config, N=N, K=K, variant=seed).to(DEV)
    return gpu_lib.fp8_quantize(w, gran_w, fmt=fmt_w)


def _two_calls(gpu_lib, x, qw, sw, gran_w, gran_a, fmt_a, fmt_w, out_dtype, qw_packed, scale_layout):
    qa, sa = gpu_lib.fp8_quantize(x, gran_a, fmt=fmt_a, scale_layout=scale_layout)
    if qw_packed is None:
        y = gpu_lib.fp8_block_gemm(qa, sa, gran_a, qw, sw, gran_w, out_dtype=out_dtype, fmt_a=fmt_a, fmt_w=fmt_w)
    else:
        y = gpu_lib.fp8_block_gemm_packed(qa, sa, gran_a, qw_packed, sw, gran_w, out_dtype=out_dtype, fmt_a=fmt_a,
                                          fmt_w=fmt_w)
    return y, qa, sa


def _compare(gpu_lib, x, qw, sw, gran_w, gran_a="per_tensor", fmt_a="e4m3", fmt_w="e4m3",
             out_dtype=torch.bfloat16, packed=False, scale_layout="row", what=""):
    qw_packed = gpu_lib.fp8_pack_weights_decode(qw) if packed else None
    w_arg = qw_packed if packed else qw
    kw = dict(gran_a=gran_a, fmt_a=fmt_a, fmt_w=fmt_w, out_dtype=out_dtype)
    y, q, s = gpu_lib.fp8_quantize_gemm_decode(x, w_arg, sw, gran_w, return_codes=True, scale_layout=scale_layout,
                                               **kw)
    y_only = gpu_lib.fp8_quantize_gemm_decode(x, w_arg, sw, gran_w, **kw)
    y2, q2, s2 = _two_calls(gpu_lib, x, qw, sw, gran_w, gran_a, fmt_a, fmt_w, out_dtype, qw_packed, scale_layout)
    torch.cuda.synchronize()
    assert s.stride() == s2.stride(), f"{what}: scale layouts differ"
    assert torch.equal(_bits(s), _bits(s2)), f"{what}: scales differ"
    assert torch.equal(q, q2), f"{what}: codes differ"
    assert torch.equal(_bits(y), _bits(y2)), f"{what}: C differs from the two calls"
    assert torch.equal(_bits(y_only), _bits(y2)), f"{what}: C (no codes asked) differs from the two calls"


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 64])
@pytest.mark.parametrize("K", [128, 512, 1024])
def test_per_tensor_shapes_equal_the_two_calls(gpu_lib, M, K):
    if M * K > 65536:
        pytest.skip("beyond the per-tensor path's size")
    x = syn.activations(1, M=M, K=K, variant=M * 7 + K).to(DEV)
    qw, sw = _weights(gpu_lib, 384, K, "block_128x128", "e4m3", K)
    _compare(gpu_lib, x, qw, sw, "block_128x128", what=f"per tensor {M}x384x{K}")


@pytest.mark.parametrize("M", [1, 7, 16, 31, 48, 64])
@pytest.mark.parametrize("K", [128, 384, 4096])
@pytest.mark.parametrize("packed", [False, True])
def test_group_shapes_equal_the_two_calls(gpu_lib, M, K, packed):
    """1x128 activations: K from one to 32 blocks (waves with none, one and
    several K blocks), every M tile count, row-major and packed weights."""
    x = syn.activations(3, M=M, K=K, variant=M * 11 + K).to(DEV)
    qw, sw = _weights(gpu_lib, 384 if not packed else 256, K, "block_128x128", "e4m3", K, config=3)
    _compare(gpu_lib, x, qw, sw, "block_128x128", gran_a="group_1x128", packed=packed,
             what=f"1x128 {M}x{qw.shape[0]}x{K} packed={packed}")


@pytest.mark.parametrize("gran_a", ["per_tensor", "group_1x128"])
@pytest.mark.parametrize("fmt_a,fmt_w", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("gran_w", ["per_tensor", "block_128x128"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_formats_granularities_dtypes(gpu_lib, gran_a, fmt_a, fmt_w, gran_w, dtype, out_dtype):
    M, N, K = 48, 256, 640
    x = syn.activations(1, M=M, K=K, variant=11).to(DEV).to(dtype)
    qw, sw = _weights(gpu_lib, N, K, gran_w, fmt_w, 12)
    _compare(gpu_lib, x, qw, sw, gran_w, gran_a, fmt_a, fmt_w, out_dtype,
             what=f"{gran_a} {fmt_a}/{fmt_w} {gran_w} {dtype} -> {out_dtype}")


@pytest.mark.parametrize("gran_a", ["per_tensor", "group_1x128"])
def test_strided_activations(gpu_lib, gran_a):
    """x as a row slice of a wider buffer whose padding holds a huge value
    (never read: it would set a scale)."""
    M, N, K = 64, 512, 512
    x = syn.activations(1, M=M, K=K, variant=3).to(DEV)
    xbuf = torch.full((M, K + 64), 3.0e38, dtype=torch.float32, device=DEV).to(torch.bfloat16)
    xbuf[:, :K] = x
    qw, sw = _weights(gpu_lib, N, K, "per_tensor", "e4m3", 4)
    _compare(gpu_lib, xbuf[:, :K], qw, sw, "per_tensor", gran_a=gran_a, what=f"strided x {gran_a}")


@pytest.mark.parametrize("packed", [False, True])
def test_kmajor_scales(gpu_lib, packed):
    """1x128 scales written K-block-major, as fp8_quantize(scale_layout="kmajor")
    writes them."""
    x = syn.activations(3, M=24, K=1024, variant=5).to(DEV)
    qw, sw = _weights(gpu_lib, 384, 1024, "block_128x128", "e4m3", 6, config=3)
    _compare(gpu_lib, x, qw, sw, "block_128x128", gran_a="group_1x128", packed=packed, scale_layout="kmajor",
             what="kmajor scales")


def test_outlier_rows_and_zero_groups(gpu_lib):
    """1x128 groups of very different magnitude in one fragment: a zero group
    (scale 0 path), a group with one huge outlier, a group of subnormal-scale
    values; each group's scale is its own."""
    M, N, K = 16, 256, 512
    x = syn.activations(3, M=M, K=K, variant=9).to(DEV).float()
    x[3, 128:256] = 0.0
    x[5, 300] = 2.5e4
    x[7, 0:128] *= 1e-30
    x[9, 384:512] = -x[9, 384:512].abs() * 1e6
    x = x.to(torch.bfloat16)
    qw, sw = _weights(gpu_lib, N, K, "block_128x128", "e4m3", 10, config=3)
    for packed in (False, True):
        _compare(gpu_lib, x, qw, sw, "block_128x128", gran_a="group_1x128", packed=packed,
                 what=f"mixed groups packed={packed}")


def test_config1_against_the_oracle(gpu_lib):
    """The 64x512x512 per-tensor configuration: codes and scale exactly as the
    oracle's per-tensor quantizer, C within the GEMM tolerance of the oracle's
    product on those codes."""
    c = syn.CONFIGS[1]
    x = syn.activations(1).to(DEV)
    w = syn.weights(1).to(DEV)
    qw, sw = gpu_lib.fp8_quantize(w, "per_tensor")
    y, q, s = gpu_lib.fp8_quantize_gemm_decode(x, qw, sw, "per_tensor", out_dtype=torch.float32, return_codes=True)
    x32 = f32_of(x.cpu())
    q_ref, s_ref = quant.quantize_per_tensor(x32)
    assert_scales_equal(s.cpu().numpy(), s_ref, "config 1 scale")
    assert_codes_equal(q.cpu().numpy(), q_ref, x32, "config 1 codes")
    y64, t = ogemm.block_gemm(q_ref, s_ref, "per_tensor", qw.cpu().numpy(), sw.cpu().numpy(), "per_tensor")
    check_gemm_tolerance(y.cpu().numpy(), y64, t, bf16=False, what="config 1 fused")
    assert y.shape == (c["M"], c["N"])


@pytest.mark.parametrize("packed", [False, True])
def test_decode_step_against_the_oracle(gpu_lib, packed):
    """The decode step 16x28672x8192 (1x128 activations, 128x128 weights) at
    full size, in the launch configuration the bench times: bit-identical to
    the two calls; codes and scales exactly as the oracle's 1x128 quantizer;
    C within the GEMM tolerance on 384 sampled columns (three 128-row weight
    blocks: the first, one in the middle and the last)."""
    c = syn.CONFIGS[3]
    M, N, K = c["M"], c["N"], c["K"]
    x = syn.activations(3).to(DEV)
    w = syn.weights(3).to(DEV)
    qw, sw = gpu_lib.fp8_quantize(w, "block_128x128")
    del w
    _compare(gpu_lib, x, qw, sw, "block_128x128", gran_a="group_1x128", packed=packed, scale_layout="kmajor",
             what=f"16x28672x8192 packed={packed}")
    w_arg = gpu_lib.fp8_pack_weights_decode(qw) if packed else qw
    y, q, s = gpu_lib.fp8_quantize_gemm_decode(x, w_arg, sw, "block_128x128", gran_a="group_1x128",
                                               out_dtype=torch.float32, return_codes=True)
    x32 = f32_of(x.cpu())
    q_ref, s_ref = quant.quantize_group_1x128(x32)
    assert_scales_equal(s.cpu().numpy(), s_ref, "decode step scales")
    assert_codes_equal(q.cpu().numpy(), q_ref, x32, "decode step codes")
    cols = np.concatenate([np.arange(0, 128), np.arange(N // 2, N // 2 + 128), np.arange(N - 128, N)])
    y64, t = ogemm.block_gemm(q_ref, s_ref, "group_1x128", qw.cpu().numpy(), sw.cpu().numpy(), "block_128x128",
                              cols=cols)
    check_gemm_tolerance(y.cpu().numpy()[:, cols], y64, t, bf16=False, what="decode step fused")
    assert y.shape == (M, N)


@pytest.mark.parametrize("gran_a", ["per_tensor", "group_1x128"])
@pytest.mark.parametrize("packed", [False, True])
def test_nonfinite_inputs_as_the_two_calls(gpu_lib, gran_a, packed):
    """NaN and infinities in x are outside the quantizers' contract (their
    codes are unspecified), but the one-launch call still returns normally
    and computes what the two calls compute: codes and scales bit for bit, C
    bit for bit wherever it is finite and non-finite in the same places."""
    M, N, K = 48, 256, 512
    x = syn.activations(3, M=M, K=K, variant=13).to(DEV).float()
    x[0, 5] = float("nan")
    x[9, 130] = float("inf")
    x[20, 300] = float("-inf")
    x = x.to(torch.bfloat16)
    qw, sw = _weights(gpu_lib, N, K, "block_128x128", "e4m3", 14, config=3)
    qw_packed = gpu_lib.fp8_pack_weights_decode(qw) if packed else None
    y, q, s = gpu_lib.fp8_quantize_gemm_decode(x, qw_packed if packed else qw, sw, "block_128x128", gran_a=gran_a,
                                               out_dtype=torch.float32, return_codes=True)
    y2, q2, s2 = _two_calls(gpu_lib, x, qw, sw, "block_128x128", gran_a, "e4m3", "e4m3", torch.float32, qw_packed,
                            "row")
    torch.cuda.synchronize()
    assert torch.equal(_bits(s), _bits(s2)), "scales differ"
    assert torch.equal(q, q2), "codes differ"
    fin = torch.isfinite(y2)
    assert torch.equal(torch.isfinite(y), fin), "non-finite outputs in different places"
    assert torch.equal(torch.isnan(y), torch.isnan(y2)), "NaN outputs in different places"
    assert torch.equal(_bits(torch.where(fin, y, 0.0)), _bits(torch.where(fin, y2, 0.0))), "finite outputs differ"
    if gran_a == "group_1x128":
        assert fin.sum() > 0, "every output non-finite: the clean groups were disturbed"
