"""GPU parity of fp8_block_gemm_quant (the GEMM with its output quantized in
the epilogue) against the CPU oracle.

The fused kernel's codes and scales must equal, bit for bit, the oracle's
1 x 128 quantization ([FP8] section "激活动态量化") of the same GEMM's fp32
output (fp8_block_gemm in fp32 mode on the prefill kernel, whose accumulators
are the same registers, so the quantization decision is taken on identical
fp32 values on both sides; for M <= 64 the reference product is taken with A
padded to 65 rows, because fp8_block_gemm runs its decode kernel there); the
fp32 output itself is held to the GEMM tolerance against the fp64 oracle by
tests/test_gpu_gemm.py and again here.

Covers: ragged M (including M <= 64, which the fused path runs on the
prefill kernel), both output formats and both input formats, both scale
layouts, the tail-balanced grid, a full-size configuration on sampled rows,
and a two-GEMM chain whose second GEMM reads the fused output directly.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, assert_scales_equal, check_gemm_tolerance
from oracle import gemm as ogemm, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _operands(gpu_lib, M, N, K, variant, fa="e4m3", fw="e4m3"):
    a = syn.activations(2, M=M, K=K, variant=variant).to(DEV)
    w = syn.weights(2, N=N, K=K, variant=variant).to(DEV)
    qa, sa = gpu_lib.fp8_quantize(a, "group_1x128", fmt=fa, scale_layout="kmajor")
    qw, sw = gpu_lib.fp8_quantize(w, "block_128x128", fmt=fw)
    return qa, sa, qw, sw


def _check(gpu_lib, qa, sa, qw, sw, fc, fa="e4m3", fw="e4m3", layout="kmajor", rows=None, what=""):
    qc, sc = gpu_lib.fp8_block_gemm_quant(qa, sa, "group_1x128", qw, sw, "block_128x128", fmt_c=fc,
                                          fmt_a=fa, fmt_w=fw, scale_layout=layout)
    M = qa.shape[0]
    if M > 64:
        y32 = gpu_lib.fp8_block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128", out_dtype=torch.float32,
                                     fmt_a=fa, fmt_w=fw).cpu().numpy()
    else:
        # fp8_block_gemm takes its split-K decode kernel for M <= 64 (another
        # summation order); the fused path always runs the prefill kernel,
        # whose rows do not depend on M: pad A with zero rows past 64
        qp = torch.zeros((65, qa.shape[1]), dtype=torch.uint8, device=DEV)
        qp[:M] = qa
        sp = torch.ones((qa.shape[1] // 128, 65), dtype=torch.float32, device=DEV).t()
        sp[:M] = sa
        y32 = gpu_lib.fp8_block_gemm(qp, sp, "group_1x128", qw, sw, "block_128x128", out_dtype=torch.float32,
                                     fmt_a=fa, fmt_w=fw).cpu().numpy()[:M]
    qc = qc.cpu().numpy()
    sc = sc.cpu().numpy()
    if rows is not None:
        y32, qc, sc = y32[rows], qc[rows], sc[rows]
    qr, sr = quant.quantize_group_1x128(y32, fc)
    assert_scales_equal(sc, sr, what + " scales")
    assert_codes_equal(qc, qr, y32, what + " codes")
    return y32


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (40, 256, 384), (300, 512, 640), (513, 384, 256)])
@pytest.mark.parametrize("fc", ["e4m3", "e5m2"])
def test_small_shapes(gpu_lib, M, N, K, fc):
    qa, sa, qw, sw = _operands(gpu_lib, M, N, K, variant=M + 1)
    y32 = _check(gpu_lib, qa, sa, qw, sw, fc, what=f"{M}x{N}x{K} {fc}")
    y64, t = ogemm.block_gemm(qa.cpu().numpy(), sa.cpu().numpy(), "group_1x128", qw.cpu().numpy(),
                              sw.cpu().numpy(), "block_128x128")
    check_gemm_tolerance(y32, y64, t, bf16=False, what="fp32 product")


@pytest.mark.parametrize("fa,fw", [("e5m2", "e4m3"), ("e4m3", "e5m2")])
def test_mixed_input_formats(gpu_lib, fa, fw):
    qa, sa, qw, sw = _operands(gpu_lib, 200, 384, 512, variant=5, fa=fa, fw=fw)
    _check(gpu_lib, qa, sa, qw, sw, "e4m3", fa=fa, fw=fw, what=f"{fa}x{fw}")


def test_row_major_scale_layout(gpu_lib):
    qa, sa, qw, sw = _operands(gpu_lib, 300, 512, 256, variant=6)
    _check(gpu_lib, qa, sa, qw, sw, "e4m3", layout="row", what="row-major scales")


def test_tail_balanced_grid(gpu_lib):
    """13 x 20 tiles: the last 4 tiles run as 256 x 128 halves on a 256-CU
    device; every row is checked over all columns."""
    M, N, K = 13 * 256, 20 * 256, 256
    qa, sa, qw, sw = _operands(gpu_lib, M, N, K, variant=7)
    rng = np.random.default_rng(91)
    rows = np.unique(np.concatenate([rng.choice(M, 200, replace=False), [0, 255, 256, M - 257, M - 1]]))
    _check(gpu_lib, qa, sa, qw, sw, "e4m3", rows=rows, what="tail-balanced")


def test_full_size_config_sampled_rows(gpu_lib):
    c = syn.CONFIGS[2]
    M, N, K = c["M"], c["N"], c["K"]
    qa, sa, qw, sw = _operands(gpu_lib, M, N, K, variant=0)
    rng = np.random.default_rng(92)
    rows = np.unique(np.concatenate([rng.choice(M, 128, replace=False), [0, 1, 255, 256, M - 1]]))
    _check(gpu_lib, qa, sa, qw, sw, "e4m3", rows=rows, what="4096x14336x4096")


def test_chain_feeds_the_next_gemm(gpu_lib):
    """GEMM 1 writes quantized codes and K-block-major scales; GEMM 2 reads them
    as its activations unchanged, and its output meets the GEMM tolerance
    against the oracle on those same codes."""
    M, K1, N1, N2 = 320, 512, 768, 384
    qa, sa, qw1, sw1 = _operands(gpu_lib, M, N1, K1, variant=8)
    h, sh = gpu_lib.fp8_block_gemm_quant(qa, sa, "group_1x128", qw1, sw1, "block_128x128")
    w2 = syn.weights(2, N=N2, K=N1, variant=9).to(DEV)
    qw2, sw2 = gpu_lib.fp8_quantize(w2, "block_128x128")
    y = gpu_lib.fp8_block_gemm(h, sh, "group_1x128", qw2, sw2, "block_128x128", out_dtype=torch.float32)
    y64, t = ogemm.block_gemm(h.cpu().numpy(), sh.cpu().numpy(), "group_1x128", qw2.cpu().numpy(),
                              sw2.cpu().numpy(), "block_128x128")
    check_gemm_tolerance(y.cpu().numpy(), y64, t, bf16=False, what="chained GEMM")
