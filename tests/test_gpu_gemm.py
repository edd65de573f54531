"""GPU parity of fp8_block_gemm against the CPU oracle.

The GPU GEMM runs on codes and scales (from the GPU quantizer, or random
codes), and the oracle computes y64 = A_hat . W_hat^T and T = |A_hat| . |W_hat|^T
in fp64 on the same codes. Acceptance: |y - y64| <= 1e-3 * T per element in
the fp32-output mode; the bf16 output is additionally allowed its own final
rounding (half a bf16 ulp) and must equal the bf16 rounding of the fp32-mode
output bit for bit. Full-size configurations are checked on sampled rows and
columns that include tile and scale-block edges.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import bf16_round_f32, check_gemm_tolerance, f32_of
from oracle import e4m3, gemm as ogemm

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_both(gpu_lib, qa, sa, ga, qw, sw, gw):
    y32 = gpu_lib.fp8_block_gemm(qa, sa, ga, qw, sw, gw, out_dtype=torch.float32)
    y16 = gpu_lib.fp8_block_gemm(qa, sa, ga, qw, sw, gw, out_dtype=torch.bfloat16)
    return y32, y16


def _compare(gpu_lib, qa, sa, ga, qw, sw, gw, rows=None, cols=None, what=""):
    y32, y16 = _run_both(gpu_lib, qa, sa, ga, qw, sw, gw)
    y32 = y32.cpu().numpy()
    y16 = f32_of(y16)
    # bf16 output is the bf16 rounding of the fp32-mode output, bit for bit
    assert np.array_equal(y16.view(np.uint32), bf16_round_f32(y32).view(np.uint32)), what + ": bf16 != bf16(fp32)"
    if rows is not None:
        y32 = y32[np.ix_(rows, cols)]
        y16 = y16[np.ix_(rows, cols)]
    y64, t = ogemm.block_gemm(qa.cpu().numpy(), sa.cpu().numpy(), ga, qw.cpu().numpy(), sw.cpu().numpy(),
                              gw, rows=rows, cols=cols)
    check_gemm_tolerance(y32, y64, t, bf16=False, what=what + " fp32")
    literal = check_gemm_tolerance(y16, y64, t, bf16=True, what=what + " bf16")
    return literal


def _quantized(gpu_lib, config, M=None, N=None, K=None, kmajor=False, variant=0):
    c = syn.CONFIGS[config]
    a = syn.activations(config, M=M, K=K, variant=variant).to(DEV)
    w = syn.weights(config, N=N, K=K, variant=variant).to(DEV)
    qa, sa = gpu_lib.fp8_quantize(a, c["gran_a"], scale_layout="kmajor" if kmajor else "row")
    qw, sw = gpu_lib.fp8_quantize(w, c["gran_w"])
    return qa, sa, c["gran_a"], qw, sw, c["gran_w"]


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 384, 512), (300, 512, 1024), (256, 256, 128),
                                   (513, 640, 384)])
def test_small_shapes_full_compare(gpu_lib, M, N, K):
    qa, sa, ga, qw, sw, gw = _quantized(gpu_lib, 2, M=M, N=N, K=K, variant=M)
    _compare(gpu_lib, qa, sa, ga, qw, sw, gw, what=f"{M}x{N}x{K}")


def test_kmajor_activation_scales(gpu_lib):
    qa, sa, ga, qw, sw, gw = _quantized(gpu_lib, 2, M=300, N=512, K=1024, kmajor=True, variant=3)
    assert sa.stride(0) == 1
    _compare(gpu_lib, qa, sa, ga, qw, sw, gw, what="kmajor")


@pytest.mark.parametrize("ga,gw", [("per_tensor", "block_128x128"), ("group_1x128", "per_tensor"),
                                   ("per_tensor", "per_tensor")])
def test_mixed_granularities(gpu_lib, ga, gw):
    a = syn.activations(2, M=200, K=640, variant=4).to(DEV)
    w = syn.weights(2, N=384, K=640, variant=4).to(DEV)
    qa, sa = gpu_lib.fp8_quantize(a, ga)
    qw, sw = gpu_lib.fp8_quantize(w, gw)
    _compare(gpu_lib, qa, sa, ga, qw, sw, gw, what=f"{ga}/{gw}")


def test_identity_weight_decodes_every_code(gpu_lib):
    """A holds all 254 finite codes; W is the identity (0x38 = 1.0) with unit
    scales, so the fp32 output must equal decode(A) * s_a exactly."""
    codes = e4m3.finite_codes()
    M, K = 4, 256
    qa = np.zeros((M, K), dtype=np.uint8)
    qa[0, :127] = codes[:127]
    qa[1, :127] = codes[127:]
    qa[2, 128:255] = codes[:127]
    qa[3, 128:255] = codes[127:]
    sa = np.ones((M, 2), dtype=np.float32)
    sa[1, 0] = 0.375
    qw = np.zeros((K, K), dtype=np.uint8)
    qw[np.arange(K), np.arange(K)] = 0x38
    sw = np.ones((2, 2), dtype=np.float32)
    y = gpu_lib.fp8_block_gemm(torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV), "group_1x128",
                               torch.from_numpy(qw).to(DEV), torch.from_numpy(sw).to(DEV), "block_128x128",
                               out_dtype=torch.float32).cpu().numpy()
    expect = e4m3.decode(qa) * np.repeat(sa, 128, axis=1)
    bad = np.argwhere(y != expect)
    assert bad.size == 0, f"first mismatch at {tuple(bad[0])}: code 0x{qa[tuple(bad[0])]:02x} gpu {y[tuple(bad[0])]} expect {expect[tuple(bad[0])]}"


def test_random_codes_and_scales(gpu_lib):
    """Uniformly random codes (every finite code, including +-448 and
    subnormals) with scales spread over 2^-12 .. 2^3."""
    rng = np.random.default_rng(301)
    M, N, K = 320, 384, 768
    def codes(shape):
        c = rng.integers(0, 256, size=shape)
        return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)
    qa, qw = codes((M, K)), codes((N, K))
    sa = (rng.uniform(0.5, 2, (M, K // 128)) * np.exp2(rng.integers(-12, 4, (M, K // 128)))).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N // 128, K // 128)) * np.exp2(rng.integers(-12, 4, (N // 128, K // 128)))).astype(np.float32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    _compare(gpu_lib, t(qa), t(sa), "group_1x128", t(qw), t(sw), "block_128x128", what="random codes")


def _sample(n, rng, extra):
    picks = set(int(i) for i in rng.choice(n, size=min(n, 96), replace=False))
    picks |= set(e for e in extra if 0 <= e < n)
    return np.array(sorted(picks))


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_config_full_size_sampled(gpu_lib, config):
    c = syn.CONFIGS[config]
    qa, sa, ga, qw, sw, gw = _quantized(gpu_lib, config)
    rng = np.random.default_rng(400 + config)
    M, N = c["M"], c["N"]
    rows = _sample(M, rng, [0, 1, 127, 128, 255, 256, M - 1])
    cols = _sample(N, rng, [0, 15, 16, 127, 128, 255, 256, 383, 511, N - 129, N - 128, N - 1])
    literal = _compare(gpu_lib, qa, sa, ga, qw, sw, gw, rows=rows, cols=cols, what=f"config {config}")
    print(f"config {config}: {literal} sampled bf16 outputs exceed the literal 1e-3*T bound (output rounding)")


def test_tail_balanced_grid(gpu_lib):
    """13 x 20 = 260 tiles of 256 x 256: on a 256-CU device the last 4 tiles
    run as 256 x 128 halves next to 256 full tiles. Sampled rows and columns
    cover the first, a middle and the last tiles (and both halves of these)."""
    M, N, K = 13 * 256, 20 * 256, 256
    qa, sa, ga, qw, sw, gw = _quantized(gpu_lib, 2, M=M, N=N, K=K, variant=7)
    rng = np.random.default_rng(77)
    rows = _sample(M, rng, [0, 255, 256, M - 257, M - 256, M - 129, M - 1])
    cols = _sample(N, rng, [0, 127, 128, 255, N - 257, N - 256, N - 129, N - 128, N - 1])
    _compare(gpu_lib, qa, sa, ga, qw, sw, gw, rows=rows, cols=cols, what="tail-balanced grid")
