"""GPU parity of the decode-packed weight path: fp8_pack_weights_decode and
fp8_block_gemm_packed.

The pack is a pure reordering of bytes, checked bit for bit against the
layout written out with NumPy index arithmetic (the definition in
include/fp8blk.h). The packed GEMM must equal fp8_block_gemm on the row-major
codes bit for bit (same kernel, same summation order) and, like it, meet the
oracle's tolerance |y - y64| <= 1e-3 * T per element.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import check_gemm_tolerance, f32_of
from oracle import gemm as ogemm

pytestmark = pytest.mark.gpu
DEV = "cuda"


def packed_reference(w: np.ndarray) -> np.ndarray:
    """Byte h * 1024 + 16 l + e of block (kb, rg) holds w[16 rg + l % 16][128 kb + 32 (l // 16) + 16 h + e]."""
    N, K = w.shape
    out = np.empty((K // 128, N // 16, 2048), dtype=np.uint8)
    h = np.arange(2)[:, None, None]
    l = np.arange(64)[None, :, None]
    e = np.arange(16)[None, None, :]
    pos = (h * 1024 + l * 16 + e).reshape(-1)
    for kb in range(K // 128):
        for rg in range(N // 16):
            rows = 16 * rg + (l % 16) + 0 * h + 0 * e
            cols = 128 * kb + 32 * (l // 16) + 16 * h + e
            out[kb, rg, pos] = w[rows.reshape(-1), cols.reshape(-1)]
    return out


def _codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 256, shape, dtype=torch.uint8, generator=g)
    # no NaN codes (S.1111.111 in E4M3): the GEMM takes finite codes only
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


@pytest.mark.parametrize("N,K,pad", [(128, 128, 0), (256, 384, 0), (384, 256, 48), (1024, 1024, 0)])
def test_pack_layout_bit_exact(gpu_lib, N, K, pad):
    w = _codes((N, K + pad), seed=N + K + pad)
    wd = w.to(DEV)[:, :K]                       # row stride K + pad
    got = gpu_lib.fp8_pack_weights_decode(wd).cpu().numpy()
    ref = packed_reference(w[:, :K].numpy())
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def _quantized(gpu_lib, M, N, K, variant, kmajor=True, fmt_a="e4m3", fmt_w="e4m3"):
    a = syn.activations(3, M=M, K=K, variant=variant).to(DEV)
    w = syn.weights(3, N=N, K=K, variant=variant).to(DEV)
    qa, sa = gpu_lib.fp8_quantize(a, "group_1x128", scale_layout="kmajor" if kmajor else "row", fmt=fmt_a)
    qw, sw = gpu_lib.fp8_quantize(w, "block_128x128", fmt=fmt_w)
    return qa, sa, qw, sw


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 256, 384), (16, 384, 1024), (17, 256, 512),
                                   (33, 512, 256), (64, 640, 768)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_packed_equals_row_major_and_oracle(gpu_lib, M, N, K, out_dtype):
    qa, sa, qw, sw = _quantized(gpu_lib, M, N, K, variant=M + N)
    packed = gpu_lib.fp8_pack_weights_decode(qw)
    y_p = gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", packed, sw, "block_128x128", out_dtype=out_dtype)
    y_r = gpu_lib.fp8_block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128", out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y_p.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                       y_r.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    y64, t = ogemm.block_gemm(qa.cpu().numpy(), sa.cpu().numpy(), "group_1x128", qw.cpu().numpy(),
                              sw.cpu().numpy(), "block_128x128")
    check_gemm_tolerance(f32_of(y_p), y64, t, bf16=out_dtype == torch.bfloat16, what=f"packed {M}x{N}x{K}")


@pytest.mark.parametrize("fmt_a,fmt_w", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
def test_packed_formats_and_row_scales(gpu_lib, fmt_a, fmt_w):
    M, N, K = 24, 384, 640
    qa, sa, qw, sw = _quantized(gpu_lib, M, N, K, variant=7, kmajor=False, fmt_a=fmt_a, fmt_w=fmt_w)
    packed = gpu_lib.fp8_pack_weights_decode(qw)
    kw = dict(out_dtype=torch.float32, fmt_a=fmt_a, fmt_w=fmt_w)
    y_p = gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", packed, sw, "block_128x128", **kw)
    y_r = gpu_lib.fp8_block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128", **kw)
    assert torch.equal(y_p.view(torch.int32), y_r.view(torch.int32))
    y64, t = ogemm.block_gemm(qa.cpu().numpy(), sa.cpu().numpy(), "group_1x128", qw.cpu().numpy(),
                              sw.cpu().numpy(), "block_128x128", fmt_a=fmt_a, fmt_w=fmt_w)
    check_gemm_tolerance(f32_of(y_p), y64, t, bf16=False, what=f"packed {fmt_a} x {fmt_w}")


def test_packed_per_tensor_scales(gpu_lib):
    M, N, K = 8, 256, 512
    a = syn.activations(3, M=M, K=K, variant=3).to(DEV)
    w = syn.weights(3, N=N, K=K, variant=3).to(DEV)
    qa, sa = gpu_lib.fp8_quantize(a, "per_tensor")
    qw, sw = gpu_lib.fp8_quantize(w, "per_tensor")
    packed = gpu_lib.fp8_pack_weights_decode(qw)
    y_p = gpu_lib.fp8_block_gemm_packed(qa, sa, "per_tensor", packed, sw, "per_tensor", out_dtype=torch.float32)
    y_r = gpu_lib.fp8_block_gemm(qa, sa, "per_tensor", qw, sw, "per_tensor", out_dtype=torch.float32)
    assert torch.equal(y_p.view(torch.int32), y_r.view(torch.int32))


def test_packed_full_decode_shape(gpu_lib):
    """16 x 28672 x 8192 (70B-style MLP up, one decode step): bit-identical to
    the row-major path, which the decode tests check against the oracle."""
    c = syn.CONFIGS[3]
    M, N, K = c["M"], c["N"], c["K"]
    qa, sa, qw, sw = _quantized(gpu_lib, M, N, K, variant=0)
    packed = gpu_lib.fp8_pack_weights_decode(qw)
    y_p = gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", packed, sw, "block_128x128")
    y_r = gpu_lib.fp8_block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128")
    assert torch.equal(y_p.view(torch.int16), y_r.view(torch.int16))
    # and a sample of columns against the oracle, including row-group and scale-block edges
    cols = np.array([0, 15, 16, 127, 128, 4095, 4096, N - 129, N - 1])
    y64, t = ogemm.block_gemm(qa.cpu().numpy(), sa.cpu().numpy(), "group_1x128", qw.cpu().numpy(),
                              sw.cpu().numpy(), "block_128x128", rows=np.arange(M), cols=cols)
    check_gemm_tolerance(f32_of(y_p)[:, cols], y64, t, bf16=True, what="packed full decode")


def test_packed_rejects_prefill_m(gpu_lib):
    qa, sa, qw, sw = _quantized(gpu_lib, 65, 128, 128, variant=1)
    packed = gpu_lib.fp8_pack_weights_decode(qw)
    with pytest.raises(gpu_lib.Fp8BlkError) as e:
        gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", packed, sw, "block_128x128")
    assert e.value.status == 3


def test_binding_rejects_column_strided_codes(gpu_lib):
    """The C ABI takes a base pointer and a row stride: the binding refuses
    views whose rows are not contiguous, and codes that are not uint8."""
    qa, sa, qw, sw = _quantized(gpu_lib, 16, 256, 256, variant=2)
    with pytest.raises(ValueError):
        gpu_lib.fp8_block_gemm(qa, sa, "group_1x128", qw.t(), sw, "block_128x128")
    with pytest.raises(ValueError):
        gpu_lib.fp8_pack_weights_decode(qw.t())
    with pytest.raises(ValueError):
        gpu_lib.fp8_block_gemm(qa.to(torch.int16), sa, "group_1x128", qw, sw, "block_128x128")
    packed = gpu_lib.fp8_pack_weights_decode(qw)
    out = torch.empty((256, 16), dtype=torch.bfloat16, device=DEV).t()
    with pytest.raises(ValueError):
        gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", packed, sw, "block_128x128", out=out)


def test_pack_past_4_gib(gpu_lib):
    """N x K = 40960 x 131072 codes (5 GiB): more 16-byte chunks than the
    packing kernel's capped grid covers in one pass (2^20 workgroups x 256
    threads = 4 GiB), so its threads loop. 2 KB blocks on both sides of the
    4 GiB boundary, and the last one, are compared byte for byte with the
    layout built from the row-major codes by index arithmetic."""
    N, K = 40960, 131072
    assert N * K > (1 << 32)
    g = torch.Generator(device=DEV).manual_seed(11)
    qw = torch.randint(0, 256, (N, K), dtype=torch.uint8, device=DEV, generator=g)
    try:
        packed = gpu_lib.fp8_pack_weights_decode(qw).view(-1)
        torch.cuda.synchronize()
        rg_count = N // 16
        first_past = (1 << 32) // 2048            # the first block at or past byte 2^32
        blocks = sorted(set([0, 1, first_past - 1, first_past, first_past + 1, N * K // 2048 - 1] +
                            [int(b) for b in np.random.default_rng(12).integers(0, N * K // 2048, 24)]))
        for b in blocks:
            kb, rg = divmod(b, rg_count)
            w = qw[16 * rg:16 * rg + 16, 128 * kb:128 * kb + 128].reshape(16, 4, 2, 16)   # [r, g, h, e]
            expect = w.permute(2, 1, 0, 3).reshape(-1)                                     # h, l = r + 16 g, e
            got = packed[b * 2048:(b + 1) * 2048]
            assert torch.equal(got, expect), f"block {b} (kb {kb}, rg {rg}) differs"
    finally:
        del qw
        torch.cuda.empty_cache()
