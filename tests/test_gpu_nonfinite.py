"""Non-finite inputs are outside the quantizers' contract (their codes are
unspecified) but must not crash a kernel or disturb other groups: each call
returns normally, and every group (or, under a supplied scale, every element)
free of NaN and infinity still matches the oracle bit for bit."""

import numpy as np
import pytest
import torch

from gpu_helpers import assert_codes_equal, assert_scales_equal
from oracle import mx, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _input():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[0, 5] = np.nan
    x[1, 130] = np.inf
    x[2, 300] = -np.inf
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return xb.to(DEV), xb.float().numpy()


def test_group_and_block_scales(gpu_lib):
    xd, x = _input()
    bad = ~np.isfinite(x)
    q, s = gpu_lib.fp8_quantize(xd, "group_1x128")
    q, s = q.cpu().numpy(), s.cpu().numpy()
    clean = ~bad.reshape(64, 4, 128).any(axis=2)
    assert clean.sum() == 64 * 4 - 3
    xz = np.where(bad, 0, x)
    qr, sr = quant.quantize_group_1x128(xz)
    for r, g in zip(*np.nonzero(clean)):
        sl = slice(128 * g, 128 * g + 128)
        assert_scales_equal(s[r, g:g + 1], sr[r, g:g + 1], f"group ({r},{g})")
        assert_codes_equal(q[r, sl], qr[r, sl], x[r, sl], f"group ({r},{g})")
    q, s = gpu_lib.fp8_quantize(xd, "block_128x128")
    qr, sr = quant.quantize_block_128x128(xz[:, 384:])
    assert_scales_equal(s.cpu().numpy()[:, 3:], sr, "clean block scale")
    assert_codes_equal(q.cpu().numpy()[:, 384:], qr, x[:, 384:], "clean block codes")
    gpu_lib.fp8_quantize(xd, "per_tensor")           # unspecified result; must return
    torch.cuda.synchronize()


def test_static_scale_elementwise(gpu_lib):
    xd, x = _input()
    s = torch.tensor([0.01], device=DEV)
    q, _ = gpu_lib.fp8_quantize_static(xd, s, record_amax=True)
    q = q.cpu().numpy()
    ok = np.isfinite(x)
    qr, _ = quant.quantize_static(np.where(ok, x, 0), np.float32(0.01))
    assert np.array_equal(q[ok], qr[ok])


def test_mx_blocks(gpu_lib):
    xd, x = _input()
    q, sb = gpu_lib.fp8_quantize_mx(xd)
    q, sb = q.cpu().numpy(), sb.cpu().numpy()
    bad = ~np.isfinite(x).reshape(64, 16, 32).all(axis=2)
    qr, sr = mx.quantize_mx(np.where(np.isfinite(x), x, 0))
    assert np.array_equal(sb[~bad], sr[~bad])
    keep = np.repeat(~bad, 32, axis=1)
    assert np.array_equal(q[keep], qr[keep])


def test_kv_groups(gpu_lib):
    rng = np.random.default_rng(42)
    kv = rng.standard_normal((2, 300, 128)).astype(np.float32)
    kv[1, 140, 7] = np.nan
    kvb = torch.from_numpy(kv).to(torch.bfloat16)
    kv = kvb.float().numpy()
    q, s = gpu_lib.fp8_kv_quantize(kvb.to(DEV))
    q, s = q.cpu().numpy(), s.cpu().numpy()
    qr, sr = quant.kv_quantize(np.where(np.isfinite(kv), kv, 0))
    for h in range(2):
        for b in range(3):
            if (h, b) == (1, 1):
                continue
            sl = slice(128 * b, min(128 * b + 128, 300))
            assert_scales_equal(s[h, b:b + 1], sr[h, b:b + 1], f"kv ({h},{b})")
            assert np.array_equal(q[h, sl], qr[h, sl]), f"kv ({h},{b})"
    back = gpu_lib.fp8_kv_dequantize(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    assert back.shape == (2, 300, 128)
