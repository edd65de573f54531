"""GPU parity of fp8_kv_quantize / fp8_kv_dequantize against the CPU oracle.

Codes, scales and the dequantized bf16 values are compared bit-exactly: in
full on small caches (ragged token counts, head_dim 64/128/256, a strided
cache view), and in full on the [8, 131072, 128] K and V tensors.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, assert_scales_equal, f32_of, pmap
from oracle import quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_full(gpu_lib, kv: torch.Tensor, token_block: int):
    x32 = f32_of(kv)
    qr, sr = quant.kv_quantize(x32, token_block)
    qg, sg = gpu_lib.fp8_kv_quantize(kv, token_block)
    assert_scales_equal(sg.cpu().numpy(), sr, "kv scales")
    assert_codes_equal(qg.cpu().numpy(), qr, x32, "kv codes")
    out = gpu_lib.fp8_kv_dequantize(qg, sg, token_block)
    ref = quant.kv_dequantize(qr, sr, token_block)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"dequant mismatch at {tuple(bad[0])}: gpu 0x{got[tuple(bad[0])]:04x} oracle 0x{ref[tuple(bad[0])]:04x}"


@pytest.mark.parametrize("heads,tokens,head_dim,token_block", [
    (1, 1, 8, 128), (3, 1000, 128, 128), (2, 4096, 128, 128), (2, 777, 64, 128),
    (1, 640, 256, 64), (4, 300, 128, 32),
])
def test_small_caches_full_compare(gpu_lib, heads, tokens, head_dim, token_block):
    k, v = syn.kv_pair(heads=heads, tokens=tokens, head_dim=head_dim, variant=1)
    _check_full(gpu_lib, k.to(DEV), token_block)
    _check_full(gpu_lib, v.to(DEV), token_block)


def test_strided_cache_view(gpu_lib):
    """K and V interleaved in one [heads, tokens, 2, head_dim] cache: each is a
    view with stride_token = 2 * head_dim."""
    k, v = syn.kv_pair(heads=2, tokens=520, head_dim=128, variant=2)
    cache = torch.stack([k, v], dim=2).to(DEV)
    for i in range(2):
        view = cache[:, :, i, :]
        assert view.stride(1) == 256
        _check_full(gpu_lib, view, 128)


def test_zero_and_tiny_blocks(gpu_lib):
    kv = torch.zeros((2, 384, 128), dtype=torch.bfloat16)
    kv[0, 128:256] = -0.0
    kv[1, 0:128] = torch.tensor(2.0 ** -133, dtype=torch.bfloat16)
    kv[1, 256:384, 5] = -7.0
    _check_full(gpu_lib, kv.to(DEV), 128)


@pytest.mark.parametrize("which", ["K", "V"])
def test_config5_full_size(gpu_lib, which):
    """Every code, scale and dequantized value of the full [8, 131072, 128]
    K or V tensor; the oracle runs one head per host thread."""
    k, v = syn.kv_pair(5)
    x = k if which == "K" else v
    del k, v
    tb = 128
    qg, sg = gpu_lib.fp8_kv_quantize(x.to(DEV), tb)
    out = gpu_lib.fp8_kv_dequantize(qg, sg, tb)
    qg, sg = qg.cpu().numpy(), sg.cpu().numpy()
    out = out.cpu().view(torch.int16).numpy().view(np.uint16)
    x32 = f32_of(x)
    del x

    def head(h):
        qr, sr = quant.kv_quantize(x32[h:h + 1], tb)
        return qr, sr, quant.kv_dequantize(qr, sr, tb)

    ref = pmap(head, range(x32.shape[0]))
    for h, (qr, sr, dr) in enumerate(ref):
        assert_scales_equal(sg[h:h + 1], sr, f"{which} scales, head {h}")
        assert_codes_equal(qg[h:h + 1], qr, x32[h:h + 1], f"{which} codes, head {h}")
        bad = np.argwhere(out[h:h + 1] != dr)
        assert bad.size == 0, f"{which} dequant, head {h}: {len(bad)} mismatches, first at {tuple(bad[0])}"
