"""fp8_kv_decode_attention_noalloc (the decode attention with the library's
fixed workspace, for callers that cannot allocate) against
fp8_kv_decode_attention with a caller-owned workspace: the same kernels, so
the outputs must be bit-identical. Two calls in a row, the second smaller
than the first (the fixed array keeps the first call's partials), in both
output types and both formats, through the C ABI; and the host-side
rejection of a call whose partials would not fit the fixed workspace."""

import ctypes

import pytest
import torch

import synth_inputs as syn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cache(gpu_lib, hkv, t, fmt, variant):
    k, v = syn.kv_pair(heads=hkv, tokens=t, head_dim=128, variant=variant)
    kc, ks = gpu_lib.fp8_kv_quantize(k.to(DEV), fmt=fmt)
    vc, vs = gpu_lib.fp8_kv_quantize(v.to(DEV), fmt=fmt)
    return kc, ks, vc, vs


def _noalloc(lib, q, kc, ks, vc, vs, fmt_id, scale, out, odt):
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    hq, d = q.shape
    hkv, t, _ = kc.shape
    return lib.fp8_kv_decode_attention_noalloc(P(q), q.stride(0), hq, hkv, t, d, P(kc), P(ks), P(vc), P(vs), 128,
                                               fmt_id, ctypes.c_float(scale), P(out), odt, out.stride(0),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_entry_point(gpu_lib, fmt, out_dtype):
    lib = gpu_lib.load_library()
    fmt_id = gpu_lib.E4M3 if fmt == "e4m3" else gpu_lib.E5M2
    odt = gpu_lib.F32 if out_dtype == torch.float32 else gpu_lib.BF16
    scale = 1.0 / 128 ** 0.5
    # first a large call, then a smaller one: 64 x 8 heads over 70000 tokens
    # (18 splits), then 12 x 3 heads over 5000 tokens (2 splits)
    for i, (hq, hkv, t) in enumerate(((64, 8, 70000), (12, 3, 5000))):
        kc, ks, vc, vs = _cache(gpu_lib, hkv, t, fmt, variant=20 + i)
        q = syn.decode_queries(heads_q=hq, variant=20 + i).to(DEV)
        ref = gpu_lib.fp8_kv_decode_attention(q, kc, ks, vc, vs, scale, fmt=fmt, out_dtype=out_dtype)
        out = torch.full((hq, 128), float("nan"), dtype=out_dtype, device=DEV)
        st = _noalloc(lib, q, kc, ks, vc, vs, fmt_id, scale, out, odt)
        assert st == gpu_lib.OK, lib.fp8blk_last_error().decode()
        torch.cuda.synchronize()
        view = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(view), ref.view(view)), f"call {i}: {hq}x{hkv}x{t} differs"
    # the binding's wrapper passes the same pointers
    out2 = torch.empty((hq, 128), dtype=out_dtype, device=DEV)
    gpu_lib.fp8_kv_decode_attention_noalloc(q, kc, ks, vc, vs, scale, out2, fmt=fmt)
    assert torch.equal(out2.view(view), ref.view(view))


def test_noalloc_rejects_partials_beyond_the_fixed_workspace(gpu_lib):
    """128 query heads over 266,113 tokens need 128 * 190 = 24320 split
    partials of 1408 tokens, more than the 24197 the 12 MiB array holds:
    refused on the host (no kernel runs, the output keeps its contents)."""
    lib = gpu_lib.load_library()
    hq, hkv, t = 128, 8, 189 * 1408 + 1
    assert lib.fp8_kv_decode_attention_workspace_size(hq, t) > 12 << 20
    kc = torch.zeros((hkv, t, 128), dtype=torch.uint8, device=DEV)
    ks = torch.zeros((hkv, (t + 127) // 128), dtype=torch.float32, device=DEV)
    q = torch.zeros((hq, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full((hq, 128), 7.0, dtype=torch.float32, device=DEV)
    st = _noalloc(lib, q, kc, ks, kc, ks, gpu_lib.E4M3, 0.1, out, gpu_lib.F32)
    assert st == gpu_lib.EUNSUPPORTED
    assert "fixed workspace" in lib.fp8blk_last_error().decode()
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
    # one split fewer fits: 128 heads over 189 * 1408 tokens
    assert lib.fp8_kv_decode_attention_workspace_size(hq, 189 * 1408) <= 12 << 20
