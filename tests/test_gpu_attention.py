"""GPU parity of fp8_kv_decode_attention against the CPU oracle.

The cache is written by the GPU quantizer (fp8_kv_quantize) and the oracle
attends over the same codes and scales in float64. Acceptance per output:
|o - o_ref| <= 1e-3 * T_o with T_o = sum_t p_t |v_hat_t| (the oracle's), plus
half a bf16 ulp for a bf16 output. Covers ragged token counts (1, a partial
32-token unit, a partial 352-token wave range, a partial 1408-token split,
several splits with a ragged last one, 129 splits),
1 to 16 query heads per kv head,
both FP8 formats, both output dtypes, and the full [8, 131072, 128] cache
with 64 query heads.
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import bf16_half_ulp, f32_of
from oracle import attention

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(gpu_lib, hq, hkv, t, fmt, out_dtype, variant, scale=None):
    k, v = syn.kv_pair(heads=hkv, tokens=t, head_dim=128, variant=variant)
    kc, ks = gpu_lib.fp8_kv_quantize(k.to(DEV), 128, fmt=fmt)
    vc, vs = gpu_lib.fp8_kv_quantize(v.to(DEV), 128, fmt=fmt)
    q = syn.decode_queries(heads_q=hq, variant=variant)
    c = 1.0 / np.sqrt(128) if scale is None else scale
    o = gpu_lib.fp8_kv_decode_attention(q.to(DEV), kc, ks, vc, vs, c, fmt=fmt, out_dtype=out_dtype)
    ref, t_o = attention.decode_attention(f32_of(q), kc.cpu().numpy(), ks.cpu().numpy(), vc.cpu().numpy(),
                                          vs.cpu().numpy(), np.float32(c), fmt)
    return f32_of(o).astype(np.float64), ref, t_o


def _check(got, ref, t_o, bf16, what):
    err = np.abs(got - ref)
    bound = 1e-3 * t_o + (bf16_half_ulp(np.maximum(np.abs(got), np.abs(ref))) if bf16 else 0.0)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} outputs out of tolerance; first at {tuple(bad[0])}: "
                           f"gpu {got[tuple(bad[0])]!r} oracle {ref[tuple(bad[0])]!r} T_o {t_o[tuple(bad[0])]!r}")
    return float((err / np.maximum(t_o, 1e-300)).max())


@pytest.mark.parametrize("t", [1, 31, 32, 33, 300, 351, 352, 353, 511, 513, 1025, 1407, 1408, 1409, 2047, 2048, 2049,
                               2816, 2817, 4096, 4097, 9000, 181000])
def test_token_counts(gpu_lib, t):
    got, ref, t_o = _run(gpu_lib, 8, 1, t, "e4m3", torch.float32, variant=t)
    _check(got, ref, t_o, False, f"T={t}")


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (16, 1), (12, 3), (64, 8)])
def test_query_groups(gpu_lib, hq, hkv):
    got, ref, t_o = _run(gpu_lib, hq, hkv, 1500, "e4m3", torch.float32, variant=hq)
    _check(got, ref, t_o, False, f"{hq}/{hkv}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_formats_and_outputs(gpu_lib, fmt, out_dtype):
    got, ref, t_o = _run(gpu_lib, 16, 2, 4100, fmt, out_dtype, variant=3)
    _check(got, ref, t_o, out_dtype == torch.bfloat16, f"{fmt} {out_dtype}")


def test_strided_query_and_output(gpu_lib):
    """q rows with a pitch of 256 elements whose other 128 hold NaN (never
    read) and an fp32 output with a pitch of 200 whose columns past 128 keep
    their sentinel."""
    hq, hkv, t = 16, 2, 3000
    k, v = syn.kv_pair(heads=hkv, tokens=t, head_dim=128, variant=31)
    kc, ks = gpu_lib.fp8_kv_quantize(k.to(DEV), 128)
    vc, vs = gpu_lib.fp8_kv_quantize(v.to(DEV), 128)
    q = syn.decode_queries(heads_q=hq, variant=31)
    qbuf = torch.full((hq, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    qbuf[:, :128] = q.to(DEV)
    obuf = torch.full((hq, 200), 7.0, dtype=torch.float32, device=DEV)
    c = 1.0 / np.sqrt(128)
    gpu_lib.fp8_kv_decode_attention(qbuf[:, :128], kc, ks, vc, vs, c, out=obuf[:, :128])
    ref, t_o = attention.decode_attention(f32_of(q), kc.cpu().numpy(), ks.cpu().numpy(), vc.cpu().numpy(),
                                          vs.cpu().numpy(), np.float32(c), "e4m3")
    _check(obuf[:, :128].cpu().numpy().astype(np.float64), ref, t_o, False, "strided q / out")
    assert bool(torch.all(obuf[:, 128:] == 7.0))


def test_peaked_softmax(gpu_lib):
    """A large softmax scale concentrates the weights on few tokens."""
    got, ref, t_o = _run(gpu_lib, 8, 1, 3000, "e4m3", torch.float32, variant=9, scale=0.8)
    _check(got, ref, t_o, False, "peaked")


def test_workspace_reuse_and_repeat(gpu_lib):
    """Two calls in a row on one workspace, the second with fewer tokens and
    another format, each match the oracle."""
    ws = torch.empty(gpu_lib.load_library().fp8_kv_decode_attention_workspace_size(16, 9000), dtype=torch.uint8,
                     device=DEV)
    for t, fmt in ((9000, "e4m3"), (777, "e5m2")):
        k, v = syn.kv_pair(heads=2, tokens=t, head_dim=128, variant=t)
        kc, ks = gpu_lib.fp8_kv_quantize(k.to(DEV), 128, fmt=fmt)
        vc, vs = gpu_lib.fp8_kv_quantize(v.to(DEV), 128, fmt=fmt)
        q = syn.decode_queries(heads_q=16, variant=t)
        o = gpu_lib.fp8_kv_decode_attention(q.to(DEV), kc, ks, vc, vs, 1 / np.sqrt(128), fmt=fmt,
                                            out_dtype=torch.float32, workspace=ws)
        ref, t_o = attention.decode_attention(f32_of(q), kc.cpu().numpy(), ks.cpu().numpy(), vc.cpu().numpy(),
                                              vs.cpu().numpy(), np.float32(1 / np.sqrt(128)), fmt)
        _check(f32_of(o).astype(np.float64), ref, t_o, False, f"repeat T={t}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_full_size_cache(gpu_lib, fmt):
    """The [8, 131072, 128] K and V cache with 64 query heads (8 per kv head)."""
    c = syn.CONFIGS[5]
    got, ref, t_o = _run(gpu_lib, c["heads_q"], c["heads"], c["tokens"], fmt, torch.bfloat16, variant=0)
    worst = _check(got, ref, t_o, True, f"full {fmt}")
    print(f"full-size {fmt}: max |err| / T_o = {worst:.3e}")
