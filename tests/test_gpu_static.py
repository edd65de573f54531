"""GPU parity of static / delayed scaling against the CPU oracle.

fp8_quantize_static casts with a caller-supplied scale (charles2530.github.io
"量化：FP8 与混合精度推理", section "scale 是控制面"; api.makesence.top section 2,
delayed scaling) and records the tensor's amax; fp8_scale_from_amax_history
turns a window of recorded amax values into the next scale. Codes, the
recorded amax and the history scale are compared bit for bit with
oracle.quant.quantize_static / scale_from_history on the same fp32 inputs
(bf16 inputs converted exactly) and the same fp32 scale.

Covers: ragged shapes in both input dtypes and formats; shapes that move a
workgroup's amax slot or leave a workgroup without one; scales that leave
headroom, that saturate most of the tensor, powers of two, values next to
2^-126 and 2^125 (where the kernel changes method) and the largest finite
float; every bf16 magnitude below sampled patterns; a zero scale; empty
tensors (amax 0); repeated calls on one amax buffer; a delayed-scaling loop
over several steps whose scales come from the GPU's own history; the full
4096 x 4096 activation tensor (sampled rows, exact amax).
"""

import numpy as np
import pytest
import torch

import synth_inputs as syn
from gpu_helpers import assert_codes_equal, assert_scales_equal, f32_of
from oracle import quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _padded(x32, dtype, rows, cols):
    ld = (cols + 15) // 16 * 16
    buf = torch.full((rows, max(ld, 16)), float("nan"), dtype=dtype)
    buf[:, :cols] = torch.from_numpy(x32).to(dtype)
    return buf.to(DEV)[:, :cols]


def _check(gpu_lib, x32, dtype, fmt, s, what, record=True):
    rows, cols = x32.shape
    xt = _padded(x32, dtype, rows, cols)
    xr = f32_of(xt)
    st = torch.tensor([s], dtype=torch.float32, device=DEV)
    got = gpu_lib.fp8_quantize_static(xt, st, fmt, record_amax=record)
    qg, ag = got if record else (got, None)
    qr, ar = quant.quantize_static(xr, np.float32(s), fmt)
    assert_codes_equal(qg.cpu().numpy(), qr, xr, what)
    if record:
        assert_scales_equal(ag.cpu().numpy(), np.array([ar], np.float32), what + " amax")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (5, 130), (64, 1000), (300, 4096)])
def test_shapes(gpu_lib, fmt, dtype, rows, cols):
    rng = np.random.default_rng(rows * 31 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-8, 8, size=(rows, 1)))).astype(np.float32)
    amax = float(np.abs(x).max())
    for mult in (1.0, 1.7, 0.05):            # exact dynamic scale, headroom, most elements saturated
        s = np.float32(amax / quant.FORMAT_MAX[fmt] * mult)
        _check(gpu_lib, x, dtype, fmt, s, f"{rows}x{cols} {fmt} s*{mult}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols,peak", [(205, 33, (204, 32)), (410, 33, (204, 32)), (411, 33, (410, 32)),
                                            (3, 2, (2, 1)), (1000, 3, (999, 2)), (1, 4, (0, 3)), (2, 1029, (1, 1028))])
def test_amax_record_geometry(gpu_lib, dtype, rows, cols, peak):
    """Shapes where a workgroup's first chunk is a short row end (its amax slot
    moves to the next chunk), where the last workgroup holds one short chunk
    and no slot, and tensors narrower than 4 columns; the largest element sits
    in that chunk. Codes around every slot must be restored."""
    rng = np.random.default_rng(rows * 3 + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[peak] = -50.0
    _check(gpu_lib, x, dtype, "e4m3", np.float32(0.05), f"{rows}x{cols}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("s", [2.0 ** -3, 1.0, 2.0 ** 20, float.fromhex("0x1.fffffcp-127"), 2.0 ** -126,
                               float.fromhex("0x1.000002p-126"), 1e-45, 2.0 ** 125, float.fromhex("0x1.000002p125"),
                               2.0 ** 126, 3.0e38, 3.4028235e38, 0.0])
def test_scale_values(gpu_lib, fmt, s):
    """Scales across the whole fp32 range, including both sides of the
    thresholds where the kernel leaves the reciprocal bracket for the exact
    division, and inputs across the whole range."""
    rng = np.random.default_rng(7)
    x = (rng.uniform(-1, 1, size=(64, 256)) * np.exp2(rng.uniform(-149, 128, size=(64, 256)))).astype(np.float32)
    x[np.isinf(x)] = 3.0e38
    _check(gpu_lib, x, torch.float32, fmt, np.float32(s), f"s={s!r}")


def test_every_bf16_magnitude(gpu_lib):
    """Every positive bf16 value up to 0x7F7F with alternating signs, under
    scales that put the quotients across the E4M3 and E5M2 ranges."""
    bits = np.arange(0, 0x7F80, dtype=np.int64)
    bits = (bits | ((bits & 1) << 15)).astype(np.uint16)
    x = quant.bf16_bits_to_f32(bits).reshape(-1, 128)
    for fmt, s in (("e4m3", 2.0 ** -130), ("e4m3", 0.37), ("e4m3", 7.0e35), ("e5m2", 1.1e-30), ("e5m2", 2.0 ** 90)):
        _check(gpu_lib, x, torch.bfloat16, fmt, np.float32(s), f"every bf16 {fmt} s={s!r}")


def test_empty_and_unrecorded(gpu_lib):
    st = torch.ones(1, dtype=torch.float32, device=DEV)
    amax = torch.full((1,), 5.0, device=DEV)
    q, a = gpu_lib.fp8_quantize_static(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), st,
                                       record_amax=True, amax=amax)
    assert q.shape == (0, 64) and float(a.item()) == 0.0
    x = np.random.default_rng(8).standard_normal((9, 40)).astype(np.float32)
    _check(gpu_lib, x, torch.bfloat16, "e4m3", np.float32(0.01), "no amax", record=False)


def test_repeated_calls_reset_amax(gpu_lib):
    """A second, smaller call on the same amax buffer records its own amax,
    not the max of both."""
    amax = torch.empty(1, dtype=torch.float32, device=DEV)
    st = torch.tensor([0.5], device=DEV)
    for scale in (100.0, 0.25):
        x = (np.random.default_rng(9).standard_normal((128, 512)) * scale).astype(np.float32)
        _, a = gpu_lib.fp8_quantize_static(torch.from_numpy(x).to(DEV), st, record_amax=True, amax=amax)
        assert_scales_equal(a.cpu().numpy(), np.array([np.abs(x).max()], np.float32), f"amax {scale}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("n", [1, 7, 256, 1000, 100003])
def test_history_scale(gpu_lib, fmt, n):
    rng = np.random.default_rng(n)
    h = np.abs(rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, size=n))).astype(np.float32)
    got = gpu_lib.fp8_scale_from_amax_history(torch.from_numpy(h).to(DEV), fmt)
    assert_scales_equal(got.cpu().numpy(), np.array([quant.scale_from_history(h, fmt)], np.float32), f"n={n}")


def test_delayed_scaling_loop(gpu_lib):
    """Eight steps of delayed scaling on the GPU: each step quantizes with the
    scale of the last 4 recorded amax values (a first scale of 1) and appends
    its own amax; the oracle runs the same loop on the CPU."""
    rng = np.random.default_rng(10)
    hist_g = torch.zeros(4, dtype=torch.float32, device=DEV)
    hist_r = np.zeros(4, np.float32)
    s_g = torch.ones(1, dtype=torch.float32, device=DEV)
    s_r = np.float32(1.0)
    for step in range(8):
        x = (rng.standard_normal((256, 1024)) * (1 + 3 * step)).astype(np.float32)
        xt = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
        xr = f32_of(xt)
        qg, ag = gpu_lib.fp8_quantize_static(xt, s_g, record_amax=True, amax=hist_g[step % 4:step % 4 + 1])
        qr, ar = quant.quantize_static(xr, s_r)
        hist_r[step % 4] = ar
        assert_codes_equal(qg.cpu().numpy(), qr, xr, f"step {step}")
        assert_scales_equal(hist_g.cpu().numpy(), hist_r, f"history after step {step}")
        gpu_lib.fp8_scale_from_amax_history(hist_g, out=s_g)
        s_r = quant.scale_from_history(hist_r)
        assert_scales_equal(s_g.cpu().numpy(), np.array([s_r], np.float32), f"scale after step {step}")


def test_full_size_activations(gpu_lib):
    a = syn.activations(2)
    amax = float(a.float().abs().max())
    s = torch.tensor([amax / 448.0 * 1.25], dtype=torch.float32)
    q, ag = gpu_lib.fp8_quantize_static(a.to(DEV), s.to(DEV), record_amax=True)
    rows = np.random.default_rng(11).choice(a.shape[0], 48, replace=False)
    qr, _ = quant.quantize_static(a[rows].float().numpy(), s.numpy()[0])
    assert_codes_equal(q.cpu().numpy()[rows], qr, a[rows].float().numpy(), "full size")
    assert float(ag.item()) == amax
