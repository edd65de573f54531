"""Shared helpers for the GPU parity tests (comparison and reporting only)."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import quant

# Host threads for running the oracle on independent pieces of a tensor
# (NumPy releases the GIL inside its array loops). At most 16: the share of
# host cores that goes with one GPU.
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    """[fn(i) for i in items], evaluated on ORACLE_THREADS host threads."""
    items = list(items)
    if len(items) <= 1 or ORACLE_THREADS == 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        return list(ex.map(fn, items))


def f32_of(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 NumPy copy of a (CPU or GPU) bf16/fp32 tensor."""
    return t.detach().to("cpu", torch.float32).numpy()


def assert_codes_equal(got, ref, x=None, what=""):
    """Bit-exact compare of uint8 code arrays; on failure name the first
    mismatch with its input bits, the oracle code and the GPU code."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    if bad.size:
        idx = tuple(bad[0])
        msg = f"{what}: {len(bad)} mismatching codes; first at {idx}: gpu 0x{int(got[idx]):02x} oracle 0x{int(ref[idx]):02x}"
        if x is not None:
            xv = np.asarray(x, dtype=np.float32)[idx]
            msg += f", x = {xv!r} (bits 0x{np.float32(xv).view(np.uint32):08x})"
        raise AssertionError(msg)


def assert_scales_equal(got, ref, what=""):
    got = np.ascontiguousarray(np.asarray(got, dtype=np.float32))
    ref = np.ascontiguousarray(np.asarray(ref, dtype=np.float32))
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    gb, rb = got.view(np.uint32), ref.view(np.uint32)
    bad = np.argwhere(gb != rb)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatching scales; first at {idx}: "
                             f"gpu {got[idx]!r} oracle {ref[idx]!r}")


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |v| (0 at v == 0)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def check_gemm_tolerance(y_gpu, y64, t, bf16: bool, what=""):
    """|y_gpu - y64| <= 1e-3 * T per element; a bf16 output may add half a bf16
    ulp for its own final rounding. Returns the number of elements that break
    the literal 1e-3 * T bound (all of them output-rounding cases in bf16)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y64)
    literal = err <= 1e-3 * t
    if bf16:
        bound = 1e-3 * t + bf16_half_ulp(np.maximum(np.abs(y_gpu), np.abs(y64)))
    else:
        bound = 1e-3 * t
    bad = np.argwhere(err > bound)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} outputs out of tolerance; first at {idx}: "
                             f"gpu {y_gpu[idx]!r} oracle {y64[idx]!r} T {t[idx]!r}")
    return int((~literal).sum())


def bf16_round_f32(y32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (nearest even) via the oracle's rounding, returned as fp32 values."""
    return quant.bf16_bits_to_f32(quant.f32_to_bf16_bits(np.asarray(y32, dtype=np.float32)))

