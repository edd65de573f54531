"""Group quantizer and KV dequantizer (oracle; test infrastructure only).

The method, per group G of elements (one scale per group):

1. a = max |x| over G                      ([FP8] section "什么是 FP8 量化", step 1;
                                            section "权重量化：128×128 分块 FP8", block max)
2. s = a / 448, one fp32 value             (same sections; scales are kept in fp32,
                                            section "权重量化", storage step)
3. q = E4M3(x / s) per element, round to nearest even, saturate at +-448
                                           (section "什么是 FP8 量化", steps 2-3;
                                            section "权重量化", per-element step)
4. dequantization is x ~ q * s             ([MIXED] section "E4M3 和 E5M2 是范围与格点的取舍",
                                            the FP8Cast / rescale equation)

Group shapes ([FP8] sections "权重量化" and "激活动态量化", "FP8 矩阵乘"; [MIXED]
section "scale 是控制面"; [LONG] section 1 and section 3):

* per tensor: the whole tensor;
* 1x128: one row (token) and 128 consecutive columns (input channels);
* 128x128: 128 rows and 128 columns of a weight matrix W in R^{N x K};
* KV: one head, 128 consecutive tokens, all of head_dim; K and V separately.

Ragged edge groups (the ceil(N/128) x ceil(K/128) grid of section "权重量化")
use only their valid elements.

Readings taken where the pages are silent:

* x / s is the IEEE fp32 correctly rounded quotient of the fp32 input value
  and the fp32 scale (the scale is stored in fp32, and x * fl32(1/s) would give
  different codes for about 0.1% of inputs). s = fl32(a / 448) is likewise a
  correctly rounded fp32 division.
* A group whose scale is zero (a == 0, or an fp32 a so small that a/448
  underflows) gets s = 0 and sign-only zero codes; it dequantizes to zero.
* Denormals are kept (no flush to zero).
* The KV dequantizer computes fl32(decode(q) * s) and rounds that to bf16
  with round-to-nearest-even.

Formats: every function takes ``fmt`` = "e4m3" (default) or "e5m2". E5M2 ([FP8]
section "FP8 是什么", format table; [VS] section 2, E5M2 KV cache) runs the same
steps with its own largest value: s = a / 57344 and codes from the E5M2 grid.
"""

import numpy as np

from . import e4m3, e5m2

FORMATS = {"e4m3": e4m3, "e5m2": e5m2}
FORMAT_MAX = {"e4m3": e4m3.E4M3_MAX, "e5m2": e5m2.E5M2_MAX}


def fmt_module(fmt: str):
    """The table module of an FP8 format name."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    return FORMATS[fmt]

GROUP = 128


def scale_of(amax, fmt: str = "e4m3") -> np.ndarray:
    """s = fl32(amax / max_fmt) (448 for E4M3, 57344 for E5M2) as a correctly
    rounded fp32 division."""
    fmt_module(fmt)
    return np.asarray(amax, dtype=np.float32) / np.float32(FORMAT_MAX[fmt])


def cast(x32: np.ndarray, s32: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Codes of fl32(x / s), elementwise; ``s`` broadcasts against ``x``.

    Where s == 0 the code is the sign of x with a zero magnitude. A quotient
    that overflows fp32 (possible only with a caller-supplied scale) lies
    beyond the format's range like any other, so it saturates: it is passed
    to the encoder as the largest finite fp32 number of its sign.
    """
    enc = fmt_module(fmt).encode
    x32 = np.asarray(x32, dtype=np.float32)
    s32 = np.broadcast_to(np.asarray(s32, dtype=np.float32), x32.shape)
    out = np.empty(x32.shape, dtype=np.uint8)
    flat_x = x32.reshape(-1)
    flat_s = s32.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 22
    for lo in range(0, flat_x.size, step):
        xs = flat_x[lo:lo + step]
        ss = flat_s[lo:lo + step]
        zero = ss == 0
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            quot = xs / np.where(zero, np.float32(1), ss)   # fp32 / fp32, IEEE
        quot = np.where(zero, np.where(np.signbit(xs), np.float32(-0.0), np.float32(0.0)), quot)
        quot = np.where(np.isinf(quot) & np.isfinite(xs), np.copysign(np.finfo(np.float32).max, quot), quot)
        flat_o[lo:lo + step] = enc(quot)
    return out


def _pad_to(a: np.ndarray, axis: int, mult: int) -> np.ndarray:
    """Zero-pad ``axis`` up to a multiple of ``mult``. Zeros never raise max|x|,
    and padded positions are dropped again by the callers."""
    n = a.shape[axis]
    extra = (-n) % mult
    if extra == 0:
        return a
    widths = [(0, 0)] * a.ndim
    widths[axis] = (0, extra)
    return np.pad(a, widths)


def quantize_per_tensor(x, fmt: str = "e4m3") -> tuple:
    """One scale for the whole tensor. Returns (codes uint8 like x, s float32 [1])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32)) if x32.size else np.float32(0)
    s = scale_of(amax, fmt).reshape(1)
    return cast(x32, s[0], fmt), s


def quantize_group_1x128(x, fmt: str = "e4m3") -> tuple:
    """x: [rows, cols]. Group = one row x 128 consecutive columns.

    Returns (codes uint8 [rows, cols], s float32 [rows, ceil(cols/128)]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    g = -(-cols // GROUP)
    xp = _pad_to(x32, 1, GROUP).reshape(rows, g, GROUP)
    amax = np.max(np.abs(xp), axis=2)
    s = scale_of(amax, fmt)
    s_full = np.repeat(s, GROUP, axis=1)[:, :cols]
    return cast(x32, s_full, fmt), s


def quantize_block_128x128(x, fmt: str = "e4m3") -> tuple:
    """x: [rows, cols] (a weight W in R^{N x K}). Group = 128 x 128 block.

    Returns (codes uint8 [rows, cols], s float32 [ceil(rows/128), ceil(cols/128)]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    gr, gc = -(-rows // GROUP), -(-cols // GROUP)
    xp = _pad_to(_pad_to(x32, 0, GROUP), 1, GROUP).reshape(gr, GROUP, gc, GROUP)
    amax = np.max(np.abs(xp), axis=(1, 3))
    s = scale_of(amax, fmt)
    s_full = np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)[:rows, :cols]
    return cast(x32, s_full, fmt), s


def kv_quantize(kv, token_block: int = GROUP, fmt: str = "e4m3") -> tuple:
    """kv: [heads, tokens, head_dim]. Group = one head x ``token_block``
    consecutive tokens x all of head_dim.

    Returns (codes uint8 [heads, tokens, head_dim],
             s float32 [heads, ceil(tokens/token_block)]).
    """
    x32 = np.asarray(kv, dtype=np.float32)
    h, t, d = x32.shape
    nb = -(-t // token_block)
    xp = _pad_to(x32, 1, token_block).reshape(h, nb, token_block, d)
    amax = np.max(np.abs(xp), axis=(2, 3))
    s = scale_of(amax, fmt)
    s_full = np.repeat(s, token_block, axis=1)[:, :t, None]
    return cast(x32, s_full, fmt), s


def quantize_static(x, s, fmt: str = "e4m3") -> tuple:
    """Static / delayed scaling ([MIXED] section "scale 是控制面": a scale taken
    from history rather than the current batch): codes of fl32(x / s) under
    the given fp32 scale s (saturating like every cast here), and the tensor's
    own amax for the caller's history. Returns (codes, amax float32)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32)) if x32.size else np.float32(0)
    return cast(x32, np.float32(s), fmt), np.float32(amax)


def scale_from_history(history, fmt: str = "e4m3") -> np.float32:
    """Delayed-scaling scale: fl32(max(history) / max_fmt) ([MIXED] section
    "scale 是控制面", amax history)."""
    return scale_of(np.max(np.abs(np.asarray(history, dtype=np.float32))), fmt)


def f32_to_bf16_bits(x32) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    The two bf16 candidates are the fp32 value with its low 16 bits cleared
    (toward zero) and the next bf16 away from zero; the nearer one wins, and a
    tie goes to the candidate whose last kept bit is 0.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    bits = x32.view(np.uint32)
    lo = bits & np.uint32(0xFFFF0000)
    hi = lo + np.uint32(0x10000)
    x64 = x32.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        vlo = lo.view(np.float32).astype(np.float64)
        vhi = hi.view(np.float32).astype(np.float64)
    dlo = np.abs(x64 - vlo)
    dhi = np.abs(vhi - x64)
    lo_is_odd = ((lo >> np.uint32(16)) & np.uint32(1)).astype(bool)
    take_hi = (dhi < dlo) | ((dhi == dlo) & lo_is_odd)
    return (np.where(take_hi, hi, lo) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def kv_dequantize(q, s, token_block: int = GROUP, fmt: str = "e4m3") -> np.ndarray:
    """bf16(fl32(decode(q) * s)) with the scale of each (head, token block).

    q: uint8 [heads, tokens, head_dim]; s: float32 [heads, ceil(tokens/token_block)].
    Returns uint16 bf16 bit patterns [heads, tokens, head_dim].
    decode(q) has at most 4 significant bits and s at most 24, so the float64
    product is exact and float32() applies the one fp32 rounding.
    """
    q = np.asarray(q, dtype=np.uint8)
    h, t, d = q.shape
    s_full = np.repeat(np.asarray(s, dtype=np.float32), token_block, axis=1)[:, :t, None]
    prod = (fmt_module(fmt).decode(q) * s_full.astype(np.float64)).astype(np.float32)
    return f32_to_bf16_bits(prod)


def dequantize_grid(q, s, group_rows: int, group_cols: int, fmt: str = "e4m3") -> np.ndarray:
    """fp64 x_hat = decode(q) * s for a 2-D code array with a scale grid of
    ``group_rows`` x ``group_cols`` groups (a per-tensor grid is one group
    spanning everything). Exact in float64."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    dec = fmt_module(fmt).decode
    if s.size == 1:
        return dec(q) * s.reshape(())
    s_full = np.repeat(np.repeat(s, group_rows, axis=0), group_cols, axis=1)[:rows, :cols]
    return dec(q) * s_full
