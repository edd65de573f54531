"""Block-scaled FP8 GEMM (oracle; test infrastructure only).

Follows [FP8] section "激活动态量化" (the full product becomes a sum over the
128-wide K blocks j of s_x * s_{w,j} times the FP8 block product, with the
scales multiplied back while accumulating) and section "FP8 矩阵乘" (weights in
128x128 blocks, activations in per-token groups of 128, FP8 products with
fp32 accumulation, partial results multiplied by their scales). [MIXED]
section "混合精度才是生产形态" adds that low-precision products are summed in
higher precision.

Reading of the printed equation: it writes y = xW, but W is defined as
N x K (N outputs, K inputs) with an ceil(N/128) x ceil(K/128) scale grid and
activations may carry one scale per 128-channel group. So

    y[m, n] = sum_j  s_a[m, j] * s_w[n // 128, j] * sum_{k in block j} qa[m, k] * qw[n, k]

with qa, qw the decoded FP8 values (E4M3, or E5M2 for either operand: [FP8]
section "FP8 是什么", format table), i.e. y = A_hat . W_hat^T with
A_hat = decode(qa) * s_a and W_hat = decode(qw) * s_w. With a per-tensor scale
the scale is one number for the whole operand.

The oracle is that definition written out: dequantize both operands to
float64 (exact: 4 significant bits times 24), then one float64 matmul. It also
returns the tolerance base T = |A_hat| . |W_hat|^T used by the acceptance bound
|y - y_ref| <= 1e-3 * T.
"""

import numpy as np

from . import quant

PER_TENSOR = "per_tensor"
GROUP_1x128 = "group_1x128"
BLOCK_128x128 = "block_128x128"


def dequant_activations(qa, sa, gran: str, fmt: str = "e4m3") -> np.ndarray:
    """A_hat [M, K] in float64. gran: per_tensor (sa [1]) or group_1x128 (sa [M, ceil(K/128)])."""
    if gran == PER_TENSOR:
        return quant.dequantize_grid(qa, np.asarray(sa).reshape(1), 1, 1, fmt)
    if gran == GROUP_1x128:
        return quant.dequantize_grid(qa, sa, 1, quant.GROUP, fmt)
    raise ValueError(gran)


def dequant_weights(qw, sw, gran: str, fmt: str = "e4m3") -> np.ndarray:
    """W_hat [N, K] in float64. gran: per_tensor (sw [1]) or block_128x128
    (sw [ceil(N/128), ceil(K/128)])."""
    if gran == PER_TENSOR:
        return quant.dequantize_grid(qw, np.asarray(sw).reshape(1), 1, 1, fmt)
    if gran == BLOCK_128x128:
        return quant.dequantize_grid(qw, sw, quant.GROUP, quant.GROUP, fmt)
    raise ValueError(gran)


def block_gemm(qa, sa, gran_a: str, qw, sw, gran_w: str, rows=None, cols=None,
               fmt_a: str = "e4m3", fmt_w: str = "e4m3") -> tuple:
    """Returns (y, T), both float64 [M, N] (or [len(rows), len(cols)] when
    ``rows``/``cols`` select a subset of outputs).

    y = A_hat . W_hat^T and T = |A_hat| . |W_hat|^T. With a selection only the
    selected rows of A_hat and W_hat are formed (each row is dequantized with
    the scales of its own groups, as in the full computation).
    """
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    sa = np.asarray(sa, dtype=np.float32)
    sw = np.asarray(sw, dtype=np.float32)
    K = qa.shape[1]
    g = quant.GROUP
    if rows is not None:
        rows = np.asarray(rows)
        qa = qa[rows]
        if gran_a == GROUP_1x128:
            sa = sa[rows]
    if cols is not None:
        cols = np.asarray(cols)
        qw = qw[cols]
        if gran_w == BLOCK_128x128:
            # one row of the block grid per selected weight row
            w_scales = np.repeat(sw[cols // g], g, axis=1)[:, :K].astype(np.float64)
            w = quant.fmt_module(fmt_w).decode(qw) * w_scales
        else:
            w = dequant_weights(qw, sw, gran_w, fmt_w)
    else:
        w = dequant_weights(qw, sw, gran_w, fmt_w)
    a = dequant_activations(qa, sa, gran_a, fmt_a)
    y = a @ w.T
    t = np.abs(a) @ np.abs(w).T
    return y, t
