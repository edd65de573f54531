"""MX block formats: FP8 codes with one power-of-two (E8M0) scale per 32
consecutive elements, and the GEMM over them (oracle; test infrastructure only).

Follows [VS] api.makesence.top, "LLM推理量化:FP8 versus INT8", section 3
(Microscaling formats with a block size of 32: MXFP8 and MXINT8, a scale
shared by each block of 32, run natively by block-scaled hardware); [FP8]
wangyu.me, "大语言模型量化技术（五）：FP8", section "什么是 FP8 量化" (a scale maps the
block into the format's range; round to nearest, ties to even, saturate).

Readings taken where the pages are silent:

* The shared scale is a power of two stored as an 8-bit biased exponent
  (E8M0: byte e means 2^(e - 127); 0xFF is not used), the format of the
  block-scaled hardware the pages refer to.
* Its value: the smallest power of two X with max|x| <= MAX * X over the
  block (MAX = 448 for E4M3, 57344 for E5M2), i.e. the pages' s = amax / MAX
  rounded up to a power of two, so that the block's largest element never
  saturates. X is clamped to [2^-127, 2^127]; an all-zero block takes
  X = 2^-127 (byte 0).
* Codes are FP8(x / X); the quotient is exact (X is a power of two), so the
  only rounding is the FP8 encoder's.
* Blocks run along the rows of a [rows, cols] tensor (32 consecutive
  columns); a ragged last block uses its valid elements.
* The GEMM is y[m, n] = sum_k (qa[m, k] * Xa[m, k // 32]) * (qw[n, k] *
  Xw[n, k // 32]): both operands are blocked along the reduction dimension.
"""

import numpy as np

from . import quant

BLOCK = 32
E8M0_BIAS = 127


def shared_exponent(amax, fmt: str = "e4m3") -> np.ndarray:
    """Integer k (X = 2^k) per block: the smallest k with amax <= MAX * 2^k,
    clamped to [-127, 127]; amax == 0 gives -127. Found by stepping k up from
    a lower bound with exact float64 comparisons."""
    amax = np.asarray(amax, dtype=np.float64)
    mx = quant.FORMAT_MAX[fmt]
    out = np.full(amax.shape, -127, dtype=np.int64)
    flat_a = amax.reshape(-1)
    flat_o = out.reshape(-1)
    for i, a in enumerate(flat_a):
        if a == 0.0:
            continue
        k = int(np.floor(np.log2(a))) - int(np.floor(np.log2(mx))) - 2    # safely below the answer
        while mx * 2.0 ** k < a:
            k += 1
        flat_o[i] = min(max(k, -127), 127)
    return out


def quantize_mx(x, fmt: str = "e4m3") -> tuple:
    """x: [rows, cols]. Returns (codes uint8 [rows, cols], scale bytes uint8
    [rows, ceil(cols / 32)] holding k + 127)."""
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    nb = -(-cols // BLOCK)
    pad = nb * BLOCK - cols
    xp = np.pad(x32, ((0, 0), (0, pad))).reshape(rows, nb, BLOCK)
    amax = np.max(np.abs(xp), axis=2)
    k = shared_exponent(amax, fmt)
    xs = np.repeat(np.exp2(k.astype(np.float64)), BLOCK, axis=1)[:, :cols]
    quot = x32.astype(np.float64) / xs                 # exact: division by a power of two
    codes = quant.fmt_module(fmt).encode(quot)
    return codes, (k + E8M0_BIAS).astype(np.uint8)


def dequantize_mx(codes, scale_bytes, fmt: str = "e4m3") -> np.ndarray:
    """float64 [rows, cols] = dec(codes) * 2^(byte - 127) of each element's block."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    k = np.asarray(scale_bytes, dtype=np.int64) - E8M0_BIAS
    xs = np.repeat(np.exp2(k.astype(np.float64)), BLOCK, axis=1)[:, :cols]
    return quant.fmt_module(fmt).decode(codes) * xs


def mx_gemm(qa, sa, qw, sw, fmt_a: str = "e4m3", fmt_w: str = "e4m3", rows=None, cols=None) -> tuple:
    """y = A_hat . W_hat^T and T = |A_hat| . |W_hat|^T in float64 (optionally
    for selected output rows / columns), A_hat and W_hat the dequantized MX
    operands ([M, K] and [N, K], both blocked along K)."""
    qa, sa, qw, sw = (np.asarray(v) for v in (qa, sa, qw, sw))
    if rows is not None:
        qa, sa = qa[rows], sa[rows]
    if cols is not None:
        qw, sw = qw[cols], sw[cols]
    a = dequantize_mx(qa, sa, fmt_a)
    w = dequantize_mx(qw, sw, fmt_w)
    return a @ w.T, np.abs(a) @ np.abs(w).T
