"""Decode attention over an FP8 KV cache (oracle; test infrastructure only).

The consumer of the KV cache the quantizer writes: [LONG] pwwt.cn Llama-3 FP8
notes, section 1 (K and V kept in FP8 with their own scales and dequantized
where attention reads them; the model uses grouped-query attention with 8 kv
heads) and section 3 (per head and per 128-token scales); [MIXED]
charles2530.github.io, "量化：FP8 与混合精度推理", section "scale 是控制面" (per-head
KV scales read by the attention backend).

For query head g of a decode step (one query token), kv head h = g // G with
G = heads_q / heads_kv:

    k_hat[t] = dec(k codes[h, t]) * s_k[h, t // 128]       (exact in float64)
    v_hat[t] = dec(v codes[h, t]) * s_v[h, t // 128]
    s_t      = c * q[g] . k_hat[t]
    p        = softmax(s)                                  (max subtracted)
    o[g]     = sum_t p_t v_hat[t]

The oracle is that definition written out in float64: dequantize, one matrix
product for the scores, exp, normalise, one matrix product for the output.
It also returns T_o[g] = sum_t p_t |v_hat[t]|, the base of the acceptance
bound |o - o_ref| <= 1e-3 * T_o.

Reading where the pages are silent: the scale c is an argument (1/sqrt(128)
for Llama-3); the KV layout is the quantizer's [heads, tokens, head_dim] with
one scale per (head, 128 tokens).
"""

import numpy as np

from . import quant


def _dequant_head(codes, scales, fmt: str, token_block: int) -> np.ndarray:
    """float64 [tokens, head_dim] = dec(codes) * scale of each token's block."""
    t = codes.shape[0]
    s = np.repeat(np.asarray(scales, dtype=np.float32).astype(np.float64), token_block)[:t]
    return quant.fmt_module(fmt).decode(codes) * s[:, None]


def decode_attention(q, k_codes, k_scales, v_codes, v_scales, softmax_scale: float, fmt: str = "e4m3",
                     token_block: int = 128) -> tuple:
    """q: [heads_q, head_dim] (float); k_codes / v_codes: uint8 [heads_kv, tokens,
    head_dim]; k_scales / v_scales: [heads_kv, ceil(tokens / token_block)].

    Returns (o, T_o), both float64 [heads_q, head_dim].
    """
    q = np.asarray(q, dtype=np.float64)
    k_codes = np.asarray(k_codes, dtype=np.uint8)
    v_codes = np.asarray(v_codes, dtype=np.uint8)
    hq, d = q.shape
    hkv = k_codes.shape[0]
    if hq % hkv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    group = hq // hkv
    o = np.empty((hq, d), dtype=np.float64)
    t_o = np.empty((hq, d), dtype=np.float64)
    for h in range(hkv):
        kh = _dequant_head(k_codes[h], k_scales[h], fmt, token_block)
        vh = _dequant_head(v_codes[h], v_scales[h], fmt, token_block)
        qg = q[h * group:(h + 1) * group]                 # [G, d]
        s = float(softmax_scale) * (qg @ kh.T)            # [G, tokens]
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[h * group:(h + 1) * group] = p @ vh
        t_o[h * group:(h + 1) * group] = p @ np.abs(vh)
    return o, t_o
