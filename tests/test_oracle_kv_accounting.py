"""KV-cache byte accounting against the numbers printed on the pages.

pwwt.cn Llama-3 FP8 notes, section 5 (the memory ledger for long context):
Llama-3-70B has 80 layers, 8 KV heads and head dimension 128, so one token's
K and V in 16-bit floats take 2 x 80 x 8 x 128 x 2 bytes (about 327 KB) and
a 128K-token context about 40 GB; FP8 halves it to about 20 GB. Section 1 of
the same page gives the same 40 GB -> 20 GB figures.

The oracle's KV format (one code byte per element, one fp32 scale per head and
128 tokens, K and V separately) is measured on a small cache and scaled to
that model: the codes take exactly half of the bf16 bytes and the scales add
2 x 80 x 8 x 1024 x 4 bytes (5 MiB) at 128K tokens.
"""

import numpy as np

from oracle import quant

LAYERS, KV_HEADS, HEAD_DIM, TOKENS = 80, 8, 128, 131072


def test_bf16_bytes_per_token_and_context():
    per_token = 2 * LAYERS * KV_HEADS * HEAD_DIM * 2
    assert per_token == 327_680                      # "327KB"
    assert per_token * TOKENS == 40 * 2 ** 30        # "40GB": exactly 40 GiB


def test_fp8_cache_halves_it_plus_the_scales():
    rng = np.random.default_rng(0)
    t = 384
    k = rng.standard_normal((KV_HEADS, t, HEAD_DIM)).astype(np.float32)
    q, s = quant.kv_quantize(k)
    assert q.dtype == np.uint8 and q.shape == k.shape          # one byte per element
    assert s.dtype == np.float32 and s.shape == (KV_HEADS, t // 128)
    code_bytes_per_token = 2 * LAYERS * q.nbytes // t          # K and V, every layer
    scale_bytes_per_128 = 2 * LAYERS * s.nbytes // (t // 128)
    codes = code_bytes_per_token * TOKENS
    scales = scale_bytes_per_128 * (TOKENS // 128)
    assert codes == 20 * 2 ** 30                                # "20GB"
    assert scales == 2 * LAYERS * KV_HEADS * 1024 * 4 == 5 * 2 ** 20
    assert abs((codes + scales) / (40 * 2 ** 30) - 0.5) < 2e-4
