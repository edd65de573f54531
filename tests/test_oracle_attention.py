"""Pins of the oracle's decode attention over the FP8 KV cache.

Sources: pwwt.cn Llama-3 FP8 notes, section 1 (FP8 K and V with their own
scales, grouped-query attention) and section 3 (per head, per 128-token
scales); charles2530.github.io "量化：FP8 与混合精度推理", section "scale 是控制面".

Independent checks: torch's scaled_dot_product_attention in float64 on the
CPU (a library routine) on the dequantized cache; closed forms (identical keys
give the mean of the values; one dominant key gives its value); invariances
(token order, the grouping of query heads onto kv heads, exact power-of-two
scaling of the V scales, a constant added to every score).
"""

import numpy as np
import pytest
import torch

from oracle import attention, e4m3, e5m2, quant


def _cache(rng, hkv, t, fmt="e4m3", d=128):
    mod = quant.fmt_module(fmt)
    codes = rng.integers(0, 256, size=(2, hkv, t, d))
    if fmt == "e4m3":
        codes = np.where((codes & 0x7F) == 0x7F, codes ^ 1, codes)
    else:
        codes = np.where((codes & 0x7F) >= 0x7C, codes & 0xBB, codes)
    codes = codes.astype(np.uint8)
    nb = -(-t // 128)
    scales = (rng.uniform(0.5, 2.0, size=(2, hkv, nb)) * 2.0 ** rng.integers(-10, -4, size=(2, hkv, nb))).astype(np.float32)
    assert np.all(np.isfinite(mod.decode(codes)))
    return codes[0], scales[0], codes[1], scales[1]


def _dequant(codes, scales, fmt):
    t = codes.shape[1]
    s = np.repeat(scales.astype(np.float64), 128, axis=1)[:, :t, None]
    return quant.fmt_module(fmt).decode(codes) * s


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("hq,hkv,t", [(8, 1, 300), (16, 2, 129), (4, 4, 1)])
def test_matches_torch_sdpa_float64(fmt, hq, hkv, t):
    rng = np.random.default_rng(hq * 1000 + t)
    kc, ks, vc, vs = _cache(rng, hkv, t, fmt)
    q = rng.standard_normal((hq, 128))
    c = 1 / np.sqrt(128)
    o, t_o = attention.decode_attention(q, kc, ks, vc, vs, c, fmt)
    kh = torch.from_numpy(_dequant(kc, ks, fmt)).repeat_interleave(hq // hkv, dim=0)   # [hq, t, d]
    vh = torch.from_numpy(_dequant(vc, vs, fmt)).repeat_interleave(hq // hkv, dim=0)
    qt = torch.from_numpy(q)[:, None, :]                                                  # [hq, 1, d]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kh, vh, scale=c)[:, 0, :].numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.all(t_o >= np.abs(o) - 1e-12)


def test_identical_keys_give_the_mean_of_the_values():
    rng = np.random.default_rng(1)
    t = 333
    kc = np.tile(rng.integers(0, 0x70, size=(1, 1, 128)).astype(np.uint8), (1, t, 1))
    ks = np.ones((1, 3), np.float32)
    _, _, vc, vs = _cache(rng, 1, t)
    q = rng.standard_normal((4, 128))
    o, _ = attention.decode_attention(q, kc, ks, vc, vs, 0.1)
    vh = _dequant(vc, vs, "e4m3")[0]
    assert np.allclose(o, np.broadcast_to(vh.mean(axis=0), o.shape), rtol=1e-12, atol=1e-15)


def test_one_dominant_key_gives_its_value():
    rng = np.random.default_rng(2)
    t = 200
    kc = np.zeros((1, t, 128), np.uint8)
    kc[0, 77, :] = 0x7E          # every dim 448
    ks = np.ones((1, 2), np.float32)
    _, _, vc, vs = _cache(rng, 1, t)
    q = np.ones((2, 128))
    # score of token 77: 448 * 128 * c, every other score 0: p of the rest ~ e^-1e4
    o, _ = attention.decode_attention(q, kc, ks, vc, vs, 0.2)
    vh = _dequant(vc, vs, "e4m3")[0]
    assert np.array_equal(o, np.broadcast_to(vh[77], o.shape))


def test_token_order_does_not_matter():
    rng = np.random.default_rng(3)
    t = 256
    kc, ks, vc, vs = _cache(rng, 2, t)
    ks[:] = ks[:, :1]            # one scale per head so that tokens may move across blocks
    vs[:] = vs[:, :1]
    q = rng.standard_normal((8, 128))
    o, _ = attention.decode_attention(q, kc, ks, vc, vs, 0.09)
    perm = rng.permutation(t)
    o2, _ = attention.decode_attention(q, kc[:, perm], ks, vc[:, perm], vs, 0.09)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14)


def test_grouping_is_per_kv_head():
    """8 query heads on 2 kv heads equal each half of the heads run against
    its own kv head alone."""
    rng = np.random.default_rng(4)
    kc, ks, vc, vs = _cache(rng, 2, 150)
    q = rng.standard_normal((8, 128))
    o, _ = attention.decode_attention(q, kc, ks, vc, vs, 0.1)
    for h in range(2):
        oh, _ = attention.decode_attention(q[4 * h:4 * h + 4], kc[h:h + 1], ks[h:h + 1], vc[h:h + 1], vs[h:h + 1], 0.1)
        assert np.array_equal(o[4 * h:4 * h + 4], oh)


def test_power_of_two_v_scale_scales_the_output_exactly():
    rng = np.random.default_rng(5)
    kc, ks, vc, vs = _cache(rng, 1, 200, "e5m2")
    q = rng.standard_normal((3, 128))
    o, t_o = attention.decode_attention(q, kc, ks, vc, vs, 0.1, "e5m2")
    o4, t4 = attention.decode_attention(q, kc, ks, vc, vs * np.float32(4), 0.1, "e5m2")
    assert np.array_equal(o4, 4 * o) and np.array_equal(t4, 4 * t_o)


def test_k_scale_moves_scores_not_a_constant_shift():
    """Scaling every K scale by 2 equals doubling the softmax scale (scores
    are c * q . k_hat); adding a constant to every score changes nothing,
    checked through a key column whose dot product with q is the same for all
    tokens."""
    rng = np.random.default_rng(6)
    kc, ks, vc, vs = _cache(rng, 1, 140)
    q = rng.standard_normal((2, 128))
    a, _ = attention.decode_attention(q, kc, ks * np.float32(2), vc, vs, 0.05)
    b, _ = attention.decode_attention(q, kc, ks, vc, vs, 0.1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)
    ks1 = np.ones_like(ks)
    kc2 = kc.copy()
    kc2[0, :, 0] = 0x38          # dim 0 = 1.0 for every token
    q2 = q.copy()
    q2[:, 0] = 0.0
    base, _ = attention.decode_attention(q2, kc2, ks1, vc, vs, 0.1)
    q2[:, 0] = 3.0               # adds 0.3 to every score
    shifted, _ = attention.decode_attention(q2, kc2, ks1, vc, vs, 0.1)
    assert np.allclose(base, shifted, rtol=1e-12, atol=1e-15)


def test_every_code_is_decoded_by_the_table():
    """Single token: o is exactly the dequantized V row, for every finite code
    of both formats."""
    for mod, fmt in ((e4m3, "e4m3"), (e5m2, "e5m2")):
        codes = mod.finite_codes()
        n = -(-codes.size // 128) * 128
        row = np.zeros(n, np.uint8)
        row[:codes.size] = codes
        for off in range(0, n, 128):
            vc = row[off:off + 128].reshape(1, 1, 128)
            kc = np.zeros((1, 1, 128), np.uint8)
            o, _ = attention.decode_attention(np.ones((1, 128)), kc, np.ones((1, 1), np.float32), vc,
                                              np.full((1, 1), 0.75, np.float32), 0.1, fmt)
            assert np.array_equal(o[0], mod.decode(vc[0, 0]) * 0.75)
