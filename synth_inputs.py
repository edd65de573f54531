"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no part of the quantization or GEMM arithmetic: it only
draws seeded random numbers with the shapes and value structure of the
workloads and rounds them to bf16. Both the HIP path and the CPU oracle take
their inputs from here.

The pages measure Llama-3 8B/70B models on long-document QA and other suites;
no weights or datasets are available, so seeded tensors of the same shapes
stand in for them:

* Llama-3-8B MLP: hidden 4096, MLP width 14336; Llama-3-70B: hidden 8192,
  MLP width 28672, fused QKV width (64 q heads + 2 x 8 kv heads) x 128 = 10240;
  KV cache with 8 kv heads x head_dim 128 ([LONG] section 5 memory arithmetic).
* Activations are mostly small with a few large outliers ([FP8] section
  "FP8 与 INT8 量化精度对比", the outlier example): N(0, 1) with either a sparse
  set of x100 entries (per-tensor case) or 8 outlier input channels x50 for
  every token.
* Weights are N(0, 0.02).
* Keys shrink toward the end of the sequence ([LONG] section 3): K = N(0, 1) *
  2^(-12 t / T); values are more spread: V = N(0, 2).
* Decode-step queries for attention over the KV cache: 64 query heads
  (Llama-3-70B, 8 per kv head) x 128, N(0, 2).

Seeds are 1000 * config + role, roles 0 = activations, 1 = outlier positions,
2 = weights, 3 = K, 4 = V, 5 = queries. fp32 draws are rounded to bf16 with
round-to-nearest-even (torch's CPU conversion).
"""

import numpy as np
import torch

ROLE_A, ROLE_OUTLIER, ROLE_W, ROLE_K, ROLE_V, ROLE_Q = 0, 1, 2, 3, 4, 5

CONFIGS = {
    1: dict(workload="per_tensor_e4m3_gemm_64x512x512", M=64, N=512, K=512,
            gran_a="per_tensor", gran_w="per_tensor"),
    2: dict(workload="llama3_8b_mlp_up_prefill_4096x14336x4096", M=4096, N=14336, K=4096,
            gran_a="group_1x128", gran_w="block_128x128"),
    3: dict(workload="llama3_70b_mlp_up_decode_16x28672x8192", M=16, N=28672, K=8192,
            gran_a="group_1x128", gran_w="block_128x128"),
    4: dict(workload="llama3_70b_qkv_prefill_8192x10240x8192", M=8192, N=10240, K=8192,
            gran_a="group_1x128", gran_w="block_128x128"),
    5: dict(workload="kv_cache_8x131072x128", heads=8, tokens=131072, head_dim=128, heads_q=64),
}


def seed_of(config: int, role: int, variant: int = 0) -> int:
    return 1000 * config + role + 100000 * variant


def to_bf16(x32: np.ndarray) -> torch.Tensor:
    """Round an fp32 NumPy array to a bf16 CPU tensor (nearest, ties to even)."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)


def activations(config: int, M: int = None, K: int = None, variant: int = 0) -> torch.Tensor:
    """bf16 [M, K] activations with the config's outlier structure."""
    c = CONFIGS[config]
    M = c["M"] if M is None else M
    K = c["K"] if K is None else K
    rng = np.random.default_rng(seed_of(config, ROLE_A, variant))
    x = rng.standard_normal((M, K), dtype=np.float32)
    pos = np.random.default_rng(seed_of(config, ROLE_OUTLIER, variant))
    if config == 1:
        # exactly round(0.1% of the entries) scaled by 100, at seeded positions
        n_out = int(round(0.001 * M * K))
        idx = pos.permutation(M * K)[:n_out]
        x.reshape(-1)[idx] *= np.float32(100.0)
    else:
        # 8 outlier input channels, x50 for every token
        ch = pos.permutation(K)[:min(8, K)]
        x[:, ch] *= np.float32(50.0)
    return to_bf16(x)


def weights(config: int, N: int = None, K: int = None, variant: int = 0) -> torch.Tensor:
    """bf16 [N, K] weights, N(0, 0.02)."""
    c = CONFIGS[config]
    N = c["N"] if N is None else N
    K = c["K"] if K is None else K
    rng = np.random.default_rng(seed_of(config, ROLE_W, variant))
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return to_bf16(w)


def kv_pair(config: int = 5, heads: int = None, tokens: int = None, head_dim: int = None,
            variant: int = 0) -> tuple:
    """(K, V) bf16 [heads, tokens, head_dim]: K = N(0,1) * 2^(-12 t / tokens), V = N(0, 2)."""
    c = CONFIGS[5]
    heads = c["heads"] if heads is None else heads
    tokens = c["tokens"] if tokens is None else tokens
    head_dim = c["head_dim"] if head_dim is None else head_dim
    rk = np.random.default_rng(seed_of(config, ROLE_K, variant))
    k = rk.standard_normal((heads, tokens, head_dim), dtype=np.float32)
    decay = np.exp2(np.float32(-12.0) * np.arange(tokens, dtype=np.float32) / np.float32(tokens))
    k *= decay[None, :, None]
    rv = np.random.default_rng(seed_of(config, ROLE_V, variant))
    v = rv.standard_normal((heads, tokens, head_dim), dtype=np.float32) * np.float32(2.0)
    return to_bf16(k), to_bf16(v)


def decode_queries(heads_q: int = 64, head_dim: int = 128, variant: int = 0) -> torch.Tensor:
    """bf16 [heads_q, head_dim] decode-step queries, N(0, 2)."""
    rq = np.random.default_rng(seed_of(5, ROLE_Q, variant))
    return to_bf16(rq.standard_normal((heads_q, head_dim), dtype=np.float32) * np.float32(2.0))


def bf16_to_f32_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 values of a bf16 CPU tensor, as NumPy."""
    return t.to(torch.float32).numpy()
