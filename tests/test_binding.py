"""The Python binding on a machine without a GPU: it loads the in-tree
library, exposes every entry point under the C ABI's name, refuses host
tensors before any HIP call (there is no CPU fallback), and raises when the
library is missing."""

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp8_quantization_block_amd", "libfp8blk.so")

NAMES = ("fp8_quantize", "fp8_block_gemm", "fp8_block_gemm_quant", "fp8_kv_quantize", "fp8_kv_dequantize",
         "fp8_kv_decode_attention", "fp8_quantize_static", "fp8_scale_from_amax_history", "fp8_quantize_mx",
         "fp8_mx_gemm", "fp8_pack_weights_decode", "fp8_block_gemm_packed", "fp8_kv_decode_attention_noalloc",
         "fp8_quantize_gemm_decode")


@pytest.fixture(scope="module")
def fp8():
    if not os.path.exists(LIB):
        pytest.skip("libfp8blk.so not built (python -m fp8_quantization_block_amd.build)")
    import fp8_quantization_block_amd as m
    m.load_library(LIB)
    return m


def test_entry_points_exist(fp8):
    lib = fp8.load_library()
    for n in NAMES:
        assert callable(getattr(fp8, n)), n
        assert hasattr(lib, n), n


def test_host_tensors_are_refused(fp8):
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    u8 = torch.zeros(256, 256, dtype=torch.uint8)
    s = torch.ones(1)
    calls = [
        lambda: fp8.fp8_quantize(x, "group_1x128"),
        lambda: fp8.fp8_quantize_static(x, s),
        lambda: fp8.fp8_scale_from_amax_history(s),
        lambda: fp8.fp8_quantize_mx(x),
        lambda: fp8.fp8_block_gemm(u8, s, "per_tensor", u8, s, "per_tensor"),
        lambda: fp8.fp8_block_gemm_quant(u8, s, "per_tensor", u8, s, "per_tensor"),
        lambda: fp8.fp8_mx_gemm(u8, u8, u8, u8),
        lambda: fp8.fp8_pack_weights_decode(u8),
        lambda: fp8.fp8_quantize_gemm_decode(x, u8, s, "per_tensor"),
        lambda: fp8.fp8_block_gemm_packed(u8, s, "per_tensor", torch.zeros(2, 16, 2048, dtype=torch.uint8), s,
                                          "per_tensor"),
        lambda: fp8.fp8_kv_quantize(torch.zeros(1, 128, 128, dtype=torch.bfloat16)),
        lambda: fp8.fp8_kv_dequantize(torch.zeros(1, 128, 128, dtype=torch.uint8), torch.ones(1, 1)),
        lambda: fp8.fp8_kv_decode_attention(torch.zeros(8, 128, dtype=torch.bfloat16),
                                            torch.zeros(1, 128, 128, dtype=torch.uint8), torch.ones(1, 1),
                                            torch.zeros(1, 128, 128, dtype=torch.uint8), torch.ones(1, 1), 0.1),
        lambda: fp8.fp8_kv_decode_attention_noalloc(torch.zeros(8, 128, dtype=torch.bfloat16),
                                                    torch.zeros(1, 128, 128, dtype=torch.uint8), torch.ones(1, 1),
                                                    torch.zeros(1, 128, 128, dtype=torch.uint8), torch.ones(1, 1), 0.1,
                                                    torch.zeros(8, 128)),
    ]
    for c in calls:
        with pytest.raises(ValueError):
            c()


def test_missing_library_raises():
    code = ("import fp8_quantization_block_amd as m\n"
            "try:\n"
            "    m.load_library('/nonexistent/libfp8blk.so')\n"
            "except RuntimeError as e:\n"
            "    print('raised', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("raised"), out.stdout + out.stderr
