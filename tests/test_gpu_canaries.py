"""Guard bands around every output buffer: each entry point writes nothing
outside its outputs' valid elements.

Every output lives inside a larger buffer filled with the byte 0xA5: 4 KB
before and after it, and the row padding between `cols` and the leading
dimension. After each call (ragged shapes, every entry point that writes
device memory, including the per-tensor and static passes whose maxima use
slots of the code buffer, and the decode-attention workspace) the bytes
outside the valid region must still be 0xA5. This catches out-of-bounds
writes without a GPU sanitizer.
"""

import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as syn

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENT = 0xA5
GUARD = 4096


class Guarded:
    """A [rows, cols] view with row stride ld (elements) inside a canary-filled buffer."""

    def __init__(self, rows, cols, ld, dtype):
        self.esz = torch.empty(0, dtype=dtype).element_size()
        self.rows, self.cols, self.ld = rows, cols, ld
        self.body = rows * ld * self.esz
        self.buf = torch.full((GUARD + self.body + GUARD,), SENT, dtype=torch.uint8, device=DEV)
        self.full = self.buf[GUARD:GUARD + self.body].view(dtype).view(rows, ld)
        self.view = self.full[:, :cols]

    def check(self, what):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        assert np.all(b[:GUARD] == SENT), f"{what}: bytes before the buffer written"
        assert np.all(b[GUARD + self.body:] == SENT), f"{what}: bytes after the buffer written"
        body = b[GUARD:GUARD + self.body].reshape(self.rows, self.ld * self.esz)
        assert np.all(body[:, self.cols * self.esz:] == SENT), f"{what}: row padding written"
        assert not np.all(body[:, :self.cols * self.esz] == SENT), f"{what}: nothing written"


def _x(rows, cols, seed=0):
    """bf16 [rows, cols] with a 16-byte-multiple row stride (the quantizers' requirement)."""
    ld = (cols + 7) // 8 * 8
    buf = torch.zeros((rows, ld), dtype=torch.bfloat16)
    buf[:, :cols] = torch.from_numpy(np.random.default_rng(seed).standard_normal((rows, cols)).astype(np.float32))
    return buf.to(DEV)[:, :cols]


@pytest.mark.parametrize("rows,cols", [(300, 200), (7, 3), (129, 1000)])
def test_quantize_granularities(gpu_lib, rows, cols):
    x = _x(rows, cols, rows)
    ldq = (cols + 15) // 16 * 16 + 16
    g = (cols + 127) // 128
    cases = [
        ("per_tensor", "row", Guarded(1, 1, 4, torch.float32)),
        ("group_1x128", "row", Guarded(rows, g, g + 1, torch.float32)),
        ("group_1x128", "kmajor", Guarded(g, rows, rows + 3, torch.float32)),
        ("block_128x128", "row", Guarded((rows + 127) // 128, g, g + 2, torch.float32)),
    ]
    for gran, layout, sc in cases:
        q = Guarded(rows, cols, ldq, torch.uint8)
        scales = sc.view.t() if layout == "kmajor" else sc.view
        gpu_lib.fp8_quantize(x, gran, out=q.view, scales=scales)
        q.check(f"{gran} {layout} codes")
        sc.check(f"{gran} {layout} scales")


@pytest.mark.parametrize("rows,cols", [(300, 200), (3, 2), (205, 33)])
def test_static_and_mx(gpu_lib, rows, cols):
    x = _x(rows, cols, rows + 1)
    ldq = (cols + 15) // 16 * 16 + 16
    q = Guarded(rows, cols, ldq, torch.uint8)
    am = Guarded(1, 1, 4, torch.float32)
    s = torch.tensor([0.01], device=DEV)
    gpu_lib.fp8_quantize_static(x, s, record_amax=True, out=q.view, amax=am.view[0])
    q.check("static codes")
    am.check("static amax")
    q = Guarded(rows, cols, ldq, torch.uint8)
    nb = (cols + 31) // 32
    sb = Guarded(rows, nb, nb + 5, torch.uint8)
    gpu_lib.fp8_quantize_mx(x, out=q.view, scales=sb.view)
    q.check("mx codes")
    sb.check("mx scale bytes")


def test_kv_quantize_and_dequantize(gpu_lib):
    lib = gpu_lib.load_library()
    h, t, d = 3, 300, 128
    kv, _ = syn.kv_pair(heads=h, tokens=t, head_dim=d, variant=4)
    kv = kv.to(DEV)
    nb = (t + 127) // 128
    q = Guarded(1, h * t * d, h * t * d, torch.uint8)
    sc = Guarded(1, h * nb, h * nb, torch.float32)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda v: ctypes.c_void_p(v.data_ptr())
    for fmt in (gpu_lib.E4M3, gpu_lib.E5M2):
        gpu_lib._check(lib.fp8_kv_quantize(P(kv), h, t, d, kv.stride(0), kv.stride(1), 128, fmt, P(q.view),
                                           P(sc.view), st))
        q.check("kv codes")
        sc.check("kv scales")
        out = Guarded(1, h * t * d, h * t * d, torch.bfloat16)
        gpu_lib._check(lib.fp8_kv_dequantize(P(q.view), P(sc.view), h, t, d, 128, fmt, P(out.view), st))
        out.check("kv dequantized")


@pytest.mark.parametrize("M", [300, 40])
def test_gemms(gpu_lib, M):
    N, K = 384, 256                     # N % 256 == 128: a half-empty tile column
    qa, sa = gpu_lib.fp8_quantize(_x(M, K, M), "group_1x128", scale_layout="kmajor")
    qw, sw = gpu_lib.fp8_quantize((_x(N, K, 5) * 0.02).contiguous(), "block_128x128")
    for dtype, ld in ((torch.bfloat16, N + 8), (torch.float32, N + 4)):
        c = Guarded(M, N, ld, dtype)
        gpu_lib.fp8_block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128", out=c.view)
        c.check(f"block GEMM {dtype} M={M}")
    qc = Guarded(M, N, N + 16, torch.uint8)
    sc = Guarded(N // 128, M, M + 4, torch.float32)
    gpu_lib.fp8_block_gemm_quant(qa, sa, "group_1x128", qw, sw, "block_128x128", out=qc.view, scales=sc.view.t())
    qc.check(f"fused quantized output M={M}")
    sc.check(f"fused output scales M={M}")
    qam, sam = gpu_lib.fp8_quantize_mx(_x(M, K, M + 2))
    qwm, swm = gpu_lib.fp8_quantize_mx((_x(N, K, 6) * 0.02).contiguous())
    c = Guarded(M, N, N + 8, torch.bfloat16)
    gpu_lib.fp8_mx_gemm(qam, sam, qwm, swm, out=c.view)
    c.check(f"MX GEMM M={M}")


@pytest.mark.parametrize("gran_a", ["per_tensor", "group_1x128"])
@pytest.mark.parametrize("packed", [False, True])
def test_quantize_gemm_decode(gpu_lib, gran_a, packed):
    M, N, K = 40, 384, 512
    x = _x(M, K, 9)
    qw, sw = gpu_lib.fp8_quantize((_x(N, K, 8) * 0.02).contiguous(), "block_128x128")
    w_arg = gpu_lib.fp8_pack_weights_decode(qw) if packed else qw
    for dtype, ld in ((torch.bfloat16, N + 8), (torch.float32, N + 4)):
        c = Guarded(M, N, ld, dtype)
        q = Guarded(M, K, K + 16, torch.uint8)
        if gran_a == "per_tensor":
            s = Guarded(1, 1, 4, torch.float32)
            sv = s.view[0]
        else:
            s = Guarded(K // 128, M, M + 3, torch.float32)   # K-block-major grid, padded
            sv = s.view.t()
        gpu_lib.fp8_quantize_gemm_decode(x, w_arg, sw, "block_128x128", gran_a=gran_a, out=c.view, codes=q.view,
                                         scales=sv)
        what = f"quantize inside the decode GEMM ({gran_a}, packed={packed}) {dtype}"
        c.check(what + " output")
        q.check(what + " codes")
        s.check(what + " scales")


def test_packed_decode(gpu_lib):
    M, N, K = 40, 384, 256
    qa, sa = gpu_lib.fp8_quantize(_x(M, K, M), "group_1x128", scale_layout="kmajor")
    qw, sw = gpu_lib.fp8_quantize((_x(N, K, 7) * 0.02).contiguous(), "block_128x128")
    pk = Guarded(1, N * K, N * K, torch.uint8)
    packed = pk.view[0].view(K // 128, N // 16, 2048)
    gpu_lib.fp8_pack_weights_decode(qw, out=packed)
    pk.check("decode-packed weights")
    for dtype, ld in ((torch.bfloat16, N + 8), (torch.float32, N + 4)):
        c = Guarded(M, N, ld, dtype)
        gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", packed, sw, "block_128x128", out=c.view)
        c.check(f"packed decode GEMM {dtype}")


def test_decode_attention(gpu_lib):
    lib = gpu_lib.load_library()
    hq, hkv, t = 16, 2, 5000
    k, v = syn.kv_pair(heads=hkv, tokens=t, head_dim=128, variant=8)
    kc, ks = gpu_lib.fp8_kv_quantize(k.to(DEV))
    vc, vs = gpu_lib.fp8_kv_quantize(v.to(DEV))
    q = syn.decode_queries(heads_q=hq, variant=8).to(DEV)
    need = lib.fp8_kv_decode_attention_workspace_size(hq, t)
    ws = Guarded(1, need, need, torch.uint8)
    for dtype, ld in ((torch.bfloat16, 136), (torch.float32, 132)):
        o = Guarded(hq, 128, ld, dtype)
        gpu_lib.fp8_kv_decode_attention(q, kc, ks, vc, vs, 1 / 128 ** 0.5, out_dtype=dtype, out=o.view,
                                        workspace=ws.view[0])
        o.check(f"attention output {dtype}")
        ws.check("attention workspace")
