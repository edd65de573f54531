"""The decode-shaped steps under HIP graph capture.

No entry point allocates, copies or clears memory on the device: each call is
its kernels on the caller's stream, so a caller may capture a whole step into
a graph and replay it, which removes the host's per-call cost that dominates
these latency-bound shapes. Each test captures a step with every output
preallocated, then replays the graph several times with new input values
copied into the captured input buffers, with eager calls and
synchronizations between the replays, and checks every replay bit for bit
against the same calls made eagerly on the same input.
"""

import pytest
import torch

import synth_inputs as syn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _capture(step):
    """A graph of one call of ``step`` on a side stream (after a warm-up call
    there, as torch's capture requires)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(g, x_static, inputs, outputs, eager):
    """For each input: copy it into the captured buffer, replay, and compare
    every output with the eager step on that input."""
    for i, x in enumerate(inputs):
        x_static.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        ref = eager(x)   # eager work between the replays
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert a.shape == b.shape
            if a.dtype in (torch.float32, torch.bfloat16):
                assert torch.equal(_bits(a), _bits(b)), f"replay {i}: output {k} differs from the eager step"
            else:
                assert torch.equal(a, b), f"replay {i}: output {k} differs from the eager step"


def test_per_tensor_two_call_step(gpu_lib):
    """Config 1 as two calls: the per-tensor quantize, then the GEMM."""
    c = syn.CONFIGS[1]
    M, N, K = c["M"], c["N"], c["K"]
    qw, sw = gpu_lib.fp8_quantize(syn.weights(1).to(DEV), "per_tensor")
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    x.copy_(syn.activations(1).to(DEV))
    qa = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        gpu_lib.fp8_quantize(x, "per_tensor", out=qa, scales=sa)
        gpu_lib.fp8_block_gemm(qa, sa, "per_tensor", qw, sw, "per_tensor", out=y)

    def eager(xi):
        q2, s2 = gpu_lib.fp8_quantize(xi, "per_tensor")
        return [q2, s2, gpu_lib.fp8_block_gemm(q2, s2, "per_tensor", qw, sw, "per_tensor")]

    g = _capture(step)
    inputs = [syn.activations(1, variant=v).to(DEV) for v in (1, 2, 3)]
    inputs.append(inputs[0] * 1e-3)   # a different scale
    _replay_and_compare(g, x, inputs, [qa, sa, y], eager)


@pytest.mark.parametrize("gran_a", ["per_tensor", "group_1x128"])
def test_fused_decode_call(gpu_lib, gran_a):
    """fp8_quantize_gemm_decode with its codes and scales returned."""
    M, N, K = (64, 512, 512) if gran_a == "per_tensor" else (16, 2048, 4096)
    cfg = 1 if gran_a == "per_tensor" else 3
    w = syn.weights(cfg, N=N, K=K).to(DEV)
    qw, sw = gpu_lib.fp8_quantize(w, "block_128x128")
    x = syn.activations(cfg, M=M, K=K).to(DEV).clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = (torch.empty(1, dtype=torch.float32, device=DEV) if gran_a == "per_tensor"
         else torch.empty((M, K // 128), dtype=torch.float32, device=DEV))

    def step():
        gpu_lib.fp8_quantize_gemm_decode(x, qw, sw, "block_128x128", gran_a=gran_a, out=y, codes=q, scales=s)

    def eager(xi):
        y2, q2, s2 = gpu_lib.fp8_quantize_gemm_decode(xi, qw, sw, "block_128x128", gran_a=gran_a,
                                                      return_codes=True)
        return [y2, q2, s2]

    g = _capture(step)
    inputs = [syn.activations(cfg, M=M, K=K, variant=v).to(DEV) for v in (4, 5, 6)]
    _replay_and_compare(g, x, inputs, [y, q, s], eager)


def test_decode_step_on_packed_weights(gpu_lib):
    """The 1x128 decode step as two calls on decode-packed weights."""
    M, N, K = 16, 2048, 4096
    qw, sw = gpu_lib.fp8_quantize(syn.weights(3, N=N, K=K).to(DEV), "block_128x128")
    pk = gpu_lib.fp8_pack_weights_decode(qw)
    x = syn.activations(3, M=M, K=K).to(DEV).clone()
    qa = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sa = torch.empty((K // 128, M), dtype=torch.float32, device=DEV).t()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        gpu_lib.fp8_quantize(x, "group_1x128", out=qa, scales=sa)
        gpu_lib.fp8_block_gemm_packed(qa, sa, "group_1x128", pk, sw, "block_128x128", out=y)

    def eager(xi):
        q2, s2 = gpu_lib.fp8_quantize(xi, "group_1x128", scale_layout="kmajor")
        return [q2, s2, gpu_lib.fp8_block_gemm_packed(q2, s2, "group_1x128", pk, sw, "block_128x128")]

    g = _capture(step)
    inputs = [syn.activations(3, M=M, K=K, variant=v).to(DEV) for v in (7, 8, 9)]
    _replay_and_compare(g, x, inputs, [qa, sa, y], eager)
