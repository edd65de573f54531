#!/usr/bin/env python3
"""Benchmark of the W8A8 FP8 hot path on one MI355X (gfx950).

Workload (one "step"): the Llama-3-70B fused QKV projection prefill, M = 8192
tokens, K = 8192, N = 10240 ((64 + 2 x 8) heads x 128), the largest
configuration:

  1. dynamic activation quantization of a bf16 [8192, 8192] tensor with one
     scale per 1 x 128 token group (fp8_quantize, K-block-major scales);
  2. the block-scaled FP8 GEMM against E4M3 weights with 128 x 128 block
     scales, fp32 accumulation, bf16 output (fp8_block_gemm).

The weights are quantized once beforehand (offline, as the method prescribes)
and that pass is timed separately. Inputs are seeded synthetic tensors of the
workload's shapes and value structure (synth_inputs), resident in HBM before
timing starts; activation buffers are rotated through 3 copies (more than the
256 MB Infinity Cache) so the quantize pass reads HBM.

Printed: one JSON line. ``value`` is the step's throughput in TFLOP/s
(2 M N K per step over the step time, quantize included); ``roofline`` is the
GEMM kernel's achieved TFLOP/s against the dense FP8 MFMA peak, from HIP event
pairs around each GEMM launch of the timed steps on the launch stream;
``passes`` lists the other passes of every configuration with their own time
and GB/s or TFLOP/s: the 4096 x 14336 x 4096 prefill GEMM and its variants,
the activation quantizers (1x128, per tensor, static, MX), the offline weight
passes, the per-tensor 64 x 512 x 512 calls in microseconds, the KV-cache
passes and decode attention at [8, 131072, 128], and the decode-shaped GEMM
16 x 28672 x 8192 on row-major and on decode-packed weights; ``clocks`` gives
the shader and memory clock levels the driver reported while the untimed
settle phase ran the step; ``cpu_baseline`` times the CPU oracle on the same
step.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=1.5,
                    help="seconds of untimed steps run first, so the GPU clock has left its idle state")
    ap.add_argument("--no-secondary", action="store_true", help="skip the KV and decode passes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["gemm", "quant", "prefill2", "mx", "small", "kv", "decode", "copy"],
                    default=None,
                    help="time one group of passes only (for profiling runs): 'gemm' the timed step's "
                         "GEMM, 'quant' the quantizers, 'prefill2' the 4096 x 14336 x 4096 GEMMs, 'small' "
                         "the per-tensor 64 x 512 x 512 calls; 'copy' times a plain 512 MB device copy, the "
                         "calibration kernel for the HBM byte counters")
    return ap.parse_args()


class Timer:
    """HIP events on the current stream, which is the stream every fp8blk call
    is launched on (the binding passes torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.stats = {}

    def run(self, fn, iters: int, warmup: int = 2, name: str = None) -> float:
        """Mean seconds per call over `iters` back-to-back calls bracketed by one
        event pair; with `name`, a second loop with an event pair around every
        call records median / min / p90 under self.stats[name]."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(iters):
            fn(i)
        e1.record(st)
        torch.cuda.synchronize()
        mean = e0.elapsed_time(e1) / iters * 1e-3
        if name is not None:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(iters)]
            for i, (a, b) in enumerate(ev):
                a.record(st)
                fn(i)
                b.record(st)
            torch.cuda.synchronize()
            t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
            self.stats[name] = {"median_us": t[len(t) // 2], "min_us": t[0],
                                "p90_us": t[min(len(t) - 1, (9 * len(t)) // 10)], "calls": len(t)}
        return mean

    def run_queued(self, fn, iters: int):
        """Device seconds per call with the calls already queued: a spin kernel
        (torch.cuda._sleep) holds the stream while the host enqueues every
        call, so the event pair around them times the device running them back
        to back, without the host's per-call cost. The spin is sized to twice
        the host's measured enqueue time; returns (seconds per call, True if
        the host finished enqueueing before the spin was over)."""
        torch = self.torch
        st = torch.cuda.current_stream()
        # spin cycles per microsecond of device time
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        torch.cuda._sleep(2_000_000)
        e1.record(st)
        torch.cuda.synchronize()
        cycles_per_us = 2_000_000 / max(e0.elapsed_time(e1) * 1e3, 1.0)
        # the host's enqueue time for `iters` calls
        h0 = time.perf_counter()
        for i in range(iters):
            fn(i)
        host_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        spin_us = 2.0 * host_s * 1e6 + 500.0
        torch.cuda._sleep(int(spin_us * cycles_per_us))
        h0 = time.perf_counter()
        e0.record(st)
        for i in range(iters):
            fn(i)
        e1.record(st)
        queued = (time.perf_counter() - h0) * 1e6 < spin_us
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e-3, queued


# HBM bytes per launch of the step's GEMM kernel (M = 8192, N = 10240,
# K = 8192), read from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
# and scaled by what the same counters read for a plain device copy of known
# size (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0). Valid only for the kernel source
# they were taken on: the key is the SHA-256 of the GEMM source files' code
# (comments and blank lines removed); any other code gives null.
GEMM_COUNTERS = {
    "sources_sha256": "75371f8ba725b1258b9cc63f0df6bc98a6ff29dcf1f70c2d102f454b607d1403",
    "fetch_kib": 530863.7,
    "write_kib": 163911.3,
}
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0


def gemm_source_sha256() -> str:
    """SHA-256 of the GEMM's source files with comments and blank lines
    removed, so that a change of wording in a comment keeps the counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("gemm.hip", "device_common.h", "internal.h"):
        with open(os.path.join(ROOT, "fp8_quantization_block_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
        h.update(code.encode("utf-8"))
    return h.hexdigest()


def gemm_traffic_bytes():
    c = GEMM_COUNTERS
    if c["sources_sha256"] is None or c["sources_sha256"] != gemm_source_sha256():
        return None
    return (c["fetch_kib"] * FETCH_FACTOR + c["write_kib"] * WRITE_FACTOR) * 1024.0


class ClockSampler:
    """Samples the device's current shader, memory and fabric clock levels
    (MHz) from the amdgpu driver's DPM tables in sysfs (the level marked '*')
    every 0.1 s on a background thread, e.g. while the settle phase keeps the
    GPU busy. Reports None where sysfs does not expose the tables."""

    KEYS = ("sclk", "mclk", "fclk")

    def __init__(self, torch):
        self.base = None
        try:
            p = torch.cuda.get_device_properties(0)
            self.base = (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
                         f"{p.pci_device_id:02x}.0")
        except Exception:
            pass
        self.samples = {k: [] for k in self.KEYS}
        self._stop = None
        self._thread = None

    def read(self):
        import re
        out = {}
        if self.base is None:
            return out
        for k in self.KEYS:
            try:
                with open(os.path.join(self.base, f"pp_dpm_{k}")) as fh:
                    text = fh.read()
            except OSError:
                continue
            m = re.search(r"(\d+)\s*mhz\s*\*", text, re.I)
            if m:
                out[k] = int(m.group(1))
        return out

    def _run(self):
        while not self._stop.wait(0.1):
            for k, v in self.read().items():
                self.samples[k].append(v)

    def start(self):
        import threading
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=5)

    def summary(self):
        res = {}
        for k, v in self.samples.items():
            if v:
                v = sorted(v)
                res[f"{k}_mhz_median"] = v[len(v) // 2]
                res[f"{k}_mhz_min"] = v[0]
                res[f"{k}_mhz_max"] = v[-1]
        if not res:
            return None
        res["samples"] = max(len(v) for v in self.samples.values())
        res["source"] = "sysfs pp_dpm_* current level, sampled every 0.1 s during the untimed settle phase"
        return res


def sha256_of(t) -> str:
    """SHA-256 of a CPU bf16 tensor's bytes, read as int16 (numpy has no
    bf16), so that a run's seeded inputs can be checked against another's."""
    import hashlib
    import torch
    return hashlib.sha256(t.contiguous().view(torch.int16).numpy().tobytes()).hexdigest()


def settle(torch, fn, seconds: float) -> None:
    """Untimed launches of `fn` for about `seconds` of wall time. An idle GPU
    starts at a low clock and needs a fraction of a second of sustained load to
    reach its working clock; without this the first timed calls run slower."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "measured at one GPU's full share of the workload, and the path would shard by rows, "
              "weight columns or kv heads with no exchange", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth_inputs as syn
    import fp8_quantization_block_amd as fp8

    fp8.load_library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    timer = Timer(torch)
    if args.only == "copy":
        copy_calibration(torch, timer, dev)
        return
    c = syn.CONFIGS[4]
    M, N, K = c["M"], c["N"], c["K"]
    print(f"# bench: {c['workload']} on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    # ---- the step's inputs, resident in HBM ---------------------------------
    # 3 rotating activation sets of 134 MB bf16 + 67 MB codes: more than the
    # 256 MB Infinity Cache, so the quantize pass reads HBM
    a_host = syn.activations(4)
    w_host = syn.weights(4)
    inputs_sha256 = {"activations_bf16": sha256_of(a_host), "weights_bf16": sha256_of(w_host)}
    w = w_host.to(dev)
    del w_host
    nsets = 3
    a_sets = [a_host.to(dev) for _ in range(nsets)]
    qa_sets = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sa_sets = [torch.empty((K // 128, M), dtype=torch.float32, device=dev).t() for _ in range(nsets)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    # the offline weight pass rotates 3 copies of the 168 MB weights
    w_sets = [w, w.clone(), w.clone()]

    def quant_w(i):
        fp8.fp8_quantize(w_sets[i % 3], "block_128x128", out=qw, scales=sw)

    def quant_a(i):
        j = i % nsets
        fp8.fp8_quantize(a_sets[j], "group_1x128", out=qa_sets[j], scales=sa_sets[j])

    def gemm(i):
        j = i % nsets
        fp8.fp8_block_gemm(qa_sets[j], sa_sets[j], "group_1x128", qw, sw, "block_128x128", out=out)

    def step(i):
        quant_a(i)
        gemm(i)

    quant_w(0)
    for i in range(nsets):
        quant_a(i)
    torch.cuda.synchronize()
    clocks = ClockSampler(torch)
    clocks.start()
    settle(torch, step, args.settle_s)
    clocks.stop()

    # ---- the timed step: warmup, then exactly `steps` steps ---------------
    # Timed first, straight after the settle phase (after a stretch of lighter
    # passes the power controller lets the clock rise and then cuts it back
    # hard once the GEMM resumes). An event pair around each GEMM launch, on
    # the launch stream, gives the GEMM kernel's own duration inside the timed
    # region, from which the roofline is computed.
    flops = 2.0 * M * N * K
    t_step = t_gemm = None
    if args.only in (None, "gemm"):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        ev = lambda: torch.cuda.Event(enable_timing=True)
        e0, e1 = ev(), ev()
        g_ev = [(ev(), ev()) for _ in range(args.steps)]
        wall0 = time.perf_counter()
        e0.record(st)
        for i in range(args.steps):
            quant_a(i)
            g_ev[i][0].record(st)
            gemm(i)
            g_ev[i][1].record(st)
        e1.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        t_step = e0.elapsed_time(e1) * 1e-3 / args.steps
        g_us = sorted(a.elapsed_time(b) * 1e3 for a, b in g_ev)
        t_gemm = sum(g_us) / len(g_us) * 1e-6
        timer.stats["gemm_8192x10240x8192_in_step"] = {"median_us": g_us[len(g_us) // 2], "min_us": g_us[0],
                                                       "p90_us": g_us[min(len(g_us) - 1, (9 * len(g_us)) // 10)],
                                                       "calls": len(g_us)}
        print(f"# timed {args.steps} steps: {t_step * 1e6:.1f} us/step, GEMM {t_gemm * 1e6:.1f} us "
              f"(wall {wall:.3f} s)", file=sys.stderr, flush=True)

    passes = {}
    if t_gemm is not None:
        passes["gemm_8192x10240x8192"] = {"us": t_gemm * 1e6, "TFLOP/s": flops / t_gemm / 1e12,
                                          "frac_fp8_peak": flops / t_gemm / 1e12 / PEAK_FP8_TFLOPS,
                                          "timing": "mean of the event pairs around each GEMM of the timed steps"}
    if args.only in (None, "quant"):
        t_qa = timer.run(quant_a, 30, warmup=args.warmup, name="act_quant_1x128_8192x8192")
        bytes_qa = M * K * 2 + M * K + M * (K // 128) * 4
        passes["act_quant_1x128_8192x8192"] = {"us": t_qa * 1e6, "GB/s": bytes_qa / t_qa / 1e9,
                                               "frac_hbm": bytes_qa / t_qa / 1e9 / PEAK_HBM_GBPS}
        t_qw = timer.run(quant_w, 12, warmup=3, name="weight_quant_128x128_offline_10240x8192")
        bytes_qw = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
        passes["weight_quant_128x128_offline_10240x8192"] = {
            "us": t_qw * 1e6, "GB/s": bytes_qw / t_qw / 1e9, "frac_hbm": bytes_qw / t_qw / 1e9 / PEAK_HBM_GBPS}
    ceiling = None
    if args.only is None:
        ceiling = mfma_ceiling(torch, dev, qa_sets[0], qw)
        if ceiling and t_gemm:
            ceiling["gemm_frac_of_mfma_plus_4_fma"] = flops / t_gemm / 1e12 / ceiling["mfma_plus_4_fma"]
    del a_sets, qa_sets, sa_sets, w_sets, w, out

    if not args.no_secondary and args.only in (None, "prefill2", "mx", "quant"):
        passes.update(passes_config2(args, torch, syn, fp8, timer, dev))
    if not args.no_secondary and args.only in (None, "small"):
        passes.update(passes_config1(args, torch, syn, fp8, timer, dev))
    if not args.no_secondary and args.only in (None, "kv"):
        passes.update(passes_kv(args, torch, syn, fp8, timer, dev))
    if not args.no_secondary and args.only in (None, "decode"):
        passes.update(passes_decode(args, torch, syn, fp8, timer, dev))

    # ---- CPU oracle on the same step ------------------------------------------
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(syn, qw.cpu().numpy(), sw.cpu().numpy(), M, N, K)

    result = {
        "metric": "block-scaled FP8 GEMM TFLOP/s (%FP8 MFMA peak) + quantize/KV GB/s (%HBM)",
        "value": (flops / t_step / 1e12) if t_step else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (t_step * 1e3) if t_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-mfma/fp32-acc/bf16-out",
        "data": "synthetic (seeded Llama-3-70B QKV-shaped activations with outlier channels, N(0,0.02) weights)",
        "config": {"workload": c["workload"], "M": M, "N": N, "K": K,
                   "act_scales": "1x128 dynamic", "weight_scales": "128x128", "parallelism": "single-gpu"},
        "roofline": None if t_gemm is None else {
            "kernel": "k_gemm_fp8_block (fp8_block_gemm), 8192 x 10240 x 8192",
            "bound": "mfma",
            "achieved": flops / t_gemm / 1e12,
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": flops / t_gemm / 1e12 / PEAK_FP8_TFLOPS,
            "traffic": gemm_traffic_bytes(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
            "algorithmic_bytes": float(M * K + N * K + 2 * M * N + 4 * (M * (K // 128) + (N // 128) * (K // 128))),
        },
        "inputs_sha256": inputs_sha256,
        "passes": passes,
        "mfma_ceiling": ceiling,
        "clocks": clocks.summary(),
        "per_call": timer.stats,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def passes_config2(args, torch, syn, fp8, timer, dev):
    """Llama-3-8B MLP up/gate prefill, 4096 x 14336 x 4096: the GEMM and its
    variants (output quantized in the epilogue, E5M2 activations, MX operands),
    and the activation quantizers at [4096, 4096] (1x128, per tensor, static
    with the amax recorded), plus the offline weight pass."""
    c = syn.CONFIGS[2]
    M, N, K = c["M"], c["N"], c["K"]
    flops = 2.0 * M * N * K
    res = {}
    a_host = syn.activations(2)
    w = syn.weights(2).to(dev)
    nsets = 11   # 11 x 50.9 MB: more than the Infinity Cache
    a_sets = [a_host.to(dev) for _ in range(nsets)]
    qa_sets = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sa_sets = [torch.empty((K // 128, M), dtype=torch.float32, device=dev).t() for _ in range(nsets)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qw, sw = fp8.fp8_quantize(w, "block_128x128")
    w_sets = [w, w.clone(), w.clone()]

    def quant_a(i):
        j = i % nsets
        fp8.fp8_quantize(a_sets[j], "group_1x128", out=qa_sets[j], scales=sa_sets[j])

    def gemm(i):
        j = i % nsets
        fp8.fp8_block_gemm(qa_sets[j], sa_sets[j], "group_1x128", qw, sw, "block_128x128", out=out)

    for i in range(nsets):
        quant_a(i)
    if args.only in (None, "prefill2"):
        # after the lighter passes before it the clock first overshoots, then
        # drops hard once the GEMM load resumes: settle it again before timing
        settle(torch, gemm, args.settle_s)
        t_g = timer.run(gemm, 30, warmup=args.warmup, name="gemm_4096x14336x4096")
        res["gemm_4096x14336x4096"] = {"us": t_g * 1e6, "TFLOP/s": flops / t_g / 1e12,
                                       "frac_fp8_peak": flops / t_g / 1e12 / PEAK_FP8_TFLOPS}
        # the GEMM's output quantized for the next layer (1 x 128 groups along
        # N) in the GEMM epilogue, against the bf16 GEMM followed by the
        # stand-alone quantizer over its output
        qc = torch.empty((M, N), dtype=torch.uint8, device=dev)
        scq = torch.empty((N // 128, M), dtype=torch.float32, device=dev).t()

        def fused(i):
            j = i % nsets
            fp8.fp8_block_gemm_quant(qa_sets[j], sa_sets[j], "group_1x128", qw, sw, "block_128x128",
                                     out=qc, scales=scq)

        def unfused(i):
            gemm(i)
            fp8.fp8_quantize(out, "group_1x128", out=qc, scales=scq)

        t_f = timer.run(fused, 20, warmup=args.warmup, name="gemm_fused_quant_out")
        t_u = timer.run(unfused, 20, warmup=args.warmup, name="gemm_then_quantize_out")
        res["gemm_fused_quant_out_4096x14336x4096"] = {"us": t_f * 1e6, "TFLOP/s": flops / t_f / 1e12,
                                                       "frac_fp8_peak": flops / t_f / 1e12 / PEAK_FP8_TFLOPS}
        res["gemm_then_quantize_out_4096x14336x4096"] = {"us": t_u * 1e6, "TFLOP/s": flops / t_u / 1e12}
        del qc, scq
        # E5M2 activations (1x128) against the E4M3 weights
        qa5 = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sa5 = torch.empty((K // 128, M), dtype=torch.float32, device=dev).t()
        fp8.fp8_quantize(a_sets[0], "group_1x128", fmt="e5m2", out=qa5, scales=sa5)

        def gemm5(i):
            fp8.fp8_block_gemm(qa5, sa5, "group_1x128", qw, sw, "block_128x128", out=out, fmt_a="e5m2")

        t5 = timer.run(gemm5, 20, warmup=args.warmup, name="gemm_e5m2_act")
        res["gemm_e5m2_act_4096x14336x4096"] = {"us": t5 * 1e6, "TFLOP/s": flops / t5 / 1e12,
                                                "frac_fp8_peak": flops / t5 / 1e12 / PEAK_FP8_TFLOPS}
        del qa5, sa5
    if args.only in (None, "mx", "prefill2"):
        # MX operands (E4M3 codes, one power-of-two scale per 32 K elements),
        # the scales applied inside the scaled MFMA
        qamx = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(nsets)]
        samx = [torch.empty((M, K // 32), dtype=torch.uint8, device=dev) for _ in range(nsets)]
        qwmx, swmx = fp8.fp8_quantize_mx(w)

        def quant_mx(i):
            j = i % nsets
            fp8.fp8_quantize_mx(a_sets[j], out=qamx[j], scales=samx[j])

        def gemm_mx(i):
            j = i % nsets
            fp8.fp8_mx_gemm(qamx[j], samx[j], qwmx, swmx, out=out)

        for i in range(nsets):
            quant_mx(i)
        t_qmx = timer.run(quant_mx, 33, warmup=args.warmup, name="act_quant_mx32")
        t_gmx = timer.run(gemm_mx, 20, warmup=args.warmup, name="gemm_mx32")
        bytes_qmx = M * K * 2 + M * K + M * (K // 32)
        res["act_quant_mx32_4096x4096"] = {"us": t_qmx * 1e6, "GB/s": bytes_qmx / t_qmx / 1e9,
                                           "frac_hbm": bytes_qmx / t_qmx / 1e9 / PEAK_HBM_GBPS}
        res["gemm_mx32_4096x14336x4096"] = {"us": t_gmx * 1e6, "TFLOP/s": flops / t_gmx / 1e12,
                                            "frac_fp8_peak": flops / t_gmx / 1e12 / PEAK_FP8_TFLOPS}
        del qamx, samx, qwmx, swmx
    if args.only in (None, "quant"):
        t_qa = timer.run(quant_a, 33, warmup=args.warmup, name="act_quant_1x128_4096x4096")
        bytes_qa = M * K * 2 + M * K + M * (K // 128) * 4
        res["act_quant_1x128_4096x4096"] = {"us": t_qa * 1e6, "GB/s": bytes_qa / t_qa / 1e9,
                                            "frac_hbm": bytes_qa / t_qa / 1e9 / PEAK_HBM_GBPS}
        # per-tensor dynamic scaling: amax pass, then the cast (the tensor is
        # read twice; algorithmic bytes count it once)
        s_pt = torch.empty(1, dtype=torch.float32, device=dev)

        def quant_pt(i):
            j = i % nsets
            fp8.fp8_quantize(a_sets[j], "per_tensor", out=qa_sets[j], scales=s_pt)

        t_pt = timer.run(quant_pt, 33, warmup=args.warmup, name="act_quant_per_tensor_4096x4096")
        bytes_pt = M * K * 2 + M * K + 4
        res["act_quant_per_tensor_4096x4096"] = {"us": t_pt * 1e6, "GB/s": bytes_pt / t_pt / 1e9,
                                                 "frac_hbm": bytes_pt / t_pt / 1e9 / PEAK_HBM_GBPS}
        # delayed scaling: the cast under a scale from the amax history,
        # recording this tensor's amax into the history
        hist = torch.full((16,), float(a_host.float().abs().max()), dtype=torch.float32, device=dev)
        s_static = fp8.fp8_scale_from_amax_history(hist)

        def quant_static(i):
            j = i % nsets
            fp8.fp8_quantize_static(a_sets[j], s_static, record_amax=True, out=qa_sets[j],
                                    amax=hist[i % 16:i % 16 + 1])

        t_qs = timer.run(quant_static, 33, warmup=args.warmup, name="act_quant_static_4096x4096")
        bytes_qs = M * K * 2 + M * K
        res["act_quant_static_amax_4096x4096"] = {"us": t_qs * 1e6, "GB/s": bytes_qs / t_qs / 1e9,
                                                  "frac_hbm": bytes_qs / t_qs / 1e9 / PEAK_HBM_GBPS}

        def quant_w(i):
            fp8.fp8_quantize(w_sets[i % 3], "block_128x128", out=qw, scales=sw)

        t_qw = timer.run(quant_w, 12, warmup=3, name="weight_quant_128x128_offline_14336x4096")
        bytes_qw = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
        res["weight_quant_128x128_offline_14336x4096"] = {
            "us": t_qw * 1e6, "GB/s": bytes_qw / t_qw / 1e9, "frac_hbm": bytes_qw / t_qw / 1e9 / PEAK_HBM_GBPS}
    return res


def passes_config1(args, torch, syn, fp8, timer, dev):
    """Per-tensor E4M3 at 64 x 512 x 512: latency-bound, so microseconds per
    call and no roofline claim: the median of per-call event pairs and the
    mean of back-to-back calls (both include the host's per-call cost when it
    exceeds the device's), and the device's own back-to-back time with the
    calls queued behind a spin (Timer.run_queued). The step is
    the activation quantize (amax pass, scale, cast) then the GEMM, as two
    calls and as the one-launch fp8_quantize_gemm_decode; the weight quantize
    is the offline pass."""
    c = syn.CONFIGS[1]
    M, N, K = c["M"], c["N"], c["K"]
    a = syn.activations(1).to(dev)
    w = syn.weights(1).to(dev)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty(1, dtype=torch.float32, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def qa_call(i):
        fp8.fp8_quantize(a, "per_tensor", out=qa, scales=sa)

    def qw_call(i):
        fp8.fp8_quantize(w, "per_tensor", out=qw, scales=sw)

    def gemm(i):
        fp8.fp8_block_gemm(qa, sa, "per_tensor", qw, sw, "per_tensor", out=out)

    def step(i):
        qa_call(i)
        gemm(i)

    def fused_step(i):
        fp8.fp8_quantize_gemm_decode(a, qw, sw, "per_tensor", out=out)

    qw_call(0)
    qa_call(0)
    res = {}
    for name, fn in (("act_quant", qa_call), ("weight_quant_offline", qw_call), ("gemm", gemm),
                     ("step_act_quant_and_gemm", step), ("step_fused_one_launch", fused_step)):
        key = f"per_tensor_64x512x512_{name}"
        t = timer.run(fn, 200, warmup=20, name=key)
        tq, queued = timer.run_queued(fn, 200)
        res[key] = {"us_per_call_median": timer.stats[key]["median_us"],
                    "us_back_to_back": t * 1e6,
                    "us_device_back_to_back": tq * 1e6 if queued else None,
                    "note": "latency-bound; no roofline claim"}
    return res


def passes_kv(args, torch, syn, fp8, timer, dev):
    """FP8 KV cache, K and V [8, 131072, 128]: quantize and dequantize in E4M3
    and E5M2, and decode attention of 64 query heads over the codes."""
    c5 = syn.CONFIGS[5]
    kh, vh = syn.kv_pair(5)
    kd, vd = kh.to(dev), vh.to(dev)
    del kh, vh
    H, T, D = c5["heads"], c5["tokens"], c5["head_dim"]
    qk = torch.empty((H, T, D), dtype=torch.uint8, device=dev)
    qv = torch.empty_like(qk)
    sk = torch.empty((H, T // 128), dtype=torch.float32, device=dev)
    sv = torch.empty_like(sk)
    ok = torch.empty((H, T, D), dtype=torch.bfloat16, device=dev)
    ov = torch.empty_like(ok)
    lib = fp8.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    n = 2 * H * T * D
    kv_bytes = n * 2 + n + 2 * H * (T // 128) * 4
    # E4M3 (the default KV format) and E5M2 (the KV format of the serving
    # recipe on the pages); same bytes, same kernels up to the conversion
    for fmt, tag in ((fp8.E4M3, ""), (fp8.E5M2, "_e5m2")):
        def kvq(i, fmt=fmt):
            fp8._check(lib.fp8_kv_quantize(kd.data_ptr(), H, T, D, T * D, D, 128, fmt, qk.data_ptr(),
                                           sk.data_ptr(), stream))
            fp8._check(lib.fp8_kv_quantize(vd.data_ptr(), H, T, D, T * D, D, 128, fmt, qv.data_ptr(),
                                           sv.data_ptr(), stream))

        def kvd(i, fmt=fmt):
            fp8._check(lib.fp8_kv_dequantize(qk.data_ptr(), sk.data_ptr(), H, T, D, 128, fmt, ok.data_ptr(),
                                             stream))
            fp8._check(lib.fp8_kv_dequantize(qv.data_ptr(), sv.data_ptr(), H, T, D, 128, fmt, ov.data_ptr(),
                                             stream))

        t_kvq = timer.run(kvq, 20, warmup=3, name="kv_quant_K+V" + tag)
        t_kvd = timer.run(kvd, 20, warmup=3, name="kv_dequant_K+V" + tag)
        res["kv_quant_K+V_8x131072x128" + tag] = {"us": t_kvq * 1e6, "GB/s": kv_bytes / t_kvq / 1e9,
                                                  "frac_hbm": kv_bytes / t_kvq / 1e9 / PEAK_HBM_GBPS}
        res["kv_dequant_K+V_8x131072x128" + tag] = {"us": t_kvd * 1e6, "GB/s": kv_bytes / t_kvd / 1e9,
                                                    "frac_hbm": kv_bytes / t_kvd / 1e9 / PEAK_HBM_GBPS}
        # decode attention of 64 query heads (8 per kv head) over the codes
        # just written: algorithmic bytes = both code tensors, their scales,
        # the bf16 query and output
        hq = c5["heads_q"]
        qd = syn.decode_queries(heads_q=hq).to(dev)
        od = torch.empty((hq, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(lib.fp8_kv_decode_attention_workspace_size(hq, T), dtype=torch.uint8, device=dev)
        # two copies of the 268 MB cache, alternated: more than the Infinity
        # Cache, so the codes stream from HBM
        caches = [(qk, sk, qv, sv), (qk.clone(), sk, qv.clone(), sv)]

        # through the C ABI, like the quantize calls above: the binding's
        # per-call shape checks would otherwise add host time to a 50 us call
        def att(i, fmt=fmt):
            ck, cks, cv, cvs = caches[i % 2]
            fp8._check(lib.fp8_kv_decode_attention(qd.data_ptr(), D, hq, H, T, D, ck.data_ptr(), cks.data_ptr(),
                                                   cv.data_ptr(), cvs.data_ptr(), 128, fmt, 1.0 / 128 ** 0.5,
                                                   od.data_ptr(), fp8.BF16, D, ws.data_ptr(), ws.numel(), stream))

        att_bytes = n + 2 * H * (T // 128) * 4 + 2 * hq * D * 2
        t_att = timer.run(att, 20, warmup=3, name="kv_decode_attention" + tag)
        res["kv_decode_attention_64q_8x131072x128" + tag] = {
            "us": t_att * 1e6, "GB/s": att_bytes / t_att / 1e9, "frac_hbm": att_bytes / t_att / 1e9 / PEAK_HBM_GBPS}
        del qd, od, ws, caches
    return res


def passes_decode(args, torch, syn, fp8, timer, dev):
    """Llama-3-70B MLP up, decode shape 16 x 28672 x 8192: the offline 128x128
    weight quantization (2 rotating copies of the 470 MB bf16 weights), the
    HBM-bound GEMM on row-major and on decode-packed weights (3 rotating copies
    of the 235 MB codes), the whole step from bf16 activations (1x128 quantize
    then GEMM, and the two in one launch) on both weight layouts, the packing
    pass, and the [16, 8192] activation quantize."""
    c3 = syn.CONFIGS[3]
    m3, n3, k3 = c3["M"], c3["N"], c3["K"]
    a3 = syn.activations(3).to(dev)
    w3 = syn.weights(3).to(dev)
    qa3, sa3 = fp8.fp8_quantize(a3, "group_1x128", scale_layout="kmajor")
    qw3, sw3 = fp8.fp8_quantize(w3, "block_128x128")
    res = {}

    w3_sets = [w3, w3.clone()]
    qw3_out = [torch.empty_like(qw3) for _ in range(2)]
    sw3_out = [torch.empty_like(sw3) for _ in range(2)]

    def wq_call(i):
        fp8.fp8_quantize(w3_sets[i % 2], "block_128x128", out=qw3_out[i % 2], scales=sw3_out[i % 2])

    t_wq = timer.run(wq_call, 10, warmup=2, name="weight_quant_128x128_offline_28672x8192")
    bytes_wq = n3 * k3 * 2 + n3 * k3 + (n3 // 128) * (k3 // 128) * 4
    res["weight_quant_128x128_offline_28672x8192"] = {"us": t_wq * 1e6, "GB/s": bytes_wq / t_wq / 1e9,
                                                      "frac_hbm": bytes_wq / t_wq / 1e9 / PEAK_HBM_GBPS}
    del w3, w3_sets, qw3_out, sw3_out

    def qa_call(i):
        fp8.fp8_quantize(a3, "group_1x128", out=qa3, scales=sa3)

    timer.run(qa_call, 200, warmup=20, name="act_quant_1x128_16x8192")
    res["act_quant_1x128_16x8192"] = {"us_per_call_median": timer.stats["act_quant_1x128_16x8192"]["median_us"],
                                      "note": "0.4 MB: latency-bound; no roofline claim"}
    o3 = torch.empty((m3, n3), dtype=torch.bfloat16, device=dev)
    qw3_sets = [qw3, qw3.clone(), qw3.clone()]

    def dec(i):
        fp8.fp8_block_gemm(qa3, sa3, "group_1x128", qw3_sets[i % 3], sw3, "block_128x128", out=o3)

    t_dec = timer.run(dec, 50, warmup=5, name="decode_gemm_16x28672x8192")
    dec_bytes = m3 * k3 + n3 * k3 + 4 * (m3 * (k3 // 128) + (n3 // 128) * (k3 // 128)) + 2 * m3 * n3
    res["decode_gemm_16x28672x8192"] = {"us": t_dec * 1e6, "GB/s": dec_bytes / t_dec / 1e9,
                                        "frac_hbm": dec_bytes / t_dec / 1e9 / PEAK_HBM_GBPS,
                                        "TFLOP/s": 2.0 * m3 * n3 * k3 / t_dec / 1e12}
    # the whole decode step from bf16 activations: the 1x128 quantize then the
    # GEMM, and the two in one launch (fp8_quantize_gemm_decode); bytes of the
    # fused step: x in bf16 instead of codes and scales
    fused_bytes = 2 * m3 * k3 + n3 * k3 + 4 * (n3 // 128) * (k3 // 128) + 2 * m3 * n3

    def step_two(i):
        qa_call(i)
        dec(i)

    def step_fused(i):
        fp8.fp8_quantize_gemm_decode(a3, qw3_sets[i % 3], sw3, "block_128x128", gran_a="group_1x128", out=o3)

    for key, fn in (("decode_step_quantize_then_gemm_16x28672x8192", step_two),
                    ("decode_step_fused_16x28672x8192", step_fused)):
        t = timer.run(fn, 50, warmup=5, name=key)
        res[key] = {"us": t * 1e6, "GB/s": fused_bytes / t / 1e9, "frac_hbm": fused_bytes / t / 1e9 / PEAK_HBM_GBPS}
    del qw3_sets
    pk3_sets = [fp8.fp8_pack_weights_decode(qw3) for _ in range(3)]
    del qw3

    def dec_packed(i):
        fp8.fp8_block_gemm_packed(qa3, sa3, "group_1x128", pk3_sets[i % 3], sw3, "block_128x128", out=o3)

    t_decp = timer.run(dec_packed, 50, warmup=5, name="decode_gemm_packed_16x28672x8192")
    res["decode_gemm_packed_16x28672x8192"] = {"us": t_decp * 1e6, "GB/s": dec_bytes / t_decp / 1e9,
                                               "frac_hbm": dec_bytes / t_decp / 1e9 / PEAK_HBM_GBPS,
                                               "TFLOP/s": 2.0 * m3 * n3 * k3 / t_decp / 1e12}

    def step_two_packed(i):
        qa_call(i)
        dec_packed(i)

    def step_fused_packed(i):
        fp8.fp8_quantize_gemm_decode(a3, pk3_sets[i % 3], sw3, "block_128x128", gran_a="group_1x128", out=o3)

    for key, fn in (("decode_step_quantize_then_gemm_packed_16x28672x8192", step_two_packed),
                    ("decode_step_fused_packed_16x28672x8192", step_fused_packed)):
        t = timer.run(fn, 50, warmup=5, name=key)
        res[key] = {"us": t * 1e6, "GB/s": fused_bytes / t / 1e9, "frac_hbm": fused_bytes / t / 1e9 / PEAK_HBM_GBPS}

    def pack(i):
        fp8.fp8_pack_weights_decode(pk3_sets[i % 3].view(n3, k3), out=pk3_sets[(i + 1) % 3])

    t_pack = timer.run(pack, 10, warmup=2, name="pack_weights_decode_28672x8192")
    res["pack_weights_decode_28672x8192_offline"] = {"us": t_pack * 1e6, "GB/s": 2.0 * n3 * k3 / t_pack / 1e9,
                                                     "frac_hbm": 2.0 * n3 * k3 / t_pack / 1e9 / PEAK_HBM_GBPS}
    del pk3_sets
    return res


def copy_calibration(torch, timer, dev):
    """A plain device-to-device copy of 512 MB (torch copy_), the reference
    kernel for scaling the HBM byte counters, and the achievable-bandwidth
    context for the HBM-bound passes."""
    n = 256 * 1024 * 1024
    x = torch.ones(n, device=dev, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    t = timer.run(lambda i: y.copy_(x), 20, warmup=3, name="copy_512MB")
    print(json.dumps({"copy_512MB": {"us": t * 1e6, "GB/s": 2 * 2 * n / t / 1e9,
                                     "bytes_read": 2 * n, "bytes_written": 2 * n},
                      "per_call": timer.stats}), flush=True)


def mfma_ceiling(torch, dev, qa, qw):
    """Throughput of the GEMM's FP8 MFMA with no memory traffic, on 2 KB of
    the workload's own activation and weight codes, alone and with the 4
    independent fp32 FMAs per MFMA that the per-K-block promotion issues, and
    (for contrast) on all-zero operands. 2 waves per SIMD, as the GEMM. The
    chip's clock under MFMA load is power-limited and power depends on the
    operand bits, so this, not the nominal peak, is what the GEMM can reach."""
    import ctypes
    path = os.path.join(ROOT, "fp8_quantization_block_amd", "libfp8blk_bench.so")
    if not os.path.exists(path):
        print("bench.py: libfp8blk_bench.so not built; skipping the MFMA ceiling", file=sys.stderr)
        return None
    lib = ctypes.CDLL(path)
    f = lib.fp8blk_bench_mfma_ceiling
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    a_codes = qa.reshape(-1)[:2048].contiguous().view(torch.int32)
    b_codes = qw.reshape(-1)[:2048].contiguous().view(torch.int32)
    zeros = torch.zeros(512, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    flops = blocks * 4 * iters * 8 * 16 * 16 * 128 * 2.0
    res = {}
    for name, a, b, fmas in (("mfma_only", a_codes, b_codes, 0), ("mfma_plus_4_fma", a_codes, b_codes, 4),
                             ("mfma_only_zero_operands", zeros, zeros, 0)):
        best = None
        for rep in range(4):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = f(a.data_ptr(), b.data_ptr(), out.data_ptr(), fmas, blocks, iters, stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"fp8blk_bench_mfma_ceiling returned {rc}")
            t = e0.elapsed_time(e1) * 1e-3
            if rep > 0:
                best = t if best is None else min(best, t)
        res[name] = flops / best / 1e12
    res["unit"] = "TFLOP/s"
    res["operands"] = "first 2 KB of the quantized activations and weights"
    return res


def cpu_baseline(syn, qw, sw, M, N, K):
    """The oracle timed on the whole step at full size: 1x128 quantization of
    the [8192, 8192] activations, then the oracle GEMM 8192 x 10240 x 8192
    (dequantize to fp64 and one fp64 matmul, plus the tolerance base), as the
    oracle stands (its matmuls use NumPy's BLAS thread pool). The weight codes
    and scales are the offline pass's, as in the GPU step."""
    import threadpoolctl
    from oracle import quant, gemm

    a = syn.activations(4).float().numpy()
    t0 = time.perf_counter()
    qa, sa = quant.quantize_group_1x128(a)
    gemm.block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128")
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    return {
        "value": 2.0 * M * N * K / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole step: act quantize {M}x{K} (1x128) + oracle GEMM {M}x{N}x{K} "
                  f"(fp64 dequant-matmul, y and T); {dt:.2f} s; host os.cpu_count()={os.cpu_count()}",
    }


if __name__ == "__main__":
    main()
