"""Build libfp8blk.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m fp8_quantization_block_amd.build [--verbose]
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8blk.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "attention.hip"]
# measurement-only kernels, loaded by bench.py alone (kept out of the product library)
BENCH_LIB = os.path.join(PKG, "libfp8blk_bench.so")
BENCH_SOURCES = ["bench_ceiling.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the GEMM promotes every partial product with VALU
    # FMAs, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile the product library (every HIP source of the path) and the
    measurement-only library; returns the product library's path."""
    _compile(BENCH_SOURCES, BENCH_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)


def _compile(sources, lib, verbose):
    """Each source to an object in parallel (each carries its own gfx950 code
    object), then one link into the shared library."""
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [lib + "." + os.path.splitext(s)[0] + ".o" for s in sources]
    cmds = [[HIPCC] + compile_flags + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
