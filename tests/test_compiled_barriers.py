"""Every workgroup barrier in the compiled kernels waits for the wave's own
LDS accesses first.

On gfx950 `s_barrier` only synchronizes instruction streams: a wave can reach
it with its own LDS reads and writes still in flight (counted by lgkmcnt).
Data a wave writes to LDS before a barrier is then not guaranteed to be there
when another wave reads it after the barrier, and a read made before the
barrier may still be pending when another wave overwrites the data. The
kernels therefore reach every barrier through a helper that waits
lgkmcnt(0) right before it (`raw_barrier`, `copies_done_barrier` in
device_common.h, or `__syncthreads`). The compiler does not add that wait by
itself: a merge through LDS in the decode-attention kernel once had ten LDS
writes outstanding at its barrier.

This test compiles the kernel sources for gfx950 with the library's flags and
checks, for every `s_barrier` in the assembly, that walking back from it an
`s_waitcnt` with lgkmcnt(0) comes before any LDS memory access, any direct
global-to-LDS copy, and any branch or block label. Lane shuffles through the
LDS hardware (`ds_bpermute`, `ds_permute`, `ds_swizzle`) touch no LDS memory
and may sit in between. Host-only check: no GPU is used.
"""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp8_quantization_block_amd import build as fp8build

HIPCC = fp8build.HIPCC
pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")

# LDS memory accesses and direct copies into LDS (not lane shuffles)
_LDS_MEM = re.compile(r"^(ds_(read|write|load|store|add|sub|rsub|max|min|and|or|xor|inc|dec|cmpst|cmpswap|"
                      r"wrxchg|append|consume|gws|condxchg)\w*"
                      r"|buffer_load\w*\s.*\blds\b|global_load_lds\w*)")
_LABEL = re.compile(r"^[.A-Za-z_][\w.$]*:")
_FUNC = re.compile(r"^([A-Za-z_][\w.$]*):")


def _assembly(src: str) -> str:
    flags = [f for f in fp8build.FLAGS if f not in ("-shared", "-fPIC", "-Wall", "-Wno-unused-function")]
    cmd = [HIPCC] + flags + ["-S", "--offload-device-only", os.path.join(fp8build.CSRC, src), "-o", "-"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


def unguarded_barriers(asm: str):
    """(function, line number, preceding lines) of every s_barrier not
    preceded, within its block, by an s_waitcnt with lgkmcnt(0) before any
    LDS memory access or direct copy into LDS."""
    lines = [l.strip() for l in asm.splitlines()]
    bad = []
    fn = None
    for i, l in enumerate(lines):
        m = _FUNC.match(l)
        if m:
            fn = m.group(1)
        if not l.startswith("s_barrier"):
            continue
        guarded = False
        for j in range(i - 1, -1, -1):
            t = lines[j]
            if not t or t.startswith(";"):
                continue
            if _LABEL.match(t) or t.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                break
            if t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
                guarded = True
                break
            if _LDS_MEM.match(t):
                break
        if not guarded:
            bad.append((fn, i + 1, lines[max(0, i - 4):i + 1]))
    return bad


def test_checker_flags_an_unguarded_barrier():
    """The checker itself: a barrier after an LDS write with no wait is
    flagged; with the wait, or with only a lane shuffle after the wait, it is
    not."""
    bad = "k:\n\tds_write_b64 v1, v[2:3]\n\ts_barrier\n"
    good = "k:\n\tds_write_b64 v1, v[2:3]\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n"
    shuffle = "k:\n\ts_waitcnt vmcnt(0) lgkmcnt(0)\n\tds_bpermute_b32 v1, v2, v3\n\ts_barrier\n"
    block_start = "k:\n\ts_waitcnt lgkmcnt(0)\n.LBB0_1:\n\ts_barrier\n"
    assert len(unguarded_barriers(bad)) == 1
    assert unguarded_barriers(good) == []
    assert unguarded_barriers(shuffle) == []
    assert len(unguarded_barriers(block_start)) == 1


def test_every_barrier_waits_for_lds():
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        asms = dict(zip(fp8build.SOURCES, ex.map(_assembly, fp8build.SOURCES)))
    total = 0
    problems = []
    for src, asm in asms.items():
        total += sum(1 for l in asm.splitlines() if l.strip().startswith("s_barrier"))
        problems += [(src,) + b for b in unguarded_barriers(asm)]
    assert total > 0, "no s_barrier found: the assembly was not parsed"
    assert not problems, (f"{len(problems)} of {total} barriers reached without waiting for LDS accesses; "
                          f"first: {problems[0]}")
