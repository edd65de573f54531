"""How the block GEMM sums a 128-deep K block: crafted dot products.

[MIXED] charles2530.github.io, "量化：FP8 与混合精度推理", section "混合精度才是生产形态":
low-precision products do not mean low-precision sums; the FP8 x FP8
products are exact and their sum must be kept in a wider type. Here the
GPU's fp32-mode output for one 128-wide K block with unit scales is the
matrix unit's block sum itself (promotion multiplies it by exactly 1 and adds
it to 0), so each crafted row pair shows how that sum is formed:

* sums whose every partial sum is an exact fp32 number (128 x 448^2; +-448^2
  cancelling in any order) must come back exact;
* one 448^2 term next to 127 terms of 2^-7 (exact sum 200704 + 127/128, which
  needs 25 significant bits) and a cancelling +-448^2 pair next to 2^-18
  terms show whether small terms are lost behind a large one;
* every result must lie within the fp32-accumulation bound
  gpu_helpers.fp32_accumulation_bound(128) * T of the exact sum, T being the
  sum of the terms' magnitudes.

Both kernels are covered: M = 16 runs the decode kernel, M = 80 the prefill
kernel. The oracle's fp64 sums of these products are exact (multiples of
2^-18 below 2^25).
"""

import numpy as np
import pytest
import torch

from gpu_helpers import check_fp32_accumulation, fp32_accumulation_bound
from oracle import e4m3, gemm as ogemm

pytestmark = pytest.mark.gpu
DEV = "cuda"

C448, CM448, C2M3, C2M4, C2M9, C1 = 0x7E, 0xFE, 0x20, 0x18, 0x01, 0x38
assert e4m3.decode(np.array([C448, CM448, C2M3, C2M4, C2M9, C1])).tolist() == [448, -448, 2 ** -3, 2 ** -4,
                                                                               2 ** -9, 1]


def _crafted():
    """(name, a codes [128], w codes [128]) per case."""
    cases = []

    def pair(name, terms):
        a = np.zeros(128, np.uint8)
        w = np.zeros(128, np.uint8)
        for k, (ca, cw) in terms.items():
            a[k], w[k] = ca, cw
        cases.append((name, a, w))

    big, nbig, small7, small18 = (C448, C448), (CM448, C448), (C2M3, C2M4), (C2M9, C2M9)
    pair("128 x 448^2", {k: big for k in range(128)})
    for pos in (0, 64, 127):
        pair(f"448^2 at k={pos} + 127 x 2^-7", {k: (big if k == pos else small7) for k in range(128)})
    pair("+448^2 k=0, -448^2 k=127, 126 x 2^-18",
         {k: (big if k == 0 else nbig if k == 127 else small18) for k in range(128)})
    pair("+448^2 k=0, -448^2 k=1, 126 x 2^-18",
         {k: (big if k == 0 else nbig if k == 1 else small18) for k in range(128)})
    pair("alternating +-448^2", {k: (big if k % 2 == 0 else nbig) for k in range(128)})
    pair("64 x +448^2 then 64 x -448^2", {k: (big if k < 64 else nbig) for k in range(128)})
    pair("-448^2 at k=5 + 127 x 2^-18", {k: (nbig if k == 5 else small18) for k in range(128)})
    rng = np.random.default_rng(4242)
    for r in range(7):
        c = rng.integers(0, 256, size=(2, 128))
        c = np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)
        cases.append((f"random codes {r}", c[0], c[1]))
    return cases


# cases whose every partial sum, in any order, is an exact fp32 number
EXACT_IN_ANY_ORDER = ("128 x 448^2", "alternating +-448^2", "64 x +448^2 then 64 x -448^2")


@pytest.mark.parametrize("M", [16, 80])
def test_block_sums_of_crafted_dot_products(gpu_lib, M):
    cases = _crafted()
    n = len(cases)
    assert n <= 16
    qa = np.zeros((M, 128), np.uint8)
    qw = np.zeros((128, 128), np.uint8)
    for i, (_, a, w) in enumerate(cases):
        qa[i], qw[i] = a, w
    sa = np.ones((M, 1), np.float32)
    sw = np.ones((1, 1), np.float32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    y32 = gpu_lib.fp8_block_gemm(t(qa), t(sa), "group_1x128", t(qw), t(sw), "block_128x128",
                                 out_dtype=torch.float32).cpu().numpy()
    y64, tt = ogemm.block_gemm(qa, sa, "group_1x128", qw, sw, "block_128x128")
    # the whole output (crafted rows against every weight row) within the bound
    worst = check_fp32_accumulation(y32, y64, tt, 128, what=f"M={M}")
    lines = []
    for i, (name, _, _) in enumerate(cases):
        got, exact, mag = float(y32[i, i]), float(y64[i, i]), float(tt[i, i])
        if name in EXACT_IN_ANY_ORDER:
            assert got == exact, f"{name}: gpu {got!r}, exact {exact!r}"
        lines.append(f"  {name:40s} gpu {got!r:>22} exact {exact!r:>22} rne32(exact) {float(np.float32(exact))!r:>14}"
                     f" err/T {abs(got - exact) / mag if mag else 0.0:.2e}")
    print(f"M={M} ({'decode' if M <= 64 else 'prefill'} kernel), bound {fp32_accumulation_bound(128):.2e} T, "
          f"max err/T {worst:.2e}\n" + "\n".join(lines))
