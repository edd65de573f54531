"""CPU oracle for the W8A8 FP8 path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the package
``fp8_quantization_block_amd`` and its HIP library) imports, links or runs
anything in this directory. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may use it.

It is a plain, slow, NumPy implementation written straight from the pages:

* ``e4m3``  -- the OCP E4M3 value table and a table-driven round-to-nearest-even
  encoder that saturates at +-448;
* ``e5m2``  -- the same for OCP E5M2 (largest value 57344, saturating);
* ``quant`` -- the amax / scale / cast quantizer for every group shape the path
  uses (per tensor, 1x128, 128x128, KV head x 128 tokens), the KV dequantizer,
  and static / delayed scaling (a cast under a supplied scale that also records
  the tensor's amax, and the scale taken from an amax history window);
* ``gemm``  -- the block-scaled GEMM as dequantize-to-fp64 followed by a plain
  fp64 matmul, plus the tolerance base |A|.|W|^T;
* ``attention`` -- decode attention over the FP8 KV cache, dequantized to fp64,
  plus the tolerance base sum_t p_t |v_hat_t|;
* ``mx`` -- MX block-32 quantization with power-of-two (E8M0) scales and the
  GEMM over MX operands.

Every function cites the page and section it follows. Pages are cited as

* [FP8]   wangyu.me, "大语言模型量化技术（五）：FP8" (LLM quantization part 5: FP8)
* [MIXED] charles2530.github.io, "量化：FP8 与混合精度推理：它不是一个 dtype 开关"
* [LONG]  pwwt.cn, Llama-3 FP8 and long-context practice notes
* [VS]    api.makesence.top, "LLM推理量化:FP8 versus INT8"

Parity status: every function here is pinned by tests under ``tests/``
(``test_oracle_*.py``) against values the pages print, closed forms,
invariants and brute force; none is "parity unpinned".
"""

from . import e4m3, e5m2, quant, gemm, attention, mx  # noqa: F401
