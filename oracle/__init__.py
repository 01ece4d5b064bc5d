"""Float64 CPU oracle for the GPTQ single-layer quantization path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything in this package.  Only the
test-suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg
of ``bench.py`` use it.  It shares no code with the HIP path.

Sources (cited by page and section throughout):

* [derivation] "GPTQ 从零推导：4-bit 权重量化为什么能“量化一列，补偿一列”"
  (hbblog.cn) -- numbered equations (1)-(68), the NumPy-style teaching
  pseudocode of section 10 and the 16-level worked example of section 11.
* [teardown] "GPTQ 完全拆解：二阶信息驱动的权重量化，如何把 175B 模型塞进一张 A100"
  (pinghaoyang.com.cn) -- the toy OBS example, the three GPTQ steps and the
  paper's Algorithm 1.

Parity status: every function is pinned by a test in ``tests/test_oracle_*``
except the conventions the pages leave open (grid-fit details, the Cholesky
retry factor, the code packing layout); those are listed as "parity unpinned"
in ``gptq_ref``'s header.
"""

from .gptq_ref import *  # noqa: F401,F403
