"""fp64 CPU oracle for one tensor-parallel rank's shard computation.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The HIP library never routes through it, and it shares no code with the HIP path:
the only module both sides read is ``workloads`` (seeded draws, no arithmetic of
the method).

Every function is the plain definition of what a rank computes, in float64 NumPy
(pure-Python loops live in ``oracle.brute`` for tiny inputs). Sources, by page:

* "CUDA tensor parallel computations" (learning notes): the worked example in
  "最小数学地基", column split ("第二类 Column Parallel"), row split ("第三类 Row
  Parallel"), the merges ("第四类 跨卡通信计算"), local element-wise work ("第五类
  局部逐元素计算") and how these compose in a block ("放进 Transformer").
* "张量并行：切分 Transformer 层的分布式训练": column/row sharding of Z = XW
  ("张量并行的核心思想"), the MLP and self-attention splits ("Transformer 层的张量并行
  切分"), the vocabulary-split output layer ("输入与输出层").
* "TensorRT LLM 中的并行策略", "注意力模块": heads split evenly; KV shared by
  grouped query heads.
* ``fp8_ref``: the same layers on OCP E4M3 operands with per-tensor scales (the pages
  name no number format; the format's own definition is restated there).

Parity status per function (pins live in ``tests/test_oracle_pins.py``):
all functions are pinned (the E4M3 table and rounding against torch's float8_e4m3fn
conversion and a bit-by-bit construction; the fp8 layers against pure-Python loops)
except two conventions the pages never state: the rotary-embedding *convention*
(rotate-half pairs (i, i+d/2), frequency theta^(-2i/d)) and the RMSNorm *formula* (the
pages name RMSNorm but not its formula; the usual x / sqrt(mean(x^2) + eps) * gamma is
used). Their closed-form properties are pinned; the choice of convention is "parity
unpinned".
"""
from .tp_ref import *  # noqa: F401,F403
from .fp8_ref import *  # noqa: F401,F403
from . import tp_ref as _tp, fp8_ref as _f8

__all__ = list(_tp.__all__) + list(_f8.__all__)
