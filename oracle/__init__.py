"""CPU oracle for single-token FP16 grouped-query-attention decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call,
link or execute anything in this package: only the tests, the smoke check
and the benchmark's CPU-baseline leg use it. It shares no code with the HIP
path (no kernels, headers, helpers, tables or pre/post-processing).

What it computes is the plain definition of the decode fixed by the
FlashInfer PR #5052 analysis page ("SM110 FP16 GQA decode"): the
``sm110_gqa_decode`` docstring in section 1 (shapes, and q_scale as an extra
factor on the scores beside 1/sqrt(128)), the 32/8/128 specialisation with 4:1 grouping in
section 2, and the benchmark's PyTorch SDPA comparator in section 3
(boolean length mask, scale 1/sqrt(128), ``enable_gqa=True``).

Modules:
  reference -- numpy float64 definition, one (batch, kv head) at a time.
  formats   -- exact widening of bfloat16 and float64 -> bfloat16 rounding.
  brute     -- scalar pure-Python loops (math.fsum) and an mpmath variant,
               used only to pin ``reference`` on tiny inputs.
"""
from .formats import bf16_to_f64, round_bf16  # noqa: F401
from .reference import (  # noqa: F401
    GROUP, HEAD_DIM, NUM_KV_HEADS, NUM_Q_HEADS,
    decode, decode_head, decode_ragged, effective_scale, round_fp16,
)
