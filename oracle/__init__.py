"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition of what the GPU
library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``exact_attention_31_amd``) never imports, calls or falls back to it, and it
shares no code with the HIP kernels.

Pages cited (by title and section; no line numbers):

* [cicada]  "已有的几种大模型上下文支持情况" — blog on standard attention and
  FlashAttention 1–4 (cicada.microarchitecture.cn/archives/2026082201).
* [FA-1拆解] "FlashAttention 完全拆解（一）：IO 感知与分块注意力算法"
  (pinghaoyang.com.cn/aigc/posts/flashattention-part-1/).
* [15-779 L5] "第 5 讲 · 案例：Transformer、注意力与 FlashAttention" — CMU 15-779
  lecture 5 notes (semidirectx.com/notes/courses/cmu15-779/lecture05/).

Every function here is pinned by ``tests/test_oracle.py`` and, for the FP8
quantisation, ``tests/test_oracle_fp8.py`` against closed forms, a 50-digit
brute force, library routines and special cases and invariants; none is
"parity unpinned".
"""

from .ref import (
    scores,
    safe_softmax,
    attention_ref,
    decode_ref,
    decode_gqa_ref,
    decode_paged_ref,
    attention_bwd_ref,
    attention_block_sparse_ref,
    masked_probs,
)
from .compare import bf16_half_ulp, o_excess, check_prefill, check_decode, bwd_allowance, check_bwd
from .fp8 import e4m3_round, quantize_blocks, dequantize_blocks, attention_fp8_ref, prescale_q

__all__ = [
    "scores",
    "safe_softmax",
    "attention_ref",
    "decode_ref",
    "decode_gqa_ref",
    "decode_paged_ref",
    "attention_bwd_ref",
    "attention_block_sparse_ref",
    "masked_probs",
    "bf16_half_ulp",
    "o_excess",
    "check_prefill",
    "check_decode",
    "bwd_allowance",
    "check_bwd",
    "e4m3_round",
    "quantize_blocks",
    "dequantize_blocks",
    "attention_fp8_ref",
    "prescale_q",
]
