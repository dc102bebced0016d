"""CPU oracle for exact scaled-dot-product attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. The GPU library never calls it and shares no
code with it; if the HIP library is missing the product path fails instead of
falling back here.

What it computes is the plain definition of attention (FlashAttention guide,
cxbdf.cn, part 1: Attention(Q, K, V) = softmax(QKᵀ/√d_k)·V, softmax per row),
with the N×N score matrix materialised in float64. The fused method reaches
this same result up to summation order (the pages call it exact, not an
approximation: Flash Attention 是什麼, adersaytech.com, section "exact, 不是
近似"), so the definition itself is the oracle.

Modules:
  attention   NumPy float64 forward and backward, whole tensors or sampled rows
              (the backward also at selected query rows and key columns)
  decode      NumPy float64 attention of new queries over a key/value cache,
              and its backward for queries and keys of different lengths
  bruteforce  pure-Python loops (math.exp / math.fsum) for tiny shapes
  dropout     Philox4x32-10 keep decisions and attention with dropout on the
              softmax weights (forward and backward)
  fp8         e4m3fn decoding and rounding, attention on decoded FP8 inputs,
              the element-wise error bound of a forward that rounds P to e4m3,
              and plain FP8 attention (the accuracy baseline)

Pins: every function here is checked in tests/test_oracle_*.py against hand-
derived worked values (tests/golden/), closed forms, invariants, finite
differences and torch's CPU float64 SDPA. No function is "parity unpinned".
"""
from .attention import (attention_fwd, attention_bwd, attention_probs,
                        attention_fwd_rows, attention_bwd_sampled, attention_bwd_rows)
from .decode import kvcache_fwd, kvcache_fwd_units, kvlen_bwd, kvlen_head_bwd
from . import bruteforce
from .dropout import (attention_bwd_dropout, attention_fwd_dropout, head_bwd_dropout,
                      head_fwd_dropout, keep_mask, keep_threshold, philox4x32_10)
from .fp8 import (attention_fwd_fp8, attention_fwd_fp8_plain, e4m3fn_decode, e4m3fn_round,
                  dequantize, head_o_bound, o_bound)

__all__ = ["attention_fwd", "attention_bwd", "attention_probs", "attention_fwd_rows",
           "attention_bwd_sampled", "attention_bwd_rows", "kvcache_fwd", "kvcache_fwd_units", "kvlen_bwd", "kvlen_head_bwd", "bruteforce",
           "attention_fwd_fp8", "attention_fwd_fp8_plain", "e4m3fn_decode", "e4m3fn_round",
           "dequantize", "head_o_bound", "o_bound",
           "attention_fwd_dropout", "attention_bwd_dropout", "head_fwd_dropout",
           "head_bwd_dropout", "keep_mask", "keep_threshold",
           "philox4x32_10"]
