"""CPU oracle for fused softmax attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct reference that the HIP
path is checked against. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product library never does,
and the oracle never imports the product library (they share no code).

Sources (cited by page title and section; no line numbers):
  [L17]  "第17讲 Tensor Core、HBM、SRAM 与 FlashAttention" (zwxr.cn news 250415),
         §2.1 (the matrix product), §5.3 (its work count),
         §8.1 (scaled dot-product attention), §8.3 (online softmax state
         m, l, o and its update rule; masks and causal attention named as
         part of a real kernel), §8.4 (exact, not bitwise identical),
         §9.2 (prefill and decode).
  [N5]   "GPU 架构与大模型高效计算" -- CS336 Lecture 5 notes (kyc001.github.io),
         §7.1-§7.2 (tiling, online softmax, recomputation in the backward pass).
  [R5]   "CS336 Lecture 5 · GPUs, TPUs -- 中文 Lecture Note" (romanrose.github.io),
         section "FlashAttention 解析" (running max/sum correction) and the
         English transcript at [01:14:15]-[01:16:33] (softmax of a tile,
         partial results written back to global memory, then continued).

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, invariants, library special cases, brute force and finite
differences). No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    online_softmax_forward,
    brute_force_forward,
    brute_force_backward,
    causal_visible,
    merge_partials,
)
from .matmul import brute_force_matmul_nt, matmul_nt  # noqa: F401
from .fp8 import (  # noqa: F401
    attention_forward_mxfp8,
    e4m3_decode,
    e4m3_encode,
    mx_dequantize,
    mx_quantize,
    mx_scale_code,
    p_rounding_bound,
)
