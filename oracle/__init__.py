"""CPU oracle for exact scaled dot-product attention (fp64 NumPy).

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the GPU kernels are checked against.  It may be imported by
``tests/``, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``, and by nothing else.  The product path (the HIP library and its
Python binding) never imports, calls or links it, and the oracle never
imports the product path: the two share no code.

Source pages (cited by site, title and section):

* claspmoon.cn, "14 · 缩放定律与高效注意力" (Scaling laws and efficient
  attention) -- §3.2 Tiling, §3.3 backward recomputation, §3.5 usage,
  §5.1 (ring attention: sequence parallelism), §6 experiment 1.
* book.anysome.cn, "高效注意力" (Efficient attention) -- §2 FlashAttention,
  §3 MQA/GQA, §4 sliding window.
* mdooai.com, "Ch.04 注意力优化：FlashAttention 与稀疏注意力" (Attention
  optimisation) -- "核心公式" (core formula) and "公式速览" (formula overview).
* transformer.xph.ink, "高效注意力：FlashAttention 与线性注意力" -- "原理与机制"
  (principle and mechanism: online softmax).
* kler.cn, "大模型高效注意力机制全解析：FlashAttention 与稀疏注意力实战" --
  §3.1.1 (safe softmax), §3.2.1 (GQA and sliding-window configuration keys).

Pins (``tests/test_oracle.py``): row-stochasticity, exact zero weight on
masked keys, convexity, closed forms (L=1, Q=0, identical keys, a two-key
worked example), shift and permutation invariance, GQA == repeated-head MHA,
window >= L == causal, agreement with PyTorch's float64 CPU
``scaled_dot_product_attention`` and with ``scipy.special.logsumexp``,
torch float64 autograd and central finite differences for the backward,
the exact identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, and the
tiled online-softmax recurrence agreeing with the direct definition; for the
chunked (ring-attention) functions: a chunk covering the whole sequence equals
the full definition, merged partials over any partition of the keys equal the
full result, summed chunk gradients equal the full gradient, brute-force
loops on tiny chunks, and the merge against ``numpy.logaddexp``; for decode:
a cache holding exactly the new tokens equals the full causal forward, each
new token equals the matching row of the whole-sequence forward (with and
without a window), per-sequence cache lengths, and a single-token rolling
window buffer in any slot order equals the windowed row; for the rolling
buffer with several new tokens: the buffer filled token by token (slot p mod
W), read back, equals the matching rows of the whole-sequence causal windowed
forward, before and after the buffer wraps; for general masks:
the family reduces to the causal/window mask, brute-force loops over
symmetric windows, global tokens and block masks, the masked forward and
backward reduce to the plain ones, global rows equal unmasked rows,
finite differences on a sparse pattern, and the row-sampled forward and dQ
equal the matching rows of the whole-sequence functions.  Every oracle
function has at least one pin; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    allowed_mask,
    position_mask,
    block_forward,
    block_backward,
    merge_partials,
    decode_forward,
    rolling_decode_forward,
    general_mask,
    forward_with_mask,
    backward_with_mask,
    forward_rows_with_mask,
    dq_rows_with_mask,
    kv_head_of,
    probabilities,
    forward,
    forward_rows,
    backward,
    tiled_online_forward,
)
