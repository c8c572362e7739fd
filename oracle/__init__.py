"""Float64 CPU oracle for exact scaled-dot-product attention (test infrastructure).

This package is test infrastructure, not part of the product path. Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it. It shares no code with the HIP kernels, the C ABI or
the Python binding, and it never touches a GPU.

Every function is the plain textbook definition written out in NumPy float64:
full-row softmax over the allowed key set, no tiling over keys and no online
rescaling.  Sources (the pages this oracle follows):

* ainews.cool, "flash-attention transformer optimization", section 技术深度解析
  (technical deep dive): the attention formula Softmax(QK^T/sqrt(d))V, the N x N
  intermediate, and recomputation of that matrix in the backward pass.
* bmjup.com, "FlashAttention-2: 下一代高效注意力机制的突破与实战解析", section 2
  (v1 vs v2, causal/window masks) and section 3.3 (sliding-window attention:
  entries outside the window get probability zero); section 4 (the
  (batch, seqlen, nheads, headdim) layout of the usage example).
* unite.ai, "What is FlashAttention", intro and worked-example section: the
  method computes exact attention, so the plain definition is the target.
* hysenlabs.com, "dao-ailab flash-attention", hardware-boundary section: MQA/GQA
  (KV heads shared by groups of query heads).

``oracle.fp8`` adds the 8-bit floating-point forward: the same definition on inputs
decoded from E4M3 codes and multiplied by per-tensor factors.

The backward pass is the analytic derivative of the forward (the pages only say
the matrix is recomputed); it is written as the softmax Jacobian-vector product.
"""

from .attention import (  # noqa: F401
    allowed_keys,
    attention_probs,
    attention_probs_rows,
    attn_fwd_head,
    attn_bwd_head,
    attn_fwd,
    attn_bwd,
    attn_fwd_rows,
    attn_bwd_dq_rows,
    attn_bwd_dkdv_cols,
    attn_bwd_dkdv_cols_from_fwd,
    attended_pairs,
    attn_fwd_varlen,
    attn_bwd_varlen,
    attn_decode,
)
from .fp8 import attn_fwd_fp8, dequantize, e4m3_decode  # noqa: F401
