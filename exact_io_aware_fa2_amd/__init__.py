"""MI355X (gfx950) exact tiled attention: forward with online softmax and a backward
that recomputes the probabilities from the stored logsumexp.

The compute path is the C-ABI library ``libfa.so`` (hand-written HIP kernels); the
Python layer in :mod:`exact_io_aware_fa2_amd.fa` only marshals arguments to it:
``forward`` / ``backward`` (bf16, optional ALiBi slopes; fp32 forward),
``forward_varlen`` / ``backward_varlen`` (packed sequences), ``forward_fp8`` (E4M3 inputs)
and ``decode`` (the newest queries over a KV cache, split over the keys).
:mod:`exact_io_aware_fa2_amd.workloads` draws the seeded synthetic inputs.
"""

__all__ = ["fa", "workloads"]
