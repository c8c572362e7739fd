"""MI355X (gfx950) exact tiled attention: forward with online softmax and a backward
that recomputes the probabilities from the stored logsumexp.

The compute path is the C-ABI library ``libfa.so`` (hand-written HIP kernels); the
Python layer in :mod:`exact_io_aware_fa2_amd.fa` only marshals arguments to it.
"""

__all__ = ["fa", "workloads"]
