"""Float64 reference for the 8-bit floating-point forward (test infrastructure only).

The pages say only that a later version of the method adds an FP8 forward pass
(ainews.cool, "flash-attention transformer optimization", opening overview: FP8 tensor
cores; hysenlabs.com, "dao-ailab flash-attention", hardware-boundary section: the
FP16/BF16 forward and backward plus an FP8 forward).  They fix neither the format nor a
scaling scheme.  The reading taken here, the plainest one:

* Q, K and V arrive as 8-bit codes in the OCP FP8 E4M3 format (the "fn" variant that the
  gfx950 matrix cores read): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 holds subnormals m/8 * 2^-6; the two codes with every exponent and
  mantissa bit set (0x7F, 0xFF) are NaN; there are no infinities.  Largest finite value
  448, smallest positive 2^-9.
* Each tensor carries one positive float32 dequantisation factor: the real input is
  factor * decoded code.
* What is computed is the exact attention of the dequantised inputs, the same definition
  as ``attention.attn_fwd``.  How a kernel rounds on the way (the fp8 products, the
  probabilities it feeds to the second product) is its own affair; the tests bound it.

All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

from .attention import attn_fwd


def e4m3_decode(codes) -> np.ndarray:
    """Float64 value of every E4M3 code (uint8 array of any shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def dequantize(codes, factor: float) -> np.ndarray:
    """factor * value of each code, float64."""
    return e4m3_decode(codes) * float(factor)


def attn_fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal=False, window=0,
                 scale=None, **kw):
    """O [B, N, Hq, d] and LSE [B, Hq, N] of attention over the dequantised inputs.

    q8 [B, N, Hq, d], k8 / v8 [B, N, Hkv, d]: E4M3 codes (uint8); descale_*: the
    per-tensor factors.  ``kw`` passes through to ``attention.attn_fwd``.
    """
    return attn_fwd(dequantize(q8, descale_q), dequantize(k8, descale_k),
                    dequantize(v8, descale_v), causal, window, scale, **kw)

