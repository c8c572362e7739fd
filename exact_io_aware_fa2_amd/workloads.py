"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

This module only draws random tensors and names the workload shapes.  It is the one
module that both the HIP path's tests/bench and the float64 oracle's callers share;
it holds none of the method's arithmetic.

Draw recipe (fixed order q, k, v, dO): ``torch.randn(shape, float32) * sigma`` from a
CPU ``torch.Generator`` seeded with ``seed``, then a round-to-nearest-even cast to the
compute dtype.  Tensors are [batch, seqlen, heads, headdim] (the layout of the usage
example on bmjup.com "FlashAttention-2 ... 实战解析", section 4).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    window: int = 0
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    sigma_do: float = 1.0
    backward: bool = True
    seed: int = 1000
    alibi: bool = False  # position bias with alibi_slopes(Hq)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32 (the value handed to the kernels)."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    def replace(self, **kw) -> "Workload":
        from dataclasses import replace
        return replace(self, **kw)


# The five configurations the method is measured on (the fifth runs twice: causal, and
# causal with a 4096-key sliding window on the same tensors).
WORKLOADS = {
    "fp32_b1_h2_n256_d64": Workload("fp32_b1_h2_n256_d64", "fp32", 1, 2, 2, 256, 64, False,
                                    backward=False, seed=1001),
    "bf16_b2_h16_n2048_d128_causal_sigma4": Workload(
        "bf16_b2_h16_n2048_d128_causal_sigma4", "bf16", 2, 16, 16, 2048, 128, True,
        sigma_q=4.0, sigma_k=4.0, seed=1002),
    "bf16_b2_h32_n8192_d128_causal": Workload("bf16_b2_h32_n8192_d128_causal", "bf16",
                                              2, 32, 32, 8192, 128, True, seed=1003),
    "bf16_b1_h16_n16384_d256": Workload("bf16_b1_h16_n16384_d256", "bf16", 1, 16, 16, 16384,
                                        256, False, seed=1004),
    "bf16_b1_hq32_hkv8_n65536_d128_causal": Workload(
        "bf16_b1_hq32_hkv8_n65536_d128_causal", "bf16", 1, 32, 8, 65536, 128, True, seed=1005),
    "bf16_b1_hq32_hkv8_n65536_d128_causal_window4096": Workload(
        "bf16_b1_hq32_hkv8_n65536_d128_causal_window4096", "bf16", 1, 32, 8, 65536, 128, True,
        window=4096, seed=1005),
}

DEFAULT_WORKLOAD = "bf16_b2_h32_n8192_d128_causal"

def alibi_slopes(h: int) -> list:
    """The geometric slope set of the ALiBi method: head i (1-based) of h gets 2^(-8 i / h)."""
    return [2.0 ** (-8.0 * i / h) for i in range(1, h + 1)]


# bf16_b2_h32_n8192_d128_causal with the ALiBi position bias (the geometric slopes above).
ALIBI_WORKLOADS = {
    "bf16_b2_h32_n8192_d128_causal_alibi": Workload(
        "bf16_b2_h32_n8192_d128_causal_alibi", "bf16", 2, 32, 32, 8192, 128, True, seed=1007,
        alibi=True),
}

# The shape of bf16_b2_h32_n8192_d128_causal with 8-bit E4M3 inputs (forward only).
FP8_WORKLOADS = {
    "fp8_b2_h32_n8192_d128_causal": Workload("fp8_b2_h32_n8192_d128_causal", "fp8", 2, 32, 32,
                                             8192, 128, True, backward=False, seed=1006),
}

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}

E4M3_MAX = 448.0


def torch_dtype(w: Workload) -> torch.dtype:
    return _TORCH_DTYPE[w.dtype]


def make_inputs(w: Workload, device: str | torch.device = "cpu", with_grad: bool | None = None):
    """Draw (q, k, v, dO) for workload ``w``; dO is None for forward-only workloads.

    The draw happens on the CPU in float32 so the values do not depend on the device;
    the rounded tensors are then moved to ``device``.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    dt = torch_dtype(w)
    shp_q = (w.B, w.N, w.Hq, w.d)
    shp_kv = (w.B, w.N, w.Hkv, w.d)

    def draw(shape, sigma):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt).to(device)

    q = draw(shp_q, w.sigma_q)
    k = draw(shp_kv, w.sigma_k)
    v = draw(shp_kv, w.sigma_v)
    want_grad = w.backward if with_grad is None else with_grad
    do = draw(shp_q, w.sigma_do) if want_grad else None
    return q, k, v, do


def small_case(name: str, dtype: str, B: int, Hq: int, Hkv: int, N: int, d: int, causal: bool,
               window: int = 0, seed: int = 7, sigma_qk: float = 1.0) -> Workload:
    """A parity-test workload of arbitrary (small) shape."""
    return Workload(name, dtype, B, Hq, Hkv, N, d, causal, window, sigma_qk, sigma_qk,
                    seed=seed)


# ------------------------------------------------------------------ packed sequences
@dataclass(frozen=True)
class VarlenWorkload:
    """Sequences of different lengths packed back to back (no padding), bf16.

    Tensors are [total, heads, headdim]; sequence s owns rows cu[s] .. cu[s+1]-1.
    """
    name: str
    lengths: tuple
    Hq: int
    Hkv: int
    d: int
    causal: bool
    window: int = 0
    seed: int = 2000
    dtype: str = "bf16"

    @property
    def total(self) -> int:
        return int(sum(self.lengths))

    @property
    def max_seqlen(self) -> int:
        return max(1, int(max(self.lengths)))

    @property
    def cu_seqlens(self) -> list:
        out = [0]
        for n in self.lengths:
            out.append(out[-1] + int(n))
        return out

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())


def length_mix(total: int, lo: int, hi: int, seed: int) -> tuple:
    """Sequence lengths drawn log-uniformly in [lo, hi] until they fill ``total`` rows
    (the last one is cut to fit): a mix of short and long documents."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out, left = [], total
    while left > 0:
        u = torch.rand((), generator=g, dtype=torch.float64).item()
        n = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
        n = max(1, min(n, left))
        out.append(n)
        left -= n
    return tuple(out)


# A packed batch with the token count of bf16_b2_h32_n8192_d128_causal (2 x 8192 rows of
# 32 heads, d=128, causal), made of documents of 128 .. 8192 rows.
VARLEN_WORKLOADS = {
    "bf16_varlen_t16384_h32_d128_causal": VarlenWorkload(
        "bf16_varlen_t16384_h32_d128_causal", length_mix(16384, 128, 8192, 2001), 32, 32, 128,
        True, seed=2001),
}


def make_varlen_inputs(w: VarlenWorkload, device: str | torch.device = "cpu"):
    """Draw packed (q, k, v, dO) in the order and manner of ``make_inputs``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)

    def draw(h):
        return torch.randn((w.total, h, w.d), generator=g, dtype=torch.float32).to(
            torch.bfloat16).to(device)

    q = draw(w.Hq)
    k = draw(w.Hkv)
    v = draw(w.Hkv)
    do = draw(w.Hq)
    return q, k, v, do


# ------------------------------------------------------------------ 8-bit inputs
def quantize_e4m3(x: torch.Tensor):
    """Per-tensor scaling into the E4M3 range: factor = amax / 448 in float32, codes = the
    round-to-nearest-even E4M3 cast of x / factor (torch's float8_e4m3fn conversion).
    Returns (codes as a uint8 tensor, factor); factor * decoded code approximates x."""
    amax = float(x.abs().max())
    factor = float(torch.tensor(amax / E4M3_MAX if amax > 0 else 1.0, dtype=torch.float32))
    y = (x.float() / factor).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), factor


def make_fp8_inputs(w: Workload, device: str | torch.device = "cpu"):
    """(q8, k8, v8, (fq, fk, fv)) for a forward-only workload: float32 draws in the order
    and manner of make_inputs (before any rounding), each quantized per tensor."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    out, factors = [], []
    for shape, sigma in (((w.B, w.N, w.Hq, w.d), w.sigma_q), ((w.B, w.N, w.Hkv, w.d), w.sigma_k),
                         ((w.B, w.N, w.Hkv, w.d), w.sigma_v)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        c, f = quantize_e4m3(x)
        out.append(c.to(device))
        factors.append(f)
    return out[0], out[1], out[2], tuple(factors)


# ------------------------------------------------------------------ decoding over a cache
@dataclass(frozen=True)
class DecodeWorkload:
    """Nq new tokens per sequence over a bf16 KV cache of Nk rows (lengths: the cached
    length of each sequence, None for Nk everywhere)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool = True
    window: int = 0
    lengths: tuple | None = None
    seed: int = 3000
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def lens(self) -> list:
        return [self.Nk] * self.B if self.lengths is None else [int(n) for n in self.lengths]


# One decoding step of 8 sequences with 32768 cached tokens each, grouped-query heads as in
# the 65536-token workload (32 query heads over 8 KV heads), d = 128.
DECODE_WORKLOADS = {
    "bf16_decode_b8_hq32_hkv8_nq1_nk32768_d128": DecodeWorkload(
        "bf16_decode_b8_hq32_hkv8_nq1_nk32768_d128", 8, 32, 8, 1, 32768, 128, seed=3001),
}


def make_decode_inputs(w: DecodeWorkload, device: str | torch.device = "cpu"):
    """(q [B, Nq, Hq, d], k_cache, v_cache [B, Nk, Hkv, d], seqlens int32 [B] or None),
    drawn in the manner of make_inputs (order q, k, v)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)

    def draw(shape):
        return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(device)

    q = draw((w.B, w.Nq, w.Hq, w.d))
    k = draw((w.B, w.Nk, w.Hkv, w.d))
    v = draw((w.B, w.Nk, w.Hkv, w.d))
    lens = None if w.lengths is None else torch.tensor(w.lens, dtype=torch.int32).to(device)
    return q, k, v, lens


# ------------------------------------------------------------------ tensors near the size limit
# The entry points accept tensors of fewer than 2^31 elements (the kernels' row and buffer
# arithmetic is 32-bit); the largest such tensors are drawn on the device itself, where a
# host draw and copy of several GiB would dominate a test.
MAX_ELEMS = 1 << 31


def device_normal(shape, seed: int, device, dtype=torch.bfloat16):
    """Seeded N(0, 1) draws made on `device` by torch's generator for that device, in dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=dtype)
