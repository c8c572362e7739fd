"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI, run the
float64 oracle on the very same (rounded) inputs, and compare against the tolerances.

Tolerances (bf16 inputs, float32 accumulation):
  O    : max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3
  LSE  : max |LSE - LSE_ref| <= 1e-3
  dQ/dK/dV : ||X - X_ref||_F / ||X_ref||_F <= 3e-2 per tensor
float32 inputs: ||O - O_ref||_F / ||O_ref||_F <= 1e-5, |LSE - LSE_ref| <= 1e-5 max(1, |LSE_ref|).
"""

from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from exact_io_aware_fa2_amd import fa

O_MAX, O_MEAN, LSE_MAX, GRAD_REL = 2e-2, 2e-3, 1e-3, 3e-2
FP32_REL = 1e-5


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def check_o(o: np.ndarray, o_ref: np.ndarray, what: str = "O"):
    err = np.abs(o - o_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert err.max() <= O_MAX, f"{what}: max abs err {err.max():.3e} > {O_MAX}"
    assert err.mean() <= O_MEAN, f"{what}: mean abs err {err.mean():.3e} > {O_MEAN}"
    return float(err.max()), float(err.mean())


def check_lse(lse: np.ndarray, lse_ref: np.ndarray, tol: float = LSE_MAX, rel: bool = False):
    err = np.abs(lse - lse_ref)
    if rel:
        err = err / np.maximum(1.0, np.abs(lse_ref))
    assert np.isfinite(lse).all(), "LSE: non-finite output"
    assert err.max() <= tol, f"LSE: max err {err.max():.3e} > {tol}"
    return float(err.max())


def check_grad(x: np.ndarray, ref: np.ndarray, what: str):
    assert np.isfinite(x).all(), f"{what}: non-finite output"
    e = rel_fro(x, ref)
    assert e <= GRAD_REL, f"{what}: relative Frobenius error {e:.3e} > {GRAD_REL}"
    return e


def gpu_fwd(q, k, v, causal, window, scale):
    o, lse = fa.forward(q, k, v, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def gpu_bwd(q, k, v, o, do, lse, causal, window, scale, return_ws=False):
    B, N, Hq, d = q.shape
    ws = fa.workspace_for(B, Hq, k.shape[2], N, d, causal, window, q.device)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, window=window, scale=scale,
                             workspace=ws)
    torch.cuda.synchronize()
    if return_ws:
        return dq, dk, dv, ws
    return dq, dk, dv
