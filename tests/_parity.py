"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI, run the
float64 oracle on the very same (rounded) inputs, and compare against the tolerances.

Tolerances (bf16 inputs, float32 accumulation):
  O    : max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3
  LSE  : max |LSE - LSE_ref| <= 1e-3
  dQ/dK/dV : ||X - X_ref||_F / ||X_ref||_F <= 3e-2 per tensor
float32 inputs: ||O - O_ref||_F / ||O_ref||_F <= 1e-5, |LSE - LSE_ref| <= 1e-5 max(1, |LSE_ref|).
E4M3 inputs (the fp8 forward): two effects, each bounded per query row i.
  * Scores.  The 8-bit matrix-core product sums its 64 code products with less than float32
    precision.  tests/test_gpu_fp8_products.py measures it against exact sums on operand
    sets built to stress it (uniform codes, log-uniform magnitudes, one dominant product per
    output, cancelling pairs; 3 million results over two seed sets): the error scales with
    2^E, E the largest exponent sum e(a_k) + e(b_k) of the 64 pairs (e of a subnormal code
    taken as -6), and reached 17197 * 2^-24 * 2^E = 1.05 * 2^-10 * 2^E; the test holds the
    hardware to 2^-9 * 2^E.  Relative to the largest actual product the error reached
    68864 * 2^-24 where a subnormal operand sat in the pair with the largest exponent sum,
    so the bound is stated with M(x) = max(|x|, 2^-6 f) >= 2^e(x) f for a value x of a
    tensor with factor f.  With a 2x margin and float32 terms, a score is off by at most
      Delta_i = (d/64) 2^-8 |scale| max_j max_c M(q_ic) M(k_jc) + 2^-22 max_j |s_ij|,
    so |LSE_i - LSE_ref_i| <= 1e-3 + Delta_i (1e-3: the float32 exp / sum / log margin).
  * Weights.  The kernel rounds each weight to E4M3 before the second product and
    normalises by the unrounded weight sum.  With w_j = P_ij / max_j P_ij the rounded weight
    is off by at most max(2^-4 w_j, 2^-10) (3 mantissa bits; subnormal spacing 2^-9 below
    2^-6, at any reference at or below the row max), masked keys exactly 0.  Together with
    weights perturbed by factors within e^(+-2 Delta_i):
      |O_ic - O_ref_ic| <= E (1.001 sum_j max(2^-4 P_ij, 2^-10 max_j P_ij) |v_jc|)
                           + (E - 1)(sum_j P_ij |v_jc| + |O_ref_ic|) + 2^-8 |O_ref_ic|
    with E = e^(4 Delta_i) (2^-8: the bf16 rounding of O).
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


def pool_map(fn, tasks):
    """fn over tasks in a pool of workers() spawned processes, one BLAS thread each (fn must
    be a module-level function); results in task order."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import oracle.attention as oa
    with ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"),
                             initializer=oa._limit_blas_threads) as ex:
        return list(ex.map(fn, tasks))


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


def fp8_score_error(q: np.ndarray, k: np.ndarray, scale: float, fq: float,
                    fk: float) -> np.ndarray:
    """Delta_i of every query row of one head: q [rows, d], k [Nk, d], dequantised with
    the factors fq, fk."""
    d = q.shape[1]
    mq = np.maximum(np.abs(q), 2.0 ** -6 * fq)          # M(q_ic) >= 2^e(q_ic) fq
    mk = np.maximum(np.abs(k), 2.0 ** -6 * fk).max(axis=0)  # max_j M(k_jc)
    maxprod = (mq * mk[None, :]).max(axis=1)            # >= max_j max_c M(q_ic) M(k_jc)
    smax = (np.abs(q) @ np.abs(k).max(axis=0)) * abs(scale)  # >= max_j |s_ij|
    return (d / 64) * 2.0 ** -8 * abs(scale) * maxprod + 2.0 ** -22 * smax


def fp8_o_bound(p: np.ndarray, v: np.ndarray, o_ref: np.ndarray, delta=0.0) -> np.ndarray:
    """Elementwise bound on |O - O_ref| for the fp8 forward of one head: p [rows, Nk] the
    oracle's probabilities of those rows, v [Nk, dv] the dequantised values, o_ref [rows, dv],
    delta the per-row score error bound (scalar or [rows])."""
    pmax = p.max(axis=1, keepdims=True)
    dlt = np.where(p > 0, np.maximum(2.0 ** -4 * p, 2.0 ** -10 * pmax), 0.0)
    big = np.exp(4.0 * np.reshape(np.asarray(delta, dtype=np.float64), (-1, 1)))
    pv = p @ np.abs(v)
    return (big * 1.001 * (dlt @ np.abs(v)) + (big - 1.0) * (pv + np.abs(o_ref))
            + 2.0 ** -8 * np.abs(o_ref) + 1e-6)


def check_fp8_lse(lse: np.ndarray, lse_ref: np.ndarray, delta: np.ndarray):
    err = np.abs(lse - lse_ref)
    assert np.isfinite(lse).all(), "LSE: non-finite output"
    worst = float((err / (LSE_MAX + delta)).max())
    assert worst <= 1.0, f"LSE: error reaches {worst:.2f} x the fp8 bound (max err {err.max():.3e})"
    return worst


def check_fp8_o(o: np.ndarray, o_ref: np.ndarray, bound: np.ndarray, what: str = "O"):
    err = np.abs(o - o_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{what}: error reaches {worst:.2f} x the fp8 rounding bound"
    return worst
