"""GPU parity on the measured workloads at their full sizes, in the launch configuration the
bench times (same entry points, same tensors, same stream use), against the float64 oracle.

Whole tensors (O, LSE, dQ, dK, dV) are compared for every workload the oracle finishes in
about half a minute on the host cores: the float32 workload, N = 2048, the N = 8192 bench
workload, the d = 256 workload and the 65536-token workload with a 4096-key window.  The
causal 65536-token workload (1.2e14 flop of float64 work for a whole backward) is compared
on: O and LSE of every head over every row; dK and dV of every KV group at three whole key
blocks, among them block 0, which every query row of the group's four heads reaches (the
longest accumulation the key-block kernel does); dQ of every head on a strided row sample.
The exact result is the target (unite.ai, "What is FlashAttention": exact attention), so the
tolerances are those of the bf16 inputs (tests/_parity.py).
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa2_amd.workloads import WORKLOADS, make_inputs
from tests._parity import (FP32_REL, check_grad, check_lse, check_o, gpu_bwd, gpu_fwd,
                           pool_map, rel_fro, to64, workers)

pytestmark = pytest.mark.gpu


def _full_tensors(w):
    q, k, v, do = make_inputs(w, "cuda")
    print(f"{w.name}: GPU forward + backward", flush=True)
    o, lse = gpu_fwd(q, k, v, w.causal, w.window, w.scale)
    dq, dk, dv = gpu_bwd(q, k, v, o, do, lse, w.causal, w.window, w.scale)
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(do)
    print(f"{w.name}: oracle forward on {workers()} workers", flush=True)
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, w.causal, w.window, w.scale,
                                     workers=workers())
    mx, mean = check_o(to64(o), o_ref)
    lerr = check_lse(to64(lse), lse_ref)
    del o_ref, lse_ref
    print(f"{w.name}: oracle backward", flush=True)
    dq_r, dk_r, dv_r, _ = oracle.attn_bwd(q64, k64, v64, do64, w.causal, w.window, w.scale,
                                          workers=workers())
    errs = {name: check_grad(to64(x), r, name)
            for name, x, r in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r))}
    print(f"{w.name}: O max {mx:.3e} mean {mean:.3e}, LSE max {lerr:.3e}, "
          + ", ".join(f"{n} rel {e:.3e}" for n, e in errs.items()), flush=True)


def test_fp32_b1_h2_n256_d64_full_tensors():
    w = WORKLOADS["fp32_b1_h2_n256_d64"]
    q, k, v, _ = make_inputs(w, "cuda")
    o, lse = gpu_fwd(q, k, v, w.causal, w.window, w.scale)
    o_ref, lse_ref = oracle.attn_fwd(to64(q), to64(k), to64(v), w.causal, w.window, w.scale)
    assert rel_fro(to64(o), o_ref) <= FP32_REL
    check_lse(to64(lse), lse_ref, tol=FP32_REL, rel=True)


def test_bf16_b2_h16_n2048_d128_causal_sigma4_full_tensors():
    _full_tensors(WORKLOADS["bf16_b2_h16_n2048_d128_causal_sigma4"])


@pytest.mark.timeout(900)
def test_bf16_b2_h32_n8192_d128_causal_full_tensors():
    _full_tensors(WORKLOADS["bf16_b2_h32_n8192_d128_causal"])


@pytest.mark.timeout(900)
def test_bf16_b1_h16_n16384_d256_full_tensors():
    _full_tensors(WORKLOADS["bf16_b1_h16_n16384_d256"])


@pytest.mark.timeout(900)
def test_bf16_b1_hq32_hkv8_n65536_d128_causal_window4096_full_tensors():
    _full_tensors(WORKLOADS["bf16_b1_hq32_hkv8_n65536_d128_causal_window4096"])


def _dkdv_cols_task(args):
    return oracle.attn_bwd_dkdv_cols_from_fwd(*args)


def _dq_rows_task(args):
    return oracle.attn_bwd_dq_rows(*args)[0]


@pytest.mark.timeout(900)
def test_bf16_b1_hq32_hkv8_n65536_d128_causal():
    w = WORKLOADS["bf16_b1_hq32_hkv8_n65536_d128_causal"]
    N, g = w.N, w.Hq // w.Hkv
    q, k, v, do = make_inputs(w, "cuda")
    print(f"{w.name}: GPU forward + backward", flush=True)
    o, lse = gpu_fwd(q, k, v, w.causal, w.window, w.scale)
    dq, dk, dv = gpu_bwd(q, k, v, o, do, lse, w.causal, w.window, w.scale)
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(do)
    # whole O and LSE of every head (the oracle's full forward)
    print(f"{w.name}: oracle forward on {workers()} workers", flush=True)
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, w.causal, w.window, w.scale,
                                     workers=workers())
    mx, mean = check_o(to64(o), o_ref)
    lerr = check_lse(to64(lse), lse_ref)
    print(f"{w.name}: O max {mx:.3e} mean {mean:.3e}, LSE max {lerr:.3e}", flush=True)
    # dK / dV at whole 256-key blocks of every KV group: block 0 (reached by all 65536 rows
    # of the group's 4 heads), a middle block and the last block; each query head's share
    # comes from the oracle's own O and LSE, summed over the group
    blocks = [np.arange(0, 256), np.arange(N // 2, N // 2 + 256), np.arange(N - 256, N)]
    tasks = [(q64[0, :, h], k64[0, :, h // g], v64[0, :, h // g], do64[0, :, h], o_ref[0, :, h],
              lse_ref[0, h], cols, w.causal, w.window, w.scale)
             for cols in blocks for h in range(w.Hq)]
    print(f"{w.name}: oracle dK/dV at {len(blocks)} key blocks x {w.Hkv} groups", flush=True)
    res = pool_map(_dkdv_cols_task, tasks)
    dk_c, dv_c = dk.float().cpu().numpy(), dv.float().cpu().numpy()
    for bi, cols in enumerate(blocks):
        dk_ref = np.zeros((w.Hkv, cols.size, w.d))
        dv_ref = np.zeros((w.Hkv, cols.size, w.d))
        for h in range(w.Hq):
            a, c = res[bi * w.Hq + h]
            dk_ref[h // g] += a
            dv_ref[h // g] += c
        for hk in range(w.Hkv):
            what = f"keys {cols[0]}..{cols[-1]}, KV head {hk}"
            check_grad(dk_c[0, cols, hk].astype(np.float64), dk_ref[hk], "dK " + what)
            check_grad(dv_c[0, cols, hk].astype(np.float64), dv_ref[hk], "dV " + what)
        ek = rel_fro(dk_c[0, cols].transpose(1, 0, 2).astype(np.float64), dk_ref)
        ev = rel_fro(dv_c[0, cols].transpose(1, 0, 2).astype(np.float64), dv_ref)
        print(f"{w.name}: keys {cols[0]}..{cols[-1]} dK rel {ek:.3e} dV rel {ev:.3e}", flush=True)
    del o_ref
    # dQ of every head on a strided sample of rows (each row's full softmax row)
    rows = np.unique(np.concatenate([np.arange(0, N, 1024), np.arange(511, N, 2048),
                                     [1, 255, 256, N - 2, N - 1]]))
    tasks = [(q64[0, :, h], k64[0, :, h // g], v64[0, :, h // g], do64[0, :, h], rows, w.causal,
              w.window, w.scale) for h in range(w.Hq)]
    print(f"{w.name}: oracle dQ at {rows.size} rows x {w.Hq} heads", flush=True)
    dq_ref = np.stack(pool_map(_dq_rows_task, tasks), axis=1)  # [rows, Hq, d]
    e = check_grad(dq.float().cpu().numpy()[0, rows].astype(np.float64), dq_ref, "dQ rows")
    print(f"{w.name}: dQ sampled rows rel {e:.3e}", flush=True)
    # properties of the whole gradient tensors
    dq_c = dq.float().cpu()
    assert torch.isfinite(dq_c).all() and np.isfinite(dk_c).all() and np.isfinite(dv_c).all()
    sum_dk = np.abs(dk_c.astype(np.float64).sum(axis=1))
    assert (sum_dk <= 3e-2 * np.abs(dk_c.astype(np.float64)).sum(axis=1)).all()
    ref_dv = do64.sum(axis=1).reshape(w.B, w.Hkv, g, w.d).sum(axis=2)
    err = np.abs(dv_c.astype(np.float64).sum(axis=1) - ref_dv)
    assert (err <= 3e-2 * np.abs(ref_dv).max()).all(), err.max()
