"""GPU parity of the 8-bit forward (fa_fwd_fp8) against the float64 oracle.

The oracle is the exact attention of the dequantised inputs.  The kernel's 8-bit products
sum with less than float32 precision and it rounds its probability weights to E4M3 before
the second product, so random inputs are checked against the per-row bounds derived in
tests/_parity.py (fp8_score_error, fp8_o_bound, check_fp8_lse).
Inputs whose scores are small integers with a unit log2 scale make every weight an exact
power of two: there the rounding is exact and O must meet the bf16 tolerances too, which
checks tiling, masks and normalisation tightly.  The 8-bit bench workload is checked over
whole tensors against the same per-row bounds.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa2_amd import fa
from exact_io_aware_fa2_amd.workloads import FP8_WORKLOADS, make_fp8_inputs, quantize_e4m3
from tests._parity import (check_fp8_lse, check_fp8_o, check_lse, check_o, fp8_o_bound,
                           fp8_score_error)

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, d, causal, window)
SHAPES = [
    (1, 1, 1, 1, 64, False, 0),
    (1, 2, 1, 17, 128, True, 0),
    (2, 2, 2, 100, 128, False, 0),
    (1, 4, 2, 255, 128, True, 0),
    (1, 4, 4, 257, 64, True, 0),
    (1, 2, 2, 257, 256, False, 0),
    (1, 2, 1, 300, 256, True, 0),
    (1, 4, 1, 513, 128, True, 1),
    (1, 4, 2, 513, 128, True, 64),
    (1, 2, 2, 600, 128, False, 100),
    (1, 2, 2, 700, 256, True, 129),
    (2, 8, 8, 1000, 64, True, 0),
]


def _ids(s):
    B, Hq, Hkv, N, d, causal, window = s
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_N{N}_d{d}_{'causal' if causal else 'full'}_w{window}"


def _codes(x):
    return x.view(torch.uint8).cpu().numpy()


def _random_case(shape, seed, sigma=1.0):
    B, Hq, Hkv, N, d, causal, window = shape
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn((B, N, h, d), generator=g) * s
          for h, s in ((Hq, sigma), (Hkv, sigma), (Hkv, 1.0))]
    out = [quantize_e4m3(x) for x in xs]
    return [c.cuda() for c, _ in out], [f for _, f in out]


def _check_random(shape, codes, factors, scale):
    B, Hq, Hkv, N, d, causal, window = shape
    q8, k8, v8 = codes
    o, lse = fa.forward_fp8(q8, k8, v8, *factors, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    qd, kd, vd = (oracle.dequantize(_codes(t), f) for t, f in zip(codes, factors))
    o_ref, lse_ref = oracle.attn_fwd(qd, kd, vd, causal, window, scale)
    o64 = o.float().cpu().double().numpy()
    lse64 = lse.cpu().double().numpy()
    g = Hq // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            delta = fp8_score_error(qd[b, :, h], kd[b, :, h // g], scale, float(factors[0]),
                                   float(factors[1]))
            check_fp8_lse(lse64[b, h], lse_ref[b, h], delta)
            p = oracle.attention_probs(qd[b, :, h], kd[b, :, h // g], causal, window, scale)
            bound = fp8_o_bound(p, vd[b, :, h // g], o_ref[b, :, h], delta)
            worst = max(worst, check_fp8_o(o64[b, :, h], o_ref[b, :, h], bound, f"O[b{b},h{h}]"))
    return worst


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_fp8_forward_random_within_bound(shape):
    codes, factors = _random_case(shape, seed=61)
    _check_random(shape, codes, factors, 1.0 / math.sqrt(shape[4]))


@pytest.mark.parametrize("shape", [(1, 2, 2, 300, 128, True, 0), (1, 2, 1, 200, 64, False, 50)],
                         ids=_ids)
def test_fp8_forward_large_logits_and_negative_scale(shape):
    codes, factors = _random_case(shape, seed=62, sigma=4.0)
    _check_random(shape, codes, factors, 1.0 / math.sqrt(shape[4]))
    _check_random(shape, codes, factors, -0.7 / math.sqrt(shape[4]))


def _exact_weight_case(shape, seed):
    """Q rows with at most two entries +-1, K entries in {-2..2}: integer scores in [-4, 4].
    With descale 1 and scale ln 2 the kernel's log2 factor is 1, so every weight is a power
    of two in [2^-8, 2^8], exact in E4M3."""
    B, Hq, Hkv, N, d, causal, window = shape
    rng = np.random.default_rng(seed)
    q = np.zeros((B, N, Hq, d))
    idx = rng.integers(0, d, size=(B, N, Hq, 2))
    val = rng.choice([-1.0, 1.0], size=(B, N, Hq, 2))
    np.put_along_axis(q, idx[..., :1], val[..., :1], axis=3)
    np.put_along_axis(q, idx[..., 1:], val[..., 1:], axis=3)
    k = rng.integers(-2, 3, size=(B, N, Hkv, d)).astype(np.float64)
    v = torch.randn((B, N, Hkv, d), generator=torch.Generator().manual_seed(seed))
    v8, fv = quantize_e4m3(v)
    to8 = lambda a: torch.tensor(a, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)  # noqa: E731
    return [to8(q).cuda(), to8(k).cuda(), v8.cuda()], [1.0, 1.0, fv]


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_fp8_forward_exact_weights_meet_bf16_tolerance(shape):
    B, Hq, Hkv, N, d, causal, window = shape
    codes, factors = _exact_weight_case(shape, seed=63)
    scale = math.log(2.0)
    o, lse = fa.forward_fp8(*codes, *factors, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    qd, kd, vd = (oracle.dequantize(_codes(t), f) for t, f in zip(codes, factors))
    o_ref, lse_ref = oracle.attn_fwd(qd, kd, vd, causal, window, scale)
    check_o(o.float().cpu().double().numpy(), o_ref)
    check_lse(lse.cpu().double().numpy(), lse_ref)


def test_fp8_forward_is_deterministic():
    shape = (1, 4, 2, 513, 128, True, 0)
    codes, factors = _random_case(shape, seed=64)
    a = fa.forward_fp8(*codes, *factors, causal=True)
    b = fa.forward_fp8(*codes, *factors, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _rows(N, rng, extra=40):
    fixed = [0, 1, 2, 63, 64, 255, 256, N // 2, N - 257, N - 256, N - 2, N - 1]
    return np.unique(np.clip(np.array(fixed + list(rng.integers(0, N, size=extra))), 0, N - 1))


def test_fp8_bench_workload_sampled():
    w = FP8_WORKLOADS["fp8_b2_h32_n8192_d128_causal"]
    q8, k8, v8, factors = make_fp8_inputs(w, "cuda")
    o, lse = fa.forward_fp8(q8, k8, v8, *factors, causal=w.causal, window=w.window,
                            scale=w.scale)
    torch.cuda.synchronize()
    o_c, lse_c = o.float().cpu(), lse.cpu()
    assert torch.isfinite(o_c).all() and torch.isfinite(lse_c).all()
    rng = np.random.default_rng(7)
    rows = _rows(w.N, rng)
    g = w.Hq // w.Hkv
    for b, h in ((0, 0), (1, 17), (1, w.Hq - 1)):
        qd = oracle.dequantize(_codes(q8[b, :, h]), factors[0])
        kd = oracle.dequantize(_codes(k8[b, :, h // g]), factors[1])
        vd = oracle.dequantize(_codes(v8[b, :, h // g]), factors[2])
        o_ref, lse_ref = oracle.attn_fwd_rows(qd, kd, vd, rows, w.causal, w.window, w.scale)
        p = oracle.attention_probs_rows(qd, kd, rows, w.causal, w.window, w.scale)
        delta = fp8_score_error(qd[rows], kd, w.scale, float(factors[0]),
                                   float(factors[1]))
        check_fp8_o(o_c[b, rows, h].double().numpy(), o_ref, fp8_o_bound(p, vd, o_ref, delta),
                    f"O[b{b},h{h}]")
        check_fp8_lse(lse_c[b, h, rows].double().numpy(), lse_ref, delta)


def _fp8_head_task(args):
    """Worst error / bound ratios (O, LSE) of one head of the fp8 forward against the float64
    oracle of the dequantised inputs, every row, in chunks of rows."""
    qd, kd, vd, o, lse, causal, window, scale, fq, fk = args
    worst_o = worst_l = 0.0
    for r0 in range(0, qd.shape[0], 512):
        rows = np.arange(r0, min(r0 + 512, qd.shape[0]))
        o_ref, lse_ref = oracle.attn_fwd_rows(qd, kd, vd, rows, causal, window, scale)
        p = oracle.attention_probs_rows(qd, kd, rows, causal, window, scale)
        delta = fp8_score_error(qd[rows], kd, scale, fq, fk)
        worst_o = max(worst_o, check_fp8_o(o[rows], o_ref, fp8_o_bound(p, vd, o_ref, delta)))
        worst_l = max(worst_l, check_fp8_lse(lse[rows], lse_ref, delta))
    return worst_o, worst_l


@pytest.mark.timeout(900)
def test_fp8_bench_workload_full_tensors():
    """The 8-bit bench workload over whole tensors: every row of every head within the
    per-element bounds of the derived fp8 tolerance."""
    from tests._parity import pool_map, workers
    w = FP8_WORKLOADS["fp8_b2_h32_n8192_d128_causal"]
    q8, k8, v8, factors = make_fp8_inputs(w, "cuda")
    o, lse = fa.forward_fp8(q8, k8, v8, *factors, causal=w.causal, window=w.window,
                            scale=w.scale)
    torch.cuda.synchronize()
    o_c, lse_c = o.double().cpu().numpy(), lse.double().cpu().numpy()
    g = w.Hq // w.Hkv
    qc, kc, vc = _codes(q8), _codes(k8), _codes(v8)
    tasks = [(oracle.dequantize(qc[b, :, h], factors[0]), oracle.dequantize(kc[b, :, h // g], factors[1]),
              oracle.dequantize(vc[b, :, h // g], factors[2]), o_c[b, :, h], lse_c[b, h], w.causal,
              w.window, w.scale, float(factors[0]), float(factors[1]))
             for b in range(w.B) for h in range(w.Hq)]
    print(f"{w.name}: oracle and bounds over {len(tasks)} heads on {workers()} workers", flush=True)
    res = pool_map(_fp8_head_task, tasks)
    print(f"{w.name}: worst O error / bound {max(r[0] for r in res):.3f}, "
          f"worst LSE error / bound {max(r[1] for r in res):.3f}", flush=True)
