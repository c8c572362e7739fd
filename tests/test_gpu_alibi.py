"""GPU parity of the ALiBi position bias (alibi_slopes) in the bf16 forward and backward,
fixed-length and packed, against the float64 oracle with the same slopes."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa2_amd import fa
from exact_io_aware_fa2_amd.workloads import (ALIBI_WORKLOADS, VarlenWorkload, alibi_slopes,
                                              make_inputs, make_varlen_inputs, small_case)
from tests._parity import check_grad, check_lse, check_o, gpu_bwd, to64

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, d, causal, window)
SHAPES = [
    (1, 2, 1, 17, 64, True, 0),
    (2, 4, 2, 100, 128, False, 0),
    (1, 4, 2, 257, 128, True, 0),
    (1, 8, 8, 300, 64, True, 0),
    (1, 4, 1, 513, 128, True, 64),
    (1, 2, 2, 600, 128, False, 100),
    (1, 2, 2, 257, 256, True, 0),
    (1, 2, 1, 300, 256, False, 0),
    (1, 2, 2, 700, 256, True, 129),
]


def _ids(s):
    B, Hq, Hkv, N, d, causal, window = s
    return f"B{B}_Hq{Hq}_Hkv{Hkv}_N{N}_d{d}_{'causal' if causal else 'full'}_w{window}"


def _slope_sets(hq):
    return {"geometric": alibi_slopes(hq),
            "mixed_sign": [(-1) ** h * 0.3 / (h + 1) for h in range(hq)],
            "steep": [2.0 + h for h in range(hq)]}


@pytest.mark.parametrize("which", ["geometric", "mixed_sign", "steep"])
@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_alibi_forward_backward_small(shape, which):
    B, Hq, Hkv, N, d, causal, window = shape
    w = small_case(_ids(shape), "bf16", B, Hq, Hkv, N, d, causal, window, seed=71)
    q, k, v, do = make_inputs(w, "cuda")
    sl = _slope_sets(Hq)[which]
    slopes = torch.tensor(sl, dtype=torch.float32, device="cuda")
    o, lse = fa.forward(q, k, v, causal=causal, window=window, scale=w.scale, alibi_slopes=slopes)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, window=window, scale=w.scale,
                             alibi_slopes=slopes)
    torch.cuda.synchronize()
    sl32 = slopes.cpu().double().numpy()  # the float32 slopes the kernels read
    o_ref, lse_ref = oracle.attn_fwd(to64(q), to64(k), to64(v), causal, window, w.scale,
                                     alibi_slopes=sl32)
    check_o(to64(o), o_ref)
    check_lse(to64(lse), lse_ref)
    dq_r, dk_r, dv_r, _ = oracle.attn_bwd(to64(q), to64(k), to64(v), to64(do), causal, window,
                                          w.scale, alibi_slopes=sl32)
    check_grad(to64(dq), dq_r, "dQ")
    check_grad(to64(dk), dk_r, "dK")
    check_grad(to64(dv), dv_r, "dV")


@pytest.mark.parametrize("shape", [(1, 4, 2, 513, 128, True, 0), (1, 2, 2, 300, 64, False, 0),
                                   (1, 2, 2, 257, 256, True, 50)], ids=_ids)
def test_alibi_zero_slopes_equal_no_bias(shape):
    """Zero slopes reproduce the unbiased results: the backward bit for bit (same order of
    work), the forward up to the order in which it visits key tiles (the biased forward
    starts at the diagonal), i.e. float32 summation order before one bf16 rounding."""
    B, Hq, Hkv, N, d, causal, window = shape
    w = small_case(_ids(shape), "bf16", B, Hq, Hkv, N, d, causal, window, seed=72)
    q, k, v, do = make_inputs(w, "cuda")
    z = torch.zeros(Hq, dtype=torch.float32, device="cuda")
    o0, l0 = fa.forward(q, k, v, causal=causal, window=window, scale=w.scale)
    o1, l1 = fa.forward(q, k, v, causal=causal, window=window, scale=w.scale, alibi_slopes=z)
    g0 = fa.backward(q, k, v, o0, do, l0, causal=causal, window=window, scale=w.scale)
    g1 = fa.backward(q, k, v, o0, do, l0, causal=causal, window=window, scale=w.scale,
                     alibi_slopes=z)
    torch.cuda.synchronize()
    do_ = (o0.float() - o1.float()).abs()
    assert do_.max().item() <= 2.0 ** -7 * max(1.0, o0.float().abs().max().item())
    assert (l0 - l1).abs().max().item() <= 1e-5 * max(1.0, l0.abs().max().item())
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [True, False])
def test_alibi_packed_sequences(causal):
    lens, hq, hkv, d = (5, 0, 300, 1, 257, 64), 4, 2, 128
    w = VarlenWorkload("alibi_packed", lens, hq, hkv, d, causal, 0, seed=73)
    q, k, v, do = make_varlen_inputs(w, "cuda")
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    slopes = torch.tensor(alibi_slopes(hq), dtype=torch.float32, device="cuda")
    o, lse = fa.forward_varlen(q, k, v, cu, w.max_seqlen, causal, 0, w.scale, alibi_slopes=slopes)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, w.max_seqlen, causal, 0, w.scale,
                                    alibi_slopes=slopes)
    torch.cuda.synchronize()
    sl = slopes.cpu().double().numpy()
    o_ref, lse_ref = oracle.attn_fwd_varlen(to64(q), to64(k), to64(v), w.cu_seqlens, causal, 0,
                                            w.scale, alibi_slopes=sl)
    check_o(to64(o), o_ref)
    check_lse(to64(lse), lse_ref)
    g_ref = oracle.attn_bwd_varlen(to64(q), to64(k), to64(v), to64(do), w.cu_seqlens, causal, 0,
                                   w.scale, alibi_slopes=sl)
    for x, r, name in zip((dq, dk, dv), g_ref, ("dQ", "dK", "dV")):
        check_grad(to64(x), r, name)


def test_alibi_bench_workload_sampled():
    w = ALIBI_WORKLOADS["bf16_b2_h32_n8192_d128_causal_alibi"]
    q, k, v, do = make_inputs(w, "cuda")
    slopes = torch.tensor(alibi_slopes(w.Hq), dtype=torch.float32, device="cuda")
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale, alibi_slopes=slopes)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=w.causal, scale=w.scale,
                             alibi_slopes=slopes)
    torch.cuda.synchronize()
    sl = slopes.cpu().double().numpy()
    rng = np.random.default_rng(9)
    N = w.N
    rows = np.unique(np.clip(np.array([0, 1, 255, 256, N // 2, N - 2, N - 1] +
                                      list(rng.integers(0, N, 30))), 0, N - 1))
    o_c, lse_c, dq_c = o.float().cpu(), lse.cpu(), dq.float().cpu()
    for b, h in ((0, 0), (1, 31)):  # the steepest and the flattest slope
        qh, kh, vh, doh = to64(q[b, :, h]), to64(k[b, :, h]), to64(v[b, :, h]), to64(do[b, :, h])
        o_ref, lse_ref = oracle.attn_fwd_rows(qh, kh, vh, rows, True, 0, w.scale, slope=sl[h])
        check_o(o_c[b, rows, h].double().numpy(), o_ref, f"O[b{b},h{h}]")
        check_lse(lse_c[b, h, rows].double().numpy(), lse_ref)
        dq_ref, _ = oracle.attn_bwd_dq_rows(qh, kh, vh, doh, rows, True, 0, w.scale, slope=sl[h])
        check_grad(dq_c[b, rows, h].double().numpy(), dq_ref, f"dQ rows [b{b},h{h}]")
        cols = rows
        dk_ref, dv_ref = oracle.attn_bwd_dkdv_cols(qh, kh, vh, doh, cols, True, 0, w.scale,
                                                   slope=sl[h])
        check_grad(dk.float().cpu()[b, cols, h].double().numpy(), dk_ref, f"dK cols [b{b},h{h}]")
        check_grad(dv.float().cpu()[b, cols, h].double().numpy(), dv_ref, f"dV cols [b{b},h{h}]")


@pytest.mark.timeout(900)
def test_alibi_bench_workload_full_tensors():
    """The ALiBi bench workload (B 2, H 32, N 8192, causal, geometric slopes) over whole
    tensors: O, LSE, dQ, dK and dV of every head from the oracle with the same slopes."""
    from tests._parity import check_grad as cg, workers
    w = ALIBI_WORKLOADS["bf16_b2_h32_n8192_d128_causal_alibi"]
    q, k, v, do = make_inputs(w, "cuda")
    slopes = torch.tensor(alibi_slopes(w.Hq), dtype=torch.float32, device="cuda")
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale, alibi_slopes=slopes)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=w.causal, scale=w.scale,
                             alibi_slopes=slopes)
    torch.cuda.synchronize()
    sl = slopes.cpu().double().numpy()
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(do)
    print(f"{w.name}: oracle forward on {workers()} workers", flush=True)
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, w.causal, 0, w.scale, workers=workers(),
                                     alibi_slopes=sl)
    mx, mean = check_o(to64(o), o_ref)
    lerr = check_lse(to64(lse), lse_ref)
    del o_ref, lse_ref
    print(f"{w.name}: oracle backward", flush=True)
    dq_r, dk_r, dv_r, _ = oracle.attn_bwd(q64, k64, v64, do64, w.causal, 0, w.scale,
                                          workers=workers(), alibi_slopes=sl)
    errs = {n: cg(to64(x), r, n) for n, x, r in (("dQ", dq, dq_r), ("dK", dk, dk_r),
                                                 ("dV", dv, dv_r))}
    print(f"{w.name}: O max {mx:.3e} mean {mean:.3e}, LSE max {lerr:.3e}, "
          + ", ".join(f"{n} rel {e:.3e}" for n, e in errs.items()), flush=True)
