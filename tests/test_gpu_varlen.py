"""GPU parity for packed variable-length sequences (fa_fwd_varlen / fa_bwd_varlen).

Small batches are compared over whole tensors with the float64 oracle's packed-sequence
functions; the batches mix empty, one-row, ragged and multi-tile sequences under every mask.
The packed 16384-row workload the bench times is compared over whole tensors, and on
sampled rows and columns of each sequence together with per-sequence properties that hold at
any size.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa2_amd import fa
from exact_io_aware_fa2_amd.workloads import (VARLEN_WORKLOADS, VarlenWorkload,
                                              make_varlen_inputs)
from tests._parity import check_grad, check_lse, check_o, to64

pytestmark = pytest.mark.gpu

# (lengths, Hq, Hkv, d, causal, window)
CASES = [
    ((1,), 1, 1, 64, False, 0),
    ((5, 0, 1, 17, 300, 257), 4, 2, 128, True, 0),
    ((0, 700, 33, 0), 2, 2, 256, True, 129),
    ((256, 256, 255), 8, 2, 64, False, 0),
    ((1000, 3, 513), 4, 1, 128, True, 64),
    ((130, 2, 64, 65, 129), 2, 2, 256, False, 33),
    ((600, 1, 400), 2, 2, 128, False, 100),
    ((31, 32, 33, 63, 64, 65, 255, 256, 257), 2, 1, 128, True, 0),
]


def _ids(c):
    lens, hq, hkv, d, causal, window = c
    return f"L{'-'.join(map(str, lens))}_Hq{hq}_Hkv{hkv}_d{d}_{'causal' if causal else 'full'}_w{window}"


def _cu(w, device="cuda"):
    return torch.tensor(w.cu_seqlens, dtype=torch.int32, device=device)


def _run(w, max_seqlen=None):
    q, k, v, do = make_varlen_inputs(w, "cuda")
    cu = _cu(w)
    ms = w.max_seqlen if max_seqlen is None else max_seqlen
    o, lse = fa.forward_varlen(q, k, v, cu, ms, w.causal, w.window, w.scale)
    ws = fa.workspace_for_varlen(w.total, w.Hq, w.Hkv, w.d, q.device)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, ms, w.causal, w.window, w.scale,
                                    workspace=ws)
    torch.cuda.synchronize()
    return (q, k, v, do), (o, lse, dq, dk, dv, ws)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_varlen_forward_backward_small(case):
    lens, hq, hkv, d, causal, window = case
    w = VarlenWorkload(_ids(case), lens, hq, hkv, d, causal, window, seed=31)
    (q, k, v, do), (o, lse, dq, dk, dv, ws) = _run(w)
    cu = w.cu_seqlens
    o_ref, lse_ref = oracle.attn_fwd_varlen(to64(q), to64(k), to64(v), cu, causal, window,
                                            w.scale)
    check_o(to64(o), o_ref)
    check_lse(to64(lse), lse_ref)
    dq_r, dk_r, dv_r, dvec_r = oracle.attn_bwd_varlen(to64(q), to64(k), to64(v), to64(do), cu,
                                                      causal, window, w.scale)
    check_grad(to64(dq), dq_r, "dQ")
    check_grad(to64(dk), dk_r, "dK")
    check_grad(to64(dv), dv_r, "dV")
    dvec = to64(ws[: hq * w.total * 4].view(torch.float32).view(hq, w.total))
    assert np.abs(dvec - dvec_r).max() <= 2e-2 * max(1.0, np.abs(dvec_r).max())


def test_varlen_loose_max_seqlen_gives_identical_results():
    """max_seqlen only sizes the grid: a looser bound (up to total) changes nothing."""
    w = VarlenWorkload("loose", (70, 0, 200, 9), 4, 2, 128, True, 0, seed=32)
    _, tight = _run(w)
    _, loose = _run(w, max_seqlen=w.total)
    for a, b in zip(tight[:5], loose[:5]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,causal,window", [(64, False, 0), (128, True, 0), (256, True, 100)])
def test_varlen_equal_lengths_match_fixed_batch_bitwise(d, causal, window):
    """Equal-length sequences packed back to back are a batch in the fixed layout; both
    entry points must run the very same arithmetic."""
    n, nb, hq, hkv = 333, 3, 4, 2
    w = VarlenWorkload("equal", (n,) * nb, hq, hkv, d, causal, window, seed=33)
    (q, k, v, do), (o, lse, dq, dk, dv, _) = _run(w)
    qb, kb, vb, dob = (t.view(nb, n, t.shape[1], d) for t in (q, k, v, do))
    ob, lseb = fa.forward(qb, kb, vb, causal=causal, window=window, scale=w.scale)
    dqb, dkb, dvb = fa.backward(qb, kb, vb, ob, dob, lseb, causal=causal, window=window,
                                scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ob.view_as(o))
    assert torch.equal(lse, lseb.permute(1, 0, 2).reshape(hq, nb * n))
    assert torch.equal(dq, dqb.view_as(dq))
    assert torch.equal(dk, dkb.view_as(dk))
    assert torch.equal(dv, dvb.view_as(dv))


def _sample(n, rng, extra=12):
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, n // 2, n - 129, n - 2, n - 1]
    return np.unique(np.clip(np.array(fixed + list(rng.integers(0, n, size=extra))), 0, n - 1))


def test_varlen_packed_workload_sampled():
    w = VARLEN_WORKLOADS["bf16_varlen_t16384_h32_d128_causal"]
    (q, k, v, do), (o, lse, dq, dk, dv, _) = _run(w)
    g = w.Hq // w.Hkv
    rng = np.random.default_rng(5)
    o_c, lse_c, dq_c = o.float().cpu(), lse.cpu(), dq.float().cpu()
    dk_c, dv_c, do_c = dk.float().cpu(), dv.float().cpu(), do.float().cpu()
    q_c, k_c, v_c = q.float().cpu(), k.float().cpu(), v.float().cpu()
    cu = w.cu_seqlens
    for s, n in enumerate(w.lengths):
        a = cu[s]
        rows = _sample(n, rng)
        for h in (0, w.Hq - 1 - s % w.Hq):
            hk = h // g
            qh = q_c[a:a + n, h].double().numpy()
            kh = k_c[a:a + n, hk].double().numpy()
            vh = v_c[a:a + n, hk].double().numpy()
            doh = do_c[a:a + n, h].double().numpy()
            o_ref, lse_ref = oracle.attn_fwd_rows(qh, kh, vh, rows, w.causal, w.window, w.scale)
            check_o(o_c[a + rows, h].double().numpy(), o_ref, f"O[seq{s},h{h}]")
            check_lse(lse_c[h, a + rows].double().numpy(), lse_ref)
            dq_ref, _ = oracle.attn_bwd_dq_rows(qh, kh, vh, doh, rows, w.causal, w.window,
                                                w.scale)
            check_grad(dq_c[a + rows, h].double().numpy(), dq_ref, f"dQ[seq{s},h{h}]")
        # dK / dV columns of KV head 0: sum over its query heads
        cols = _sample(n, rng, extra=4)
        dk_ref = np.zeros((cols.size, w.d))
        dv_ref = np.zeros((cols.size, w.d))
        for h in range(g):
            x, y = oracle.attn_bwd_dkdv_cols(q_c[a:a + n, h].double().numpy(),
                                             k_c[a:a + n, 0].double().numpy(),
                                             v_c[a:a + n, 0].double().numpy(),
                                             do_c[a:a + n, h].double().numpy(), cols, w.causal,
                                             w.window, w.scale)
            dk_ref += x
            dv_ref += y
        check_grad(dk_c[a + cols, 0].double().numpy(), dk_ref, f"dK cols seq{s}")
        check_grad(dv_c[a + cols, 0].double().numpy(), dv_ref, f"dV cols seq{s}")
        # per-sequence properties on the full tensors: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
        sdk = dk_c[a:a + n].double().sum(dim=0)
        assert sdk.abs().max().item() <= 3e-2 * dk_c[a:a + n].double().abs().sum(dim=0).max().item()
        ref_dv = do_c[a:a + n].double().sum(dim=0).view(w.Hkv, g, w.d).sum(dim=1)
        err = (dv_c[a:a + n].double().sum(dim=0) - ref_dv).abs().max().item()
        assert err <= 3e-2 * ref_dv.abs().max().item() + 0.5, (s, err)
    for t in (o_c, lse_c, dq_c, dk_c, dv_c):
        assert torch.isfinite(t).all()


def _seq_head_task(args):
    """Forward and backward of one (sequence, head) pair with the float64 oracle."""
    q, k, v, do, causal, window, scale = args
    o, lse = oracle.attn_fwd_head(q, k, v, causal, window, scale)
    dq, dk, dv, _ = oracle.attn_bwd_head(q, k, v, do, causal, window, scale)
    return o, lse, dq, dk, dv


@pytest.mark.timeout(900)
def test_varlen_packed_workload_full_tensors():
    """The packed 16384-row bench workload over whole tensors: every (sequence, head) pair's
    O, LSE, dQ and its share of dK / dV from the oracle, at the bf16 tolerances."""
    from tests._parity import pool_map, workers
    w = VARLEN_WORKLOADS["bf16_varlen_t16384_h32_d128_causal"]
    (q, k, v, do), (o, lse, dq, dk, dv, _) = _run(w)
    g = w.Hq // w.Hkv
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(do)
    cu = w.cu_seqlens
    pairs = [(s, h) for s in range(len(w.lengths)) for h in range(w.Hq) if w.lengths[s] > 0]
    print(f"{w.name}: oracle over {len(pairs)} (sequence, head) pairs on {workers()} workers",
          flush=True)
    res = pool_map(_seq_head_task, [
        (q64[cu[s]:cu[s + 1], h], k64[cu[s]:cu[s + 1], h // g], v64[cu[s]:cu[s + 1], h // g],
         do64[cu[s]:cu[s + 1], h], w.causal, w.window, w.scale) for s, h in pairs])
    o_ref, lse_ref = np.zeros_like(q64), np.zeros((w.Hq, w.total))
    dq_ref, dk_ref, dv_ref = np.zeros_like(q64), np.zeros_like(k64), np.zeros_like(v64)
    for (s, h), (oh, lh, dqh, dkh, dvh) in zip(pairs, res):
        a, b = cu[s], cu[s + 1]
        o_ref[a:b, h], lse_ref[h, a:b], dq_ref[a:b, h] = oh, lh, dqh
        dk_ref[a:b, h // g] += dkh
        dv_ref[a:b, h // g] += dvh
    mx, mean = check_o(to64(o), o_ref)
    lerr = check_lse(to64(lse), lse_ref)
    errs = {n: check_grad(to64(x), r, n) for n, x, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref),
                                                          ("dV", dv, dv_ref))}
    print(f"{w.name}: O max {mx:.3e} mean {mean:.3e}, LSE max {lerr:.3e}, "
          + ", ".join(f"{n} rel {e:.3e}" for n, e in errs.items()), flush=True)
