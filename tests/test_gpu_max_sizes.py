"""GPU parity at the largest sizes the entry points accept: every query-side tensor just
under 2^31 elements, the limit of the kernels' 32-bit row and buffer-offset arithmetic
(anything larger is rejected, see test_abi.py).

Sliding windows keep the work linear in N.  The oracle evaluates sampled rows and columns
where the offsets are largest (last batch entry, last head, last rows), in the middle and
at the start, each on a slice of the sequence that holds every key and query row those
outputs depend on: with a causal window w, row i reads keys [i - w + 1, i] and key j is read
by rows [j, j + w - 1], so rows [lo, hi) need keys from lo - w + 1 and columns [lo, hi) need
rows up to hi + w - 2 (rows of the slice whose own keys were cut off lie before lo and, being
causal, never reach a sampled column).
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa2_amd import fa
from exact_io_aware_fa2_amd.workloads import MAX_ELEMS, device_normal, quantize_e4m3
from tests._parity import (check_fp8_lse, check_fp8_o, check_grad, check_lse, check_o,
                           fp8_o_bound, fp8_score_error, gpu_bwd, gpu_fwd, to64)

pytestmark = pytest.mark.gpu

B, HQ, HKV, D = 2, 8, 2, 128
N_MAX = (MAX_ELEMS - 1) // (B * HQ * D)  # 1048575: B*N*Hq*d = 2^31 - 2048
WINDOW = 192
SCALE = D ** -0.5


def _span(lo, hi, n, window):
    """Slice [s, e) of a sequence of n rows that determines rows and columns [lo, hi)."""
    return max(0, lo - window + 1), min(n, hi + window - 1)


def _free(*ts):
    del ts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _samples(n):
    return [(0, 40), (n // 2 - 20, n // 2 + 20), (n - 40, n)]


def test_bf16_forward_backward_at_the_size_limit():
    assert B * N_MAX * HQ * D < MAX_ELEMS <= B * (N_MAX + 1) * HQ * D
    dev = "cuda"
    q = device_normal((B, N_MAX, HQ, D), 901, dev)
    k = device_normal((B, N_MAX, HKV, D), 902, dev)
    v = device_normal((B, N_MAX, HKV, D), 903, dev)
    do = device_normal((B, N_MAX, HQ, D), 904, dev)
    o, lse = gpu_fwd(q, k, v, True, WINDOW, SCALE)
    dq, dk, dv = gpu_bwd(q, k, v, o, do, lse, True, WINDOW, SCALE)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all().item()
    g = HQ // HKV
    for (b, h), (lo, hi) in zip([(0, 0), (1, 3), (B - 1, HQ - 1)], _samples(N_MAX)):
        s, e = _span(lo, hi, N_MAX, WINDOW)
        rows = np.arange(lo, hi) - s
        qh, kh, vh, doh = (to64(x[b, s:e, hh]) for x, hh in
                           ((q, h), (k, h // g), (v, h // g), (do, h)))
        o_ref, lse_ref = oracle.attn_fwd_rows(qh, kh, vh, rows, True, WINDOW, SCALE)
        check_o(to64(o[b, lo:hi, h]), o_ref, f"O[b{b},h{h},{lo}:{hi}]")
        check_lse(to64(lse[b, h, lo:hi]), lse_ref)
        dq_ref, _ = oracle.attn_bwd_dq_rows(qh, kh, vh, doh, rows, True, WINDOW, SCALE)
        check_grad(to64(dq[b, lo:hi, h]), dq_ref, f"dQ[b{b},h{h},{lo}:{hi}]")
        hk = h // g
        dk_ref = np.zeros((hi - lo, D))
        dv_ref = np.zeros((hi - lo, D))
        for hq in range(hk * g, (hk + 1) * g):
            a, c = oracle.attn_bwd_dkdv_cols(to64(q[b, s:e, hq]), kh, vh, to64(do[b, s:e, hq]),
                                             rows, True, WINDOW, SCALE)
            dk_ref += a
            dv_ref += c
        check_grad(to64(dk[b, lo:hi, hk]), dk_ref, f"dK[b{b},h{hk},{lo}:{hi}]")
        check_grad(to64(dv[b, lo:hi, hk]), dv_ref, f"dV[b{b},h{hk},{lo}:{hi}]")
    _free(q, k, v, do, o, lse, dq, dk, dv)


def test_fp8_forward_at_the_size_limit():
    dev = "cuda"
    codes, factors = [], []
    for shape, seed in (((B, N_MAX, HQ, D), 911), ((B, N_MAX, HKV, D), 912),
                        ((B, N_MAX, HKV, D), 913)):
        c, f = quantize_e4m3(device_normal(shape, seed, dev))
        codes.append(c)
        factors.append(f)
    o, lse = fa.forward_fp8(*codes, *factors, causal=True, window=WINDOW, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    g = HQ // HKV
    for (b, h), (lo, hi) in zip([(0, 1), (1, 4), (B - 1, HQ - 1)], _samples(N_MAX)):
        s, e = _span(lo, hi, N_MAX, WINDOW)
        rows = np.arange(lo, hi) - s
        qd, kd, vd = (oracle.dequantize(x[b, s:e, hh].cpu().numpy(), f) for x, hh, f in
                      ((codes[0], h, factors[0]), (codes[1], h // g, factors[1]),
                       (codes[2], h // g, factors[2])))
        o_ref, lse_ref = oracle.attn_fwd_rows(qd, kd, vd, rows, True, WINDOW, SCALE)
        p = oracle.attention_probs_rows(qd, kd, rows, True, WINDOW, SCALE)
        delta = fp8_score_error(qd[rows], kd, SCALE, float(factors[0]), float(factors[1]))
        check_fp8_o(to64(o[b, lo:hi, h]), o_ref, fp8_o_bound(p, vd, o_ref, delta),
                    f"O[b{b},h{h},{lo}:{hi}]")
        check_fp8_lse(to64(lse[b, h, lo:hi]), lse_ref, delta)
    _free(*codes, o, lse)


def test_varlen_forward_backward_at_the_size_limit():
    total = (MAX_ELEMS - 1) // (HQ * D)  # 2097151 packed rows
    lens = [1, 1048575, 0, 700001]
    lens.append(total - sum(lens))
    cu_host = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    assert cu_host[-1] == total and total * HQ * D < MAX_ELEMS
    dev = "cuda"
    q = device_normal((total, HQ, D), 921, dev)
    k = device_normal((total, HKV, D), 922, dev)
    v = device_normal((total, HKV, D), 923, dev)
    do = device_normal((total, HQ, D), 924, dev)
    cu = torch.tensor(cu_host, dtype=torch.int32, device=dev)
    ms = max(lens)
    o, lse = fa.forward_varlen(q, k, v, cu, ms, True, WINDOW, SCALE)
    ws = fa.workspace_for_varlen(total, HQ, HKV, D, q.device)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, ms, True, WINDOW, SCALE,
                                    workspace=ws)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all().item()
    g = HQ // HKV
    # (sequence, query head, rows inside the sequence)
    picks = [(1, 0, (0, 40)), (1, 5, (lens[1] - 40, lens[1])), (3, 2, (350000, 350040)),
             (4, HQ - 1, (lens[4] - 40, lens[4])), (0, HQ - 1, (0, 1))]
    for sq, h, (lo, hi) in picks:
        n, off = lens[sq], int(cu_host[sq])
        s, e = _span(lo, hi, n, WINDOW)
        rows = np.arange(lo, hi) - s
        sl = slice(off + s, off + e)
        qh, kh, vh, doh = (to64(x[sl, hh]) for x, hh in ((q, h), (k, h // g), (v, h // g),
                                                         (do, h)))
        o_ref, lse_ref = oracle.attn_fwd_rows(qh, kh, vh, rows, True, WINDOW, SCALE)
        check_o(to64(o[off + lo:off + hi, h]), o_ref, f"O[seq{sq},h{h},{lo}:{hi}]")
        check_lse(to64(lse[h, off + lo:off + hi]), lse_ref)
        dq_ref, _ = oracle.attn_bwd_dq_rows(qh, kh, vh, doh, rows, True, WINDOW, SCALE)
        check_grad(to64(dq[off + lo:off + hi, h]), dq_ref, f"dQ[seq{sq},h{h}]")
        hk = h // g
        dk_ref = np.zeros((hi - lo, D))
        dv_ref = np.zeros((hi - lo, D))
        for hq in range(hk * g, (hk + 1) * g):
            a, c = oracle.attn_bwd_dkdv_cols(to64(q[sl, hq]), kh, vh, to64(do[sl, hq]), rows,
                                             True, WINDOW, SCALE)
            dk_ref += a
            dv_ref += c
        check_grad(to64(dk[off + lo:off + hi, hk]), dk_ref, f"dK[seq{sq},h{hk}]")
        check_grad(to64(dv[off + lo:off + hi, hk]), dv_ref, f"dV[seq{sq},h{hk}]")
    _free(q, k, v, do, o, lse, dq, dk, dv, ws)


def test_decode_at_the_size_limit():
    Bd, Hq, Hkv, Nq = 4, 32, 8, 1
    nk = (MAX_ELEMS - 1) // (Bd * Hq * D)  # 131071 cached rows
    lens = [nk, 1, 65536, nk - 1]
    dev = "cuda"
    q = device_normal((Bd, Nq, Hq, D), 931, dev)
    k = device_normal((Bd, nk, Hkv, D), 932, dev)
    v = device_normal((Bd, nk, Hkv, D), 933, dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o, lse = fa.decode(q, k, v, sl, True, 0, SCALE)
    torch.cuda.synchronize()
    for b in (0, 1, Bd - 1):
        n = lens[b]
        o_ref, lse_ref = oracle.attn_decode(to64(q[b:b + 1]), to64(k[b:b + 1, :n]),
                                            to64(v[b:b + 1, :n]), [n], True, 0, SCALE)
        check_o(to64(o[b:b + 1]), o_ref, f"O[b{b}]")
        check_lse(to64(lse[b:b + 1]), lse_ref)
    _free(q, k, v, o, lse)
