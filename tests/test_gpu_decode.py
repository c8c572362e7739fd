"""GPU parity of fa_decode (the newest queries over a KV cache, split over the keys and
merged) against the float64 oracle's attn_decode."""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa2_amd import fa
from exact_io_aware_fa2_amd.workloads import DECODE_WORKLOADS, DecodeWorkload, make_decode_inputs
from tests._parity import check_lse, check_o, to64

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Nq, Nk, d, causal, window, lengths, num_splits)
CASES = [
    (1, 1, 1, 1, 1, 64, True, 0, None, 1),
    (2, 4, 2, 1, 300, 128, True, 0, (300, 17), 0),
    (2, 8, 2, 4, 1000, 128, True, 0, (1000, 513), 3),
    (1, 32, 8, 1, 4097, 128, True, 0, None, 0),
    (3, 4, 4, 2, 700, 64, False, 0, (700, 1, 0), 5),
    (2, 4, 1, 3, 2000, 128, True, 129, (2000, 130), 0),
    (1, 16, 2, 5, 800, 128, True, 0, None, 7),
    (1, 2, 2, 1, 50, 64, True, 0, None, 16),
    (2, 8, 8, 8, 333, 64, False, 40, (333, 100), 2),
]


def _ids(c):
    B, Hq, Hkv, Nq, Nk, d, causal, window, lens, ns = c
    return (f"B{B}_Hq{Hq}_Hkv{Hkv}_Nq{Nq}_Nk{Nk}_d{d}_{'causal' if causal else 'full'}_w{window}"
            f"_L{'-'.join(map(str, lens)) if lens else 'all'}_s{ns}")


def _check(o, lse, o_ref, lse_ref):
    """Rows with no allowed key must give O = 0 and LSE = -inf; the rest the usual bf16
    tolerances."""
    lse64 = to64(lse)
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse64), dead)
    o64 = to64(o)
    dead_rows = dead.transpose(0, 2, 1)  # [B, Nq, Hq]
    assert np.all(o64[dead_rows] == 0.0)
    live = ~dead_rows
    if live.any():
        check_o(o64[live], o_ref[live])
        check_lse(lse64[~dead], lse_ref[~dead])


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_small(case):
    B, Hq, Hkv, Nq, Nk, d, causal, window, lens, ns = case
    w = DecodeWorkload(_ids(case), B, Hq, Hkv, Nq, Nk, d, causal, window, lens, seed=81)
    q, k, v, sl = make_decode_inputs(w, "cuda")
    o, lse = fa.decode(q, k, v, sl, causal, window, w.scale, num_splits=ns)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(to64(q), to64(k), to64(v), w.lens, causal, window,
                                        w.scale)
    _check(o, lse, o_ref, lse_ref)


def test_decode_negative_scale_and_split_invariance():
    w = DecodeWorkload("negscale", 2, 8, 2, 2, 1500, 128, True, 0, (1500, 700), seed=82)
    q, k, v, sl = make_decode_inputs(w, "cuda")
    o_ref, lse_ref = oracle.attn_decode(to64(q), to64(k), to64(v), w.lens, True, 0, -0.05)
    outs = [fa.decode(q, k, v, sl, True, 0, -0.05, num_splits=ns) for ns in (1, 4, 13)]
    torch.cuda.synchronize()
    for o, lse in outs:
        _check(o, lse, o_ref, lse_ref)
    a, b = outs[0], outs[2]
    assert (a[0].float() - b[0].float()).abs().max().item() <= 2e-2
    assert (a[1] - b[1]).abs().max().item() <= 1e-4


def test_decode_unused_cache_rows_are_not_read():
    w = DecodeWorkload("unused", 2, 4, 2, 1, 600, 64, True, 0, (600, 250), seed=83)
    q, k, v, sl = make_decode_inputs(w, "cuda")
    o1, l1 = fa.decode(q, k, v, sl, num_splits=3)
    k2, v2 = k.clone(), v.clone()
    k2[1, 250:] = float("nan")
    v2[1, 250:] = float("nan")
    o2, l2 = fa.decode(q, k2, v2, sl, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_bench_workload_full():
    w = DECODE_WORKLOADS["bf16_decode_b8_hq32_hkv8_nq1_nk32768_d128"]
    q, k, v, sl = make_decode_inputs(w, "cuda")
    o, lse = fa.decode(q, k, v, sl, w.causal, w.window, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(to64(q), to64(k), to64(v), w.lens, w.causal, w.window,
                                        w.scale)
    _check(o, lse, o_ref, lse_ref)
