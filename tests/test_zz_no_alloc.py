"""fa_bwd_noalloc (the backward for callers that cannot allocate) against fa_bwd, through the
C ABI: bitwise equal gradients on two calls in a row (the second smaller, so it reuses the
static workspace the first one filled), no change in free device memory across its calls,
and sizes beyond its static workspace rejected before any launch."""

import pytest
import torch

from exact_io_aware_fa2_amd import fa
from exact_io_aware_fa2_amd.workloads import make_inputs, small_case

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, N, d, causal, window, seed):
    w = small_case("noalloc", "bf16", B, Hq, Hkv, N, d, causal, window, seed=seed)
    q, k, v, do = make_inputs(w, "cuda")
    o, lse = fa.forward(q, k, v, causal=causal, window=window, scale=w.scale)
    return w, q, k, v, do, o, lse


def _grads(fn, w, q, k, v, do, o, lse, **kw):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fn(q, k, v, o, do, lse, dq, dk, dv, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window,
            w.scale, **kw)
    assert st == fa.FA_OK, fa.fa_last_error()
    return dq, dk, dv


def test_noalloc_backward_equals_fa_bwd_on_two_calls():
    cases = [(2, 8, 2, 1000, 128, True, 0, 1), (1, 4, 4, 333, 64, False, 100, 2)]
    for B, Hq, Hkv, N, d, causal, window, seed in cases:  # the second call is smaller
        w, q, k, v, do, o, lse = _case(B, Hq, Hkv, N, d, causal, window, seed)
        ws = fa.workspace_for(B, Hq, Hkv, N, d, causal, window, q.device)
        ref = _grads(fa.fa_bwd, w, q, k, v, do, o, lse, workspace=ws,
                     workspace_bytes=ws.numel())
        got = _grads(fa.fa_bwd_noalloc, w, q, k, v, do, o, lse)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"{name} differs from fa_bwd at {tuple(q.shape)}"


def test_noalloc_backward_leaves_free_memory_unchanged():
    w, q, k, v, do, o, lse = _case(1, 8, 2, 2048, 128, True, 0, 3)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = (q, k, v, o, do, lse, dq, dk, dv, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window,
            w.scale)
    assert fa.fa_bwd_noalloc(*args) == fa.FA_OK  # warm: code objects already resident
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        assert fa.fa_bwd_noalloc(*args) == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0


def test_noalloc_backward_rejects_sizes_beyond_its_workspace():
    fake = 1 << 12
    st = fa.fa_bwd_noalloc(*([fake] * 9), 1, 64, 8, 65537, 64, 1, 0, 0.125)
    assert st == fa.FA_ERR_WORKSPACE and "static workspace" in fa.fa_last_error()
