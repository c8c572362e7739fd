"""Pins for the float64 oracle (CPU only; no GPU, no HIP library).

Every test checks the oracle against something other than itself: hand-derived
closed forms, invariants of the softmax, central finite differences, brute-force
enumeration, or an independent library routine (PyTorch's CPU float64 attention).
"""

import ast
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_probs, attention_probs_rows, attn_fwd_fp8, e4m3_decode, attn_bwd,
                    attn_bwd_dkdv_cols, attn_bwd_dkdv_cols_from_fwd, attn_bwd_dq_rows,
                    attn_bwd_head, attn_bwd_varlen, attn_fwd, attn_fwd_head, attn_fwd_rows,
                    attn_fwd_varlen, allowed_keys, attended_pairs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


# ------------------------------------------------------------------ helpers
def _eval_expr(s: str) -> float:
    """Evaluate a fixture expression: numbers, + - * /, unary minus and ln()."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            if isinstance(node.op, ast.Add):
                return a + b
            if isinstance(node.op, ast.Sub):
                return a - b
            if isinstance(node.op, ast.Mult):
                return a * b
            if isinstance(node.op, ast.Div):
                return a / b
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id == "ln" and len(node.args) == 1):
            return math.log(ev(node.args[0]))
        raise ValueError(f"unsupported expression {s!r}")
    return ev(ast.parse(s, mode="eval"))


def _arr(x):
    return np.vectorize(_eval_expr, otypes=[float])(np.array(x, dtype=object))


def _rand(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


# ------------------------------------------------------------------ golden fixtures
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_fixture(case):
    q = _arr(case["q"])[None]
    k = _arr(case["k"])[None]
    v = _arr(case["v"])[None]
    scale = _eval_expr(case["scale"])
    o, lse = attn_fwd(q, k, v, case["causal"], case["window"], scale)
    np.testing.assert_allclose(o[0], _arr(case["O"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], _arr(case["LSE"]), rtol=0, atol=1e-13)
    if "dO" in case:
        do = _arr(case["dO"])[None]
        dq, dk, dv, _ = attn_bwd(q, k, v, do, case["causal"], case["window"], scale)
        np.testing.assert_allclose(dq[0], _arr(case["dQ"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk[0], _arr(case["dK"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[0], _arr(case["dV"]), rtol=0, atol=1e-13)


# ------------------------------------------------------------------ masks
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [0, 1, 3, 7])
def test_allowed_keys_enumeration(causal, window):
    n = 11
    for i in range(n):
        lo, hi = allowed_keys(i, n, causal, window)
        brute = [j for j in range(n)
                 if (not causal or j <= i) and (window == 0 or j >= i - window + 1)]
        assert list(range(lo, hi)) == brute


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5), (False, 5), (True, 1)])
def test_attended_pairs_closed_form(causal, window):
    n = 37
    if not causal and window == 0:
        expect = n * n
    elif causal and window == 0:
        expect = n * (n + 1) // 2
    elif causal:
        w = window
        expect = w * (w + 1) // 2 + (n - w) * w
    else:
        # non-causal left bound: row i sees n - max(0, i - w + 1) keys
        expect = sum(n - max(0, i - window + 1) for i in range(n))
    assert attended_pairs(n, causal, window) == expect


# ------------------------------------------------------------------ forward pins
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 4), (False, 4)])
def test_rows_sum_to_one_and_masked_zero(causal, window):
    rng = np.random.default_rng(0)
    n, d = 23, 8
    q, k = _rand(rng, n, d, sigma=3), _rand(rng, n, d, sigma=3)
    p = attention_probs(q, k, causal, window, 0.4)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    for i in range(n):
        lo, hi = allowed_keys(i, n, causal, window)
        assert np.all(p[i, :lo] == 0) and np.all(p[i, hi:] == 0)
        assert np.all(p[i, lo:hi] > 0)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_v_ones_gives_ones(causal, window):
    rng = np.random.default_rng(1)
    b, n, h, d = 2, 19, 2, 5
    q, k = _rand(rng, b, n, h, d, sigma=4), _rand(rng, b, n, h, d, sigma=4)
    v = np.ones((b, n, h, 7))
    o, _ = attn_fwd(q, k, v, causal, window, 0.7)
    np.testing.assert_allclose(o, 1.0, atol=1e-13)


@pytest.mark.parametrize("which", ["q", "k"])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 4), (False, 4)])
def test_equal_scores_give_mean_of_v(which, causal, window):
    rng = np.random.default_rng(2)
    n, d = 17, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    if which == "q":
        q[:] = 0
    else:
        k[:] = 0
    o, lse = attn_fwd_head(q, k, v, causal, window, 1.3)
    for i in range(n):
        lo, hi = allowed_keys(i, n, causal, window)
        np.testing.assert_allclose(o[i], v[lo:hi].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[i], math.log(hi - lo), atol=1e-13)


def test_causal_row0_is_v0():
    rng = np.random.default_rng(3)
    n, d = 9, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attn_fwd_head(q, k, v, True, 0, 0.5)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * q[0] @ k[0], atol=1e-15)


def test_two_keys_sigmoid_closed_form():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 2, 1), _rand(rng, 2, 1), _rand(rng, 2, 1)
    scale = 0.9
    o, lse = attn_fwd_head(q, k, v, False, 0, scale)
    for i in range(2):
        s0, s1 = scale * q[i, 0] * k[0, 0], scale * q[i, 0] * k[1, 0]
        p0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        assert abs(o[i, 0] - (p0 * v[0, 0] + (1 - p0) * v[1, 0])) < 1e-14
        assert abs(lse[i] - math.log(math.exp(s0) + math.exp(s1))) < 1e-14


def test_large_logits_stay_finite():
    # scores of several hundred: the plain exp would overflow without the max shift
    q = np.array([[30.0, 0.0], [0.0, 30.0]])
    k = np.array([[30.0, 0.0], [29.0, 0.0], [0.0, 30.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    o, lse = attn_fwd_head(q, k, v, False, 0, 1.0)
    # row 0: s = (900, 870, 0) -> weight of key 1 relative e^-30
    e = math.exp(-30.0)
    np.testing.assert_allclose(o[0, 0], (1 + 2 * e) / (1 + e), rtol=1e-14)
    np.testing.assert_allclose(lse[0], 900 + math.log1p(e), rtol=1e-15)
    np.testing.assert_allclose(o[1, 0], 3.0, rtol=1e-14)


def test_shift_and_permutation_equivariance():
    rng = np.random.default_rng(5)
    n, d = 13, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    s = 0.8
    o, lse = attn_fwd_head(q, k, v, False, 0, s)
    c = rng.standard_normal(d)
    # v -> v + c shifts O by c (rows of P sum to one)
    o2, _ = attn_fwd_head(q, k, v + c, False, 0, s)
    np.testing.assert_allclose(o2, o + c, atol=1e-13)
    # k -> k + c adds s*q_i.c to every score of row i: O unchanged, LSE shifted
    o3, lse3 = attn_fwd_head(q, k + c, v, False, 0, s)
    np.testing.assert_allclose(o3, o, atol=1e-13)
    np.testing.assert_allclose(lse3, lse + s * q @ c, atol=1e-13)
    # permuting (k, v) jointly leaves O unchanged (non-causal)
    perm = rng.permutation(n)
    o4, lse4 = attn_fwd_head(q, k[perm], v[perm], False, 0, s)
    np.testing.assert_allclose(o4, o, atol=1e-13)
    np.testing.assert_allclose(lse4, lse, atol=1e-13)
    # permuting queries permutes O
    o5, lse5 = attn_fwd_head(q[perm], k, v, False, 0, s)
    np.testing.assert_allclose(o5, o[perm], atol=1e-13)
    np.testing.assert_allclose(lse5, lse[perm], atol=1e-13)


def test_scale_folds_into_q():
    rng = np.random.default_rng(6)
    n, d = 11, 3
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o1, l1 = attn_fwd_head(q, k, v, True, 0, 0.25)
    o2, l2 = attn_fwd_head(0.25 * q, k, v, True, 0, 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    # a negative scale is the same as negating q
    o3, l3 = attn_fwd_head(q, k, v, True, 3, -0.5)
    o4, l4 = attn_fwd_head(-q, k, v, True, 3, 0.5)
    np.testing.assert_allclose(o3, o4, atol=1e-14)
    np.testing.assert_allclose(l3, l4, atol=1e-14)


def test_window_at_least_n_equals_plain_causal():
    rng = np.random.default_rng(7)
    n, d = 15, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o1, l1 = attn_fwd_head(q, k, v, True, 0, 0.6)
    o2, l2 = attn_fwd_head(q, k, v, True, n, 0.6)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # window 1 with causal: each row sees only itself
    o3, l3 = attn_fwd_head(q, k, v, True, 1, 0.6)
    np.testing.assert_allclose(o3, v, atol=1e-15)
    np.testing.assert_allclose(l3, 0.6 * np.einsum("nd,nd->n", q, k), atol=1e-14)


def test_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng(8)
    b, n, hq, hkv, d = 2, 10, 6, 2, 3
    q = _rand(rng, b, n, hq, d)
    k, v = _rand(rng, b, n, hkv, d), _rand(rng, b, n, hkv, d)
    o, lse = attn_fwd(q, k, v, True, 0, 0.5)
    g = hq // hkv
    for h in range(hq):
        for bi in range(b):
            oh, lh = attn_fwd_head(q[bi, :, h], k[bi, :, h // g], v[bi, :, h // g], True, 0, 0.5)
            np.testing.assert_array_equal(o[bi, :, h], oh)
            np.testing.assert_array_equal(lse[bi, h], lh)


def test_row_chunking_is_exact():
    rng = np.random.default_rng(9)
    n, d = 300, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    for causal, window in [(True, 0), (True, 50), (False, 0), (False, 40)]:
        o1, l1 = attn_fwd_head(q, k, v, causal, window, 0.4, row_chunk=64)
        o2, l2 = attn_fwd_head(q, k, v, causal, window, 0.4, row_chunk=7)
        np.testing.assert_allclose(o1, o2, atol=1e-12)
        np.testing.assert_allclose(l1, l2, atol=1e-12)
        g1 = attn_bwd_head(q, k, v, do, causal, window, 0.4, row_chunk=64)
        g2 = attn_bwd_head(q, k, v, do, causal, window, 0.4, row_chunk=13)
        for a, b_ in zip(g1, g2):
            np.testing.assert_allclose(a, b_, atol=1e-12)


def test_sampled_rows_match_full():
    rng = np.random.default_rng(10)
    n, d = 200, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    rows = np.array([0, 1, 63, 64, 127, 199])
    cols = np.array([0, 5, 100, 150, 199])
    for causal, window in [(True, 0), (True, 30), (False, 0)]:
        o, l = attn_fwd_head(q, k, v, causal, window, 0.3)
        orows, lrows = attn_fwd_rows(q, k, v, rows, causal, window, 0.3)
        np.testing.assert_allclose(orows, o[rows], atol=1e-13)
        np.testing.assert_allclose(lrows, l[rows], atol=1e-13)
        dq, dk, dv, dvec = attn_bwd_head(q, k, v, do, causal, window, 0.3)
        dqr, dr = attn_bwd_dq_rows(q, k, v, do, rows, causal, window, 0.3)
        np.testing.assert_allclose(dqr, dq[rows], atol=1e-13)
        np.testing.assert_allclose(dr, dvec[rows], atol=1e-13)
        dkc, dvc = attn_bwd_dkdv_cols(q, k, v, do, cols, causal, window, 0.3, row_chunk=37)
        np.testing.assert_allclose(dkc, dk[cols], atol=1e-12)
        np.testing.assert_allclose(dvc, dv[cols], atol=1e-12)


@pytest.mark.parametrize("causal,window,slope", [(True, 0, 0.0), (True, 30, 0.0), (False, 0, 0.0),
                                                 (False, 25, 0.0), (True, 0, 0.2),
                                                 (False, 0, -0.1)])
def test_dkdv_columns_from_forward_match_full_backward(causal, window, slope):
    """dK/dV at selected keys from the forward's O and LSE equal the columns of the full
    analytic backward (itself pinned by finite differences and torch's autograd), for every
    mask, with a position bias, large logits, and row chunks that split the rows unevenly."""
    rng = np.random.default_rng(31)
    n, d = 230, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    q = 3.0 * q  # large logits: nearly one-hot rows
    cols = np.array([0, 1, 31, 32, 100, 150, 228, 229])
    o, lse = attn_fwd_head(q, k, v, causal, window, 0.3, slope=slope)
    _, dk, dv, _ = attn_bwd_head(q, k, v, do, causal, window, 0.3, slope=slope)
    dkc, dvc = attn_bwd_dkdv_cols_from_fwd(q, k, v, do, o, lse, cols, causal, window, 0.3,
                                           row_chunk=41, slope=slope)
    np.testing.assert_allclose(dkc, dk[cols], atol=1e-11, rtol=1e-10)
    np.testing.assert_allclose(dvc, dv[cols], atol=1e-11, rtol=1e-10)
    # a plausible slip (D taken from the wrong row, or P without its normaliser) is caught
    dk_bad, _ = attn_bwd_dkdv_cols_from_fwd(q, k, v, do, np.roll(o, 1, axis=0), lse, cols,
                                            causal, window, 0.3, slope=slope)
    assert np.abs(dk_bad - dk[cols]).max() > 1e-3
    _, dv_bad = attn_bwd_dkdv_cols_from_fwd(q, k, v, do, o, lse - 0.1, cols, causal, window,
                                            0.3, slope=slope)
    assert np.abs(dv_bad - dv[cols]).max() > 1e-3


# ------------------------------------------------------------------ backward pins
def _loss(q, k, v, do, causal, window, scale):
    o, _ = attn_fwd(q, k, v, causal, window, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 2), (False, 2)])
def test_finite_differences(causal, window):
    rng = np.random.default_rng(11)
    b, n, hq, hkv, d = 1, 5, 2, 1, 3
    q = _rand(rng, b, n, hq, d)
    k = _rand(rng, b, n, hkv, d)
    v = _rand(rng, b, n, hkv, d)
    do = _rand(rng, b, n, hq, d)
    scale = 0.7
    dq, dk, dv, _ = attn_bwd(q, k, v, do, causal, window, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, causal, window, scale)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, causal, window, scale)
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 6)])
def test_backward_invariants(causal, window):
    rng = np.random.default_rng(12)
    b, n, hq, hkv, d = 1, 29, 4, 2, 5
    q, do = _rand(rng, b, n, hq, d), _rand(rng, b, n, hq, d)
    k, v = _rand(rng, b, n, hkv, d), _rand(rng, b, n, hkv, d)
    scale = 0.45
    o, _ = attn_fwd(q, k, v, causal, window, scale)
    dq, dk, dv, dvec = attn_bwd(q, k, v, do, causal, window, scale)
    g = hq // hkv
    # D_i equals dO_i . O_i (rows of P sum to one)
    np.testing.assert_allclose(dvec, np.einsum("bnhd,bnhd->bhn", do, o), atol=1e-12)
    # sum_j dK_j = 0 (invariance of softmax to a per-row shift of K)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # sum_j dV_j = sum over the group's query heads of sum_i dO_i
    for hk in range(hkv):
        expect = do[:, :, hk * g:(hk + 1) * g].sum(axis=(1, 2))
        np.testing.assert_allclose(dv[:, :, hk].sum(axis=1), expect, atol=1e-12)
    # rows of dS sum to zero: checked through sum_j dS_ij k_j with k = const
    kc = np.ones_like(k)
    dq_c, _, _, _ = attn_bwd(q, kc, v, do, causal, window, scale)
    np.testing.assert_allclose(dq_c, 0.0, atol=1e-12)


# ------------------------------------------------------------------ independent library
@pytest.mark.parametrize("causal,window,hq,hkv", [(False, 0, 4, 4), (True, 0, 4, 2), (True, 16, 4, 1),
                                                  (False, 16, 2, 2)])
def test_matches_torch_sdpa_cpu_float64(causal, window, hq, hkv):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(13)
    b, n, d = 2, 70, 16
    q = _rand(rng, b, n, hq, d, sigma=2)
    k = _rand(rng, b, n, hkv, d, sigma=2)
    v = _rand(rng, b, n, hkv, d)
    do = _rand(rng, b, n, hq, d)
    scale = 1 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, causal, window, scale)
    dq, dk, dv, _ = attn_bwd(q, k, v, do, causal, window, scale)

    tq = torch.tensor(q).transpose(1, 2).requires_grad_()
    tk = torch.tensor(k).transpose(1, 2).requires_grad_()
    tv = torch.tensor(v).transpose(1, 2).requires_grad_()
    g = hq // hkv
    ke = tk.repeat_interleave(g, dim=1)
    ve = tv.repeat_interleave(g, dim=1)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    mask = torch.ones(n, n, dtype=torch.bool)
    if causal:
        mask &= j <= i
    if window:
        mask &= j >= i - window + 1
    to = F.scaled_dot_product_attention(tq, ke, ve, attn_mask=mask, scale=scale)
    to.backward(torch.tensor(do).transpose(1, 2))
    np.testing.assert_allclose(o, to.detach().transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    # LSE against torch.logsumexp of the masked score matrix
    s = torch.einsum("bhnd,bhmd->bhnm", tq.detach(), ke.detach()) * scale
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_process_pool_matches_serial():
    rng = np.random.default_rng(14)
    b, n, hq, hkv, d = 1, 40, 4, 2, 8
    q, do = _rand(rng, b, n, hq, d), _rand(rng, b, n, hq, d)
    k, v = _rand(rng, b, n, hkv, d), _rand(rng, b, n, hkv, d)
    o1, l1 = attn_fwd(q, k, v, True, 0, 0.3)
    o2, l2 = attn_fwd(q, k, v, True, 0, 0.3, workers=2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    g1 = attn_bwd(q, k, v, do, True, 0, 0.3)
    g2 = attn_bwd(q, k, v, do, True, 0, 0.3, workers=2)
    for a, b_ in zip(g1, g2):
        np.testing.assert_allclose(a, b_, atol=1e-14)


# ------------------------------------------------------------------ packed sequences
VARLEN_LENS = [5, 0, 1, 17, 9]


def _packed(rng, lens, hq, hkv, d):
    t = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    do = rng.standard_normal((t, hq, d))
    return cu, q, k, v, do


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3), (False, 4)])
def test_varlen_matches_torch_block_diagonal_mask(causal, window):
    """Packed sequences = one attention over all rows with a block-diagonal mask (masks
    counted inside each block), evaluated by torch's float64 SDPA and autograd."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(21)
    hq, hkv, d = 4, 2, 8
    cu, q, k, v, do = _packed(rng, VARLEN_LENS, hq, hkv, d)
    scale = 0.4
    o, lse = attn_fwd_varlen(q, k, v, cu, causal, window, scale)
    dq, dk, dv, dvec = attn_bwd_varlen(q, k, v, do, cu, causal, window, scale)
    t = q.shape[0]
    seq = np.repeat(np.arange(len(VARLEN_LENS)), VARLEN_LENS)
    pos = np.arange(t) - cu[seq]
    same = seq[:, None] == seq[None, :]
    i, j = pos[:, None], pos[None, :]
    ok = same.copy()
    if causal:
        ok &= j <= i
    if window:
        ok &= j >= i - window + 1
    mask = torch.tensor(ok)
    g = hq // hkv
    tq = torch.tensor(q).transpose(0, 1)[None].requires_grad_()
    tk = torch.tensor(k).transpose(0, 1)[None].requires_grad_()
    tv = torch.tensor(v).transpose(0, 1)[None].requires_grad_()
    to = F.scaled_dot_product_attention(tq, tk.repeat_interleave(g, dim=1),
                                        tv.repeat_interleave(g, dim=1), attn_mask=mask,
                                        scale=scale)
    to.backward(torch.tensor(do).transpose(0, 1)[None])
    np.testing.assert_allclose(o, to.detach()[0].transpose(0, 1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad[0].transpose(0, 1).numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad[0].transpose(0, 1).numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad[0].transpose(0, 1).numpy(), atol=1e-11)
    s_ = torch.einsum("hnd,hmd->hnm", torch.tensor(q).transpose(0, 1),
                      torch.tensor(k).transpose(0, 1).repeat_interleave(g, dim=0)) * scale
    s_ = s_.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s_, dim=-1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dvec, np.einsum("thd,thd->ht", do, o), atol=1e-12)


def test_varlen_equal_lengths_equal_a_batch():
    rng = np.random.default_rng(22)
    n, nb, hq, hkv, d = 13, 3, 2, 1, 4
    cu, q, k, v, do = _packed(rng, [n] * nb, hq, hkv, d)
    o, lse = attn_fwd_varlen(q, k, v, cu, True, 5, 0.6)
    ob, lseb = attn_fwd(q.reshape(nb, n, hq, d), k.reshape(nb, n, hkv, d),
                        v.reshape(nb, n, hkv, d), True, 5, 0.6)
    np.testing.assert_array_equal(o, ob.reshape(nb * n, hq, d))
    np.testing.assert_array_equal(lse, lseb.transpose(1, 0, 2).reshape(hq, nb * n))
    g = attn_bwd_varlen(q, k, v, do, cu, True, 5, 0.6)
    gb = attn_bwd(q.reshape(nb, n, hq, d), k.reshape(nb, n, hkv, d), v.reshape(nb, n, hkv, d),
                  do.reshape(nb, n, hq, d), True, 5, 0.6)
    for a, bt in zip(g[:3], gb[:3]):
        np.testing.assert_array_equal(a, bt.reshape(a.shape))


def test_varlen_sequences_are_independent():
    rng = np.random.default_rng(23)
    cu, q, k, v, do = _packed(rng, [6, 7], 2, 2, 4)
    o1, l1 = attn_fwd_varlen(q, k, v, cu, False, 0, 0.5)
    k2 = k.copy()
    k2[:6] += rng.standard_normal(k2[:6].shape)  # change only the first sequence's keys
    o2, l2 = attn_fwd_varlen(q, k2, v, cu, False, 0, 0.5)
    np.testing.assert_array_equal(o1[6:], o2[6:])
    np.testing.assert_array_equal(l1[:, 6:], l2[:, 6:])
    assert np.abs(o1[:6] - o2[:6]).max() > 1e-6


def test_varlen_rejects_bad_offsets():
    rng = np.random.default_rng(24)
    cu, q, k, v, _ = _packed(rng, [3, 4], 1, 1, 2)
    for bad in ([1, 3, 7], [0, 5, 4], [0, 3, 6]):
        with pytest.raises(ValueError):
            attn_fwd_varlen(q, k, v, bad)


# ------------------------------------------------------------------ 8-bit inputs
def test_attention_probs_rows_match_full_matrix():
    rng = np.random.default_rng(40)
    q, k = rng.standard_normal((37, 8)), rng.standard_normal((37, 8))
    rows = np.array([0, 5, 36, 17])
    for causal, window in [(False, 0), (True, 0), (True, 6), (False, 9)]:
        full = attention_probs(q, k, causal, window, 0.3)
        np.testing.assert_array_equal(attention_probs_rows(q, k, rows, causal, window, 0.3),
                                      full[rows])


def test_e4m3_decode_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert np.isnan(ours).sum() == 2  # 0x7F and 0xFF only


def test_e4m3_decode_closed_forms():
    # bias 7, 3 mantissa bits, subnormals below 2^-6, no infinities
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x78: 256.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, val in cases.items():
        assert e4m3_decode(np.array([c], np.uint8))[0] == val, hex(c)
    assert np.signbit(e4m3_decode(np.array([0x80], np.uint8))[0])


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5)])
def test_attn_fwd_fp8_is_attention_of_dequantized_inputs(causal, window):
    """Against torch's float8 decode and float64 SDPA (an independent path)."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(41)
    b, n, hq, hkv, d = 2, 19, 4, 2, 16
    codes = [rng.integers(0, 256, size=(b, n, h, d), dtype=np.uint8) for h in (hq, hkv, hkv)]
    codes = [np.where((c & 0x7F) == 0x7F, 0x3A, c).astype(np.uint8) for c in codes]  # no NaN
    f = (0.02, 0.011, 0.5)
    o, lse = attn_fwd_fp8(*codes, *f, causal, window, 0.25)
    t = [torch.tensor(c).view(torch.float8_e4m3fn).double() * fi for c, fi in zip(codes, f)]
    g = hq // hkv
    tq = t[0].transpose(1, 2)
    tk = t[1].transpose(1, 2).repeat_interleave(g, dim=1)
    tv = t[2].transpose(1, 2).repeat_interleave(g, dim=1)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    ok = torch.ones(n, n, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window:
        ok &= j >= i - window + 1
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=ok, scale=0.25)
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), rtol=1e-12, atol=1e-12)
    s = (tq @ tk.transpose(-1, -2) * 0.25).masked_fill(~ok, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("offset", [0.0, 1.3, 3.0])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 7)])
@pytest.mark.parametrize("delta", [0.0, 0.01])
def test_fp8_error_bound_holds_for_e4m3_rounded_weights(offset, causal, window, delta):
    """The per-element bound the fp8 GPU tests use, checked against weights rounded to E4M3
    by torch (round to nearest even) at a reference `offset` log2 units below the row max,
    normalised by the unrounded sum, with scores perturbed by up to `delta`."""
    torch = pytest.importorskip("torch")
    from tests._parity import fp8_o_bound
    rng = np.random.default_rng(42)
    n, d = 300, 32
    q = rng.standard_normal((n, d)) * 2.0
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    p = attention_probs(q, k, causal, window, 0.3)
    o_ref = p @ v
    # scores perturbed by up to +-delta (the worst direction pattern of a +-1 draw)
    pert = np.exp(delta * rng.choice([-1.0, 1.0], size=p.shape))
    w = p * pert / (p * pert).max(axis=1, keepdims=True) * 2.0 ** offset
    wr = torch.tensor(w).float().to(torch.float8_e4m3fn).double().numpy()
    o_emul = (wr @ v) / w.sum(axis=1, keepdims=True)
    bound = fp8_o_bound(p, v, o_ref, delta)
    err = np.abs(o_emul - o_ref)
    assert (err <= bound).all(), float((err / bound).max())
    assert (err / bound).max() > 0.02  # the bound is not vacuous for this data


def test_quantize_e4m3_roundtrip():
    torch = pytest.importorskip("torch")
    from exact_io_aware_fa2_amd.workloads import quantize_e4m3
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4000, generator=g) * 3.0
    codes, f = quantize_e4m3(x)
    y = e4m3_decode(codes.numpy()) * f
    assert np.abs(y).max() == pytest.approx(float(x.abs().max()), rel=2 ** -4)
    xs = x.double().numpy()
    normal = np.abs(xs) >= 2.0 ** -6 * f
    assert (np.abs(y - xs)[normal] <= 2.0 ** -4 * np.abs(xs)[normal] * (1 + 1e-6)).all()
    assert (np.abs(y - xs)[~normal] <= 2.0 ** -10 * f * (1 + 1e-6)).all()


def test_fp8_score_error_dominates_brute_force_terms():
    # Delta_i >= (d/64) 2 * 2^-9 |scale| max_j max_c 2^(e(q_ic) + e(k_jc)) fq fk + 2^-22 max_j
    # |s_ij|, with the exponents taken from the codes themselves (subnormal codes at -6)
    from tests._parity import fp8_score_error
    torch = pytest.importorskip("torch")
    from exact_io_aware_fa2_amd.workloads import quantize_e4m3
    g = torch.Generator().manual_seed(43)
    xq = torch.randn(50, 128, generator=g) * 3
    xk = torch.randn(70, 128, generator=g)
    xq[:, :5] *= 1e-4  # subnormal codes
    (cq, fq), (ck, fk) = quantize_e4m3(xq), quantize_e4m3(xk)
    cq, ck = cq.numpy(), ck.numpy()
    q, k = e4m3_decode(cq) * fq, e4m3_decode(ck) * fk
    assert ((cq & 0x78) == 0).any() and (q != 0).any()  # some subnormal codes present
    got = fp8_score_error(q, k, -0.2, fq, fk)
    eq = np.exp2(np.maximum((cq.astype(np.int64) >> 3) & 0xF, 1) - 7.0) * fq
    ek = np.exp2(np.maximum((ck.astype(np.int64) >> 3) & 0xF, 1) - 7.0) * fk
    align = (eq[:, None, :] * ek[None, :, :]).max(axis=2).max(axis=1)
    smax = np.abs(q @ k.T * 0.2).max(axis=1)
    need = (128 / 64) * 2 * 2.0 ** -9 * 0.2 * align + 2.0 ** -22 * smax
    assert (got >= need * (1 - 1e-12)).all()


# ------------------------------------------------------------------ ALiBi position bias
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 6), (False, 5)])
def test_alibi_matches_torch_float_bias_and_autograd(causal, window):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(50)
    b, n, hq, hkv, d = 2, 23, 4, 2, 8
    q, k, v, do = (rng.standard_normal((b, n, h, d)) for h in (hq, hkv, hkv, hq))
    slopes = np.array([0.5, 0.125, -0.05, 0.0])
    o, lse = attn_fwd(q, k, v, causal, window, 0.3, alibi_slopes=slopes)
    dq, dk, dv, _ = attn_bwd(q, k, v, do, causal, window, 0.3, alibi_slopes=slopes)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    ok = torch.ones(n, n, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window:
        ok &= j >= i - window + 1
    bias = -torch.tensor(slopes)[:, None, None] * (i - j).abs().double()  # [hq, n, n]
    bias = bias.masked_fill(~ok, float("-inf"))[None]
    g = hq // hkv
    tq = torch.tensor(q).transpose(1, 2).requires_grad_()
    tk = torch.tensor(k).transpose(1, 2).requires_grad_()
    tv = torch.tensor(v).transpose(1, 2).requires_grad_()
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(g, dim=1),
                                         tv.repeat_interleave(g, dim=1), attn_mask=bias, scale=0.3)
    out.backward(torch.tensor(do).transpose(1, 2))
    np.testing.assert_allclose(o, out.detach().transpose(1, 2).numpy(), atol=1e-12)
    s = tq.detach() @ tk.detach().repeat_interleave(g, dim=1).transpose(-1, -2) * 0.3 + bias
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.transpose(1, 2).numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.transpose(1, 2).numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.transpose(1, 2).numpy(), atol=1e-11)


def test_alibi_zero_queries_closed_form():
    """Q = 0 leaves only the bias: causal row i weighs key i - t by e^(-m t), so
    LSE_i = ln((1 - e^(-m (i+1))) / (1 - e^(-m))) and O_i is that geometric average of V."""
    rng = np.random.default_rng(51)
    n, d, m = 40, 4, 0.3
    q = np.zeros((1, n, 1, d))
    k = rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    o, lse = attn_fwd(q, k, v, True, 0, 0.7, alibi_slopes=[m])
    i = np.arange(n)
    np.testing.assert_allclose(lse[0, 0], np.log((1 - np.exp(-m * (i + 1))) / (1 - np.exp(-m))),
                               rtol=1e-13)
    for r in (0, 1, 17, n - 1):
        w = np.exp(-m * (r - np.arange(r + 1)))
        np.testing.assert_allclose(o[0, r, 0], w @ v[0, :r + 1, 0] / w.sum(), rtol=1e-12)


def test_alibi_gradients_match_finite_differences():
    rng = np.random.default_rng(52)
    b, n, h, d = 1, 7, 2, 3
    q, k, v, do = (rng.standard_normal((b, n, h, d)) for _ in range(4))
    slopes = [0.4, 0.9]
    dq, dk, dv, _ = attn_bwd(q, k, v, do, True, 4, 0.5, alibi_slopes=slopes)

    def loss(qq, kk, vv):
        return float((attn_fwd(qq, kk, vv, True, 4, 0.5, alibi_slopes=slopes)[0] * do).sum())

    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_alibi_packed_positions_start_at_each_sequence():
    rng = np.random.default_rng(53)
    n, nb, hq, d = 11, 3, 2, 4
    cu, q, k, v, do = _packed(rng, [n] * nb, hq, hq, d)
    sl = [0.3, 0.05]
    o, lse = attn_fwd_varlen(q, k, v, cu, True, 0, 0.5, alibi_slopes=sl)
    ob, lseb = attn_fwd(q.reshape(nb, n, hq, d), k.reshape(nb, n, hq, d), v.reshape(nb, n, hq, d),
                        True, 0, 0.5, alibi_slopes=sl)
    np.testing.assert_array_equal(o, ob.reshape(nb * n, hq, d))
    g = attn_bwd_varlen(q, k, v, do, cu, True, 0, 0.5, alibi_slopes=sl)
    gb = attn_bwd(q.reshape(nb, n, hq, d), k.reshape(nb, n, hq, d), v.reshape(nb, n, hq, d),
                  do.reshape(nb, n, hq, d), True, 0, 0.5, alibi_slopes=sl)
    for a, bt in zip(g[:3], gb[:3]):
        np.testing.assert_array_equal(a, bt.reshape(a.shape))


# ------------------------------------------------------------------ decoding over a cache
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 5), (False, 0), (False, 7)])
def test_decode_equals_last_rows_of_full_attention(causal, window):
    """Decoding the last Nq queries against the whole sequence's keys is the last Nq rows
    of ordinary attention over that sequence (the batched oracle)."""
    from oracle import attn_decode
    rng = np.random.default_rng(60)
    b, n, nq, hq, hkv, d = 2, 29, 3, 4, 2, 8
    q, k, v = (rng.standard_normal((b, n, h, d)) for h in (hq, hkv, hkv))
    o_full, lse_full = attn_fwd(q, k, v, causal, window, 0.4)
    o, lse = attn_decode(q[:, n - nq:], k, v, None, causal, window, 0.4)
    np.testing.assert_allclose(o, o_full[:, n - nq:], atol=1e-13)
    np.testing.assert_allclose(lse, lse_full[:, :, n - nq:], atol=1e-13)


def test_decode_per_sequence_lengths_and_unused_cache_rows():
    from oracle import attn_decode
    rng = np.random.default_rng(61)
    b, nk, nq, hq, hkv, d = 3, 20, 2, 2, 1, 4
    q = rng.standard_normal((b, nq, hq, d))
    k, v = rng.standard_normal((b, nk, hkv, d)), rng.standard_normal((b, nk, hkv, d))
    lens = [20, 7, 1]
    o, lse = attn_decode(q, k, v, lens, True, 0, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[1, 7:] = 1e3  # rows past a sequence's length are never read
    v2[1, 7:] = np.nan
    o2, lse2 = attn_decode(q, k2, v2, lens, True, 0, 0.5)
    np.testing.assert_array_equal(o, o2)
    for bi, n in enumerate(lens):
        o_full, lse_full = attn_fwd(np.concatenate([np.zeros((1, n - nq, hq, d)) if n >= nq else
                                                    np.zeros((1, 0, hq, d)),
                                                    q[bi:bi + 1, max(0, nq - n):]], axis=1),
                                    k[bi:bi + 1, :n], v[bi:bi + 1, :n], True, 0, 0.5)
        if n >= nq:
            np.testing.assert_allclose(o[bi], o_full[0, n - nq:], atol=1e-13)
    # sequence 2 has one key and two queries: query 0 sits at position -1 and sees nothing
    assert np.all(o[2, 0] == 0) and np.all(np.isneginf(lse[2, :, 0]))
    np.testing.assert_allclose(o[2, 1], np.repeat(v[2, 0], hq // hkv, axis=0), atol=1e-15)


def test_decode_matches_torch_sdpa_with_explicit_mask():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    from oracle import attn_decode
    rng = np.random.default_rng(62)
    b, nk, nq, hq, hkv, d = 1, 40, 4, 4, 2, 8
    q = rng.standard_normal((b, nq, hq, d))
    k, v = rng.standard_normal((b, nk, hkv, d)), rng.standard_normal((b, nk, hkv, d))
    o, lse = attn_decode(q, k, v, [33], True, 9, 0.3)
    pos = torch.arange(33 - nq, 33)[:, None]
    j = torch.arange(33)[None, :]
    ok = (j <= pos) & (j >= pos - 8)
    tq = torch.tensor(q).transpose(1, 2)
    tk = torch.tensor(k[:, :33]).transpose(1, 2).repeat_interleave(2, dim=1)
    tv = torch.tensor(v[:, :33]).transpose(1, 2).repeat_interleave(2, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=ok, scale=0.3)
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), atol=1e-13)
    s = (tq @ tk.transpose(-1, -2) * 0.3).masked_fill(~ok, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-13)
