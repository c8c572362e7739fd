"""Plain float64 attention: forward, analytic backward, and sampled variants.

Test infrastructure only (see the package docstring): the tests, the smoke check
and the CPU-baseline leg of the bench may call it; the product path may not.

Notation follows the pages: Q, K, V with rows = sequence positions, head dim d,
scores S = scale * Q K^T, P = softmax(S) row by row, O = P V.  Shapes of the
full-tensor entry points are (batch, seqlen, nheads, headdim), the layout given in
the usage example of bmjup.com "FlashAttention-2 ... 实战解析", section 4.
Query head ``hq`` reads KV head ``hq // (Hq // Hkv)`` (grouped-query attention,
hysenlabs.com "dao-ailab flash-attention", hardware-boundary section; consecutive
groups of query heads share one KV head).

Masking (bmjup.com, section 2.3 and section 3.3):
* causal: query i sees keys j <= i;
* sliding window W > 0: query i sees keys j >= i - W + 1 (W keys ending at the
  diagonal when causal); W = 0 means no window;
* a masked entry has probability 0, i.e. score -inf before the softmax.  It never
  enters the normaliser.

Position bias (bmjup.com, FAQ on inference: the ``alibi_slopes`` argument, no bias when
it is None; hysenlabs.com, hardware-boundary section: ALiBi): with a slope m_h per query
head, score_ij = scale * q_i . k_j - m_h * |i - j|, positions counted from the start of the
sequence, added before the mask and the softmax.  The slopes are constants (no gradient);
slope 0 is plain attention.

All arithmetic is float64.  Rows are processed in chunks to bound memory; each row's
softmax always spans its whole allowed key set, so chunking over rows is exact (no
chunking over keys, no running rescale).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

DEFAULT_ROW_CHUNK = 1024


# --------------------------------------------------------------------------- masks
def allowed_keys(i: int, n_keys: int, causal: bool, window: int) -> tuple[int, int]:
    """Half-open key range [lo, hi) that query row ``i`` may attend.

    causal keeps j <= i; window W > 0 keeps j >= i - W + 1 (bmjup.com, section 2.3
    and section 3.3).  An empty range (lo >= hi) means the row attends nothing.
    """
    hi = min(i + 1, n_keys) if causal else n_keys
    lo = max(0, i - window + 1) if window > 0 else 0
    return lo, hi


def _mask(rows: np.ndarray, cols: np.ndarray, causal: bool, window: int) -> np.ndarray:
    """Boolean matrix: True where query rows[a] may attend key cols[b]."""
    i = rows[:, None]
    j = cols[None, :]
    ok = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= j >= i - window + 1
    return ok


def _key_span(rows: np.ndarray, n_keys: int, causal: bool, window: int) -> tuple[int, int]:
    """Smallest key range holding every key any of ``rows`` may attend."""
    lo = max(0, int(rows.min()) - window + 1) if window > 0 else 0
    hi = min(int(rows.max()) + 1, n_keys) if causal else n_keys
    return lo, max(lo, hi)


# ------------------------------------------------------------------ row-level core
def _probs_rows(q, k, rows, causal, window, scale, slope=0.0):
    """Softmax rows of S = scale * Q K^T for the query ``rows``.

    Returns (P, LSE, lo, hi): P covers keys [lo, hi) (zero where masked), LSE is the
    natural-log normaliser  LSE_i = m_i + ln sum_j exp(s_ij - m_i),  m_i = max_j s_ij
    over the allowed set.  A row with no allowed key gets P = 0 and LSE = -inf.
    """
    n_keys = k.shape[0]
    lo, hi = _key_span(rows, n_keys, causal, window)
    cols = np.arange(lo, hi)
    s = scale * (q[rows] @ k[lo:hi].T)
    if slope:
        s = s - slope * np.abs(rows[:, None] - cols[None, :]).astype(np.float64)
    ok = _mask(rows, cols, causal, window)
    s = np.where(ok, s, -np.inf)
    if s.shape[1] == 0:
        m = np.full(rows.size, -np.inf)
    else:
        m = s.max(axis=1)
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    e = np.exp(s - m0[:, None])  # exp(-inf) = 0 for masked entries
    denom = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(finite, m0 + np.log(np.where(finite, denom, 1.0)), -np.inf)
        p = np.where(finite[:, None], e / np.where(finite, denom, 1.0)[:, None], 0.0)
    return p, lse, lo, hi


def _as64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _chunks(n: int, r: int):
    for r0 in range(0, n, r):
        yield np.arange(r0, min(n, r0 + r))


# ------------------------------------------------------------------ one head
def attention_probs(q, k, causal=False, window=0, scale=None, slope=0.0) -> np.ndarray:
    """The full N x N probability matrix P of one head (small N only)."""
    q = _as64(q)
    k = _as64(k)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    rows = np.arange(q.shape[0])
    p, _, lo, hi = _probs_rows(q, k, rows, causal, window, scale, slope)
    full = np.zeros((q.shape[0], k.shape[0]))
    full[:, lo:hi] = p
    return full


def attention_probs_rows(q, k, rows, causal=False, window=0, scale=None,
                         slope=0.0) -> np.ndarray:
    """Rows ``rows`` of the probability matrix P of one head, full width [len(rows), Nk]."""
    q = _as64(q)
    k = _as64(k)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, k.shape[0]))
    for a in range(0, rows.size, 64):
        rr = rows[a:a + 64]
        p, _, lo, hi = _probs_rows(q, k, rr, causal, window, scale, slope)
        out[a:a + 64, lo:hi] = p
    return out


def attn_fwd_rows(q, k, v, rows, causal=False, window=0, scale=None, slope=0.0):
    """O and LSE of one head for the selected query ``rows`` only.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv] of one (batch, query head) pair.
    Returns (O[rows] as [len(rows), dv], LSE[rows]).  Each requested row is the full
    definition; rows are processed in small groups so any subset is cheap.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.zeros(rows.size)
    for a in range(0, rows.size, 64):
        rr = rows[a:a + 64]
        p, l, lo, hi = _probs_rows(q, k, rr, causal, window, scale, slope)
        o[a:a + 64] = p @ v[lo:hi]
        lse[a:a + 64] = l
    return o, lse


def attn_fwd_head(q, k, v, causal=False, window=0, scale=None, row_chunk=DEFAULT_ROW_CHUNK,
                  slope=0.0):
    """Forward of one head: O = softmax(scale * Q K^T (masked)) V and its LSE.

    (ainews.cool "flash-attention transformer optimization", technical deep dive:
    Softmax(QK^T/sqrt(d))V, with the 1/sqrt(d) factor passed as ``scale``.)
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for rows in _chunks(n, row_chunk):
        p, l, lo, hi = _probs_rows(q, k, rows, causal, window, scale, slope)
        o[rows] = p @ v[lo:hi]
        lse[rows] = l
    return o, lse


def _bwd_rows(q, k, v, do, rows, causal, window, scale, slope=0.0):
    """Backward quantities for ``rows`` of one head.

    With L = sum(O * dO) (the upstream gradient dO), the chain rule through the
    row softmax gives, for each row i over its allowed keys:
        dP_ij = dO_i . v_j
        D_i   = sum_j P_ij dP_ij             (the Jacobian-vector product term)
        dS_ij = P_ij (dP_ij - D_i)
        dQ_i  = scale * sum_j dS_ij k_j
        dK_j += scale * dS_ij q_i ,  dV_j += P_ij dO_i
    Returns (P, dS, D, lo, hi) for the caller to contract.
    """
    p, _, lo, hi = _probs_rows(q, k, rows, causal, window, scale, slope)
    dp = do[rows] @ v[lo:hi].T
    dvec = (p * dp).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    return p, ds, dvec, lo, hi


def attn_bwd_head(q, k, v, do, causal=False, window=0, scale=None, row_chunk=DEFAULT_ROW_CHUNK,
                  slope=0.0):
    """Gradients of L = sum(O * dO) for one head: (dQ, dK, dV, D).

    The pages state only that the backward rebuilds the attention matrix from Q, K
    and V instead of storing it (ainews.cool "flash-attention transformer
    optimization", technical deep dive, item 2); this is the analytic derivative.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros(n)
    for rows in _chunks(n, row_chunk):
        p, ds, d_r, lo, hi = _bwd_rows(q, k, v, do, rows, causal, window, scale, slope)
        dq[rows] = scale * (ds @ k[lo:hi])
        dk[lo:hi] += scale * (ds.T @ q[rows])
        dv[lo:hi] += p.T @ do[rows]
        dvec[rows] = d_r
    return dq, dk, dv, dvec


def attn_bwd_dq_rows(q, k, v, do, rows, causal=False, window=0, scale=None, slope=0.0):
    """dQ (and D) of one head for the selected query ``rows`` only (row-local)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, q.shape[1]))
    dvec = np.zeros(rows.size)
    for a in range(0, rows.size, 64):
        rr = rows[a:a + 64]
        _, ds, d_r, lo, hi = _bwd_rows(q, k, v, do, rr, causal, window, scale, slope)
        dq[a:a + 64] = scale * (ds @ k[lo:hi])
        dvec[a:a + 64] = d_r
    return dq, dvec


def attn_bwd_dkdv_cols(q, k, v, do, cols, causal=False, window=0, scale=None,
                       row_chunk=DEFAULT_ROW_CHUNK, slope=0.0):
    """This query head's contribution to dK and dV at the selected key ``cols``.

    Only query rows that can attend some selected key are visited (causal: rows
    >= min(cols); window W: rows <= max(cols) + W - 1); each visited row still uses
    its full softmax row.  Sum the result over the query heads of a KV group to get
    that group's dK/dV.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    n = q.shape[0]
    r0 = int(cols.min()) if causal else 0
    r1 = min(n, int(cols.max()) + window) if window > 0 else n
    dk = np.zeros((cols.size, k.shape[1]))
    dv = np.zeros((cols.size, v.shape[1]))
    for a in range(r0, r1, row_chunk):
        rows = np.arange(a, min(r1, a + row_chunk))
        p, ds, _, lo, hi = _bwd_rows(q, k, v, do, rows, causal, window, scale, slope)
        sel = cols - lo
        inside = (sel >= 0) & (sel < hi - lo)
        if not inside.any():
            continue
        idx = np.where(inside)[0]
        dk[idx] += scale * (ds[:, sel[idx]].T @ q[rows])
        dv[idx] += p[:, sel[idx]].T @ do[rows]
    return dk, dv


def attn_bwd_dkdv_cols_from_fwd(q, k, v, do, o, lse, cols, causal=False, window=0, scale=None,
                                row_chunk=DEFAULT_ROW_CHUNK, slope=0.0):
    """Like ``attn_bwd_dkdv_cols``, but from this head's forward outputs O and LSE (of this
    same oracle) instead of whole softmax rows.

    The probability of an allowed pair is P_ij = exp(s_ij - LSE_i) (LSE_i is the row's
    natural-log normaliser, so this is the softmax itself), and D_i = sum_c dO_ic O_ic equals
    sum_j P_ij dP_ij; with them only the selected key columns are needed (ainews.cool
    "flash-attention transformer optimization", technical deep dive, item 2: the matrix is
    rebuilt from what the forward kept).  Cost is linear in the number of rows, so the heavy
    key blocks of very long sequences can be checked.  q [N, d], k/v [Nk, d], do/o [N, dv],
    lse [N]; returns this query head's dK, dV at ``cols``.
    """
    q, k, v, do, o = _as64(q), _as64(k), _as64(v), _as64(do), _as64(o)
    lse = _as64(lse)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    n = q.shape[0]
    r0 = int(cols.min()) if causal else 0
    r1 = min(n, int(cols.max()) + window) if window > 0 else n
    dk = np.zeros((cols.size, k.shape[1]))
    dv = np.zeros((cols.size, v.shape[1]))
    kc, vc = k[cols], v[cols]
    for a in range(r0, r1, row_chunk):
        rows = np.arange(a, min(r1, a + row_chunk))
        s = scale * (q[rows] @ kc.T)
        if slope:
            s = s - slope * np.abs(rows[:, None] - cols[None, :]).astype(np.float64)
        ok = _mask(rows, cols, causal, window) & np.isfinite(lse[rows])[:, None]
        p = np.where(ok, np.exp(np.where(ok, s - lse[rows][:, None], 0.0)), 0.0)
        dp = do[rows] @ vc.T
        dvec = (do[rows] * o[rows]).sum(axis=1)
        ds = p * (dp - dvec[:, None])
        dk += scale * (ds.T @ q[rows])
        dv += p.T @ do[rows]
    return dk, dv


# ------------------------------------------------------------------ full tensors
def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [batch, seqlen, heads, headdim]")
    b, n, hq, d = q.shape
    if k.shape[:2] != (b, n) or v.shape[:3] != k.shape[:3] or k.shape[3] != d:
        raise ValueError("k/v shapes do not match q")
    hkv = k.shape[2]
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    return b, n, hq, hkv, d


def _fwd_task(args):
    q, k, v, causal, window, scale, row_chunk, *slope = args
    return attn_fwd_head(q, k, v, causal, window, scale, row_chunk, *slope)


def _bwd_task(args):
    q, k, v, do, causal, window, scale, row_chunk, *slope = args
    return attn_bwd_head(q, k, v, do, causal, window, scale, row_chunk, *slope)


def _slopes(alibi_slopes, hq: int) -> np.ndarray:
    if alibi_slopes is None:
        return np.zeros(hq)
    m = np.asarray(alibi_slopes, dtype=np.float64).reshape(-1)
    if m.size != hq:
        raise ValueError(f"alibi_slopes must hold one slope per query head ({hq})")
    return m


def _limit_blas_threads():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: BLAS keeps its default
        pass


def _run(tasks, fn, workers):
    if workers is None or workers <= 1:
        return [fn(t) for t in tasks]
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=_limit_blas_threads) as ex:
        return list(ex.map(fn, tasks))


def default_workers(_=None) -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def attn_fwd(q, k, v, causal=False, window=0, scale=None, row_chunk=DEFAULT_ROW_CHUNK,
             workers=None, alibi_slopes=None):
    """Forward over [B, N, Hq, d] inputs (KV: [B, N, Hkv, d]).

    Returns O [B, N, Hq, dv] and LSE [B, Hq, N], float64.  ``workers`` > 1 runs the
    (batch, head) pairs in a process pool (heads are independent).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    b, n, hq, hkv, d = _check_shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = hq // hkv
    m = _slopes(alibi_slopes, hq)
    tasks = [(q[bi, :, h], k[bi, :, h // g], v[bi, :, h // g], causal, window, scale, row_chunk,
              m[h]) for bi in range(b) for h in range(hq)]
    res = _run(tasks, _fwd_task, workers)
    o = np.zeros((b, n, hq, v.shape[3]))
    lse = np.zeros((b, hq, n))
    for t, (oh, lh) in enumerate(res):
        bi, h = divmod(t, hq)
        o[bi, :, h] = oh
        lse[bi, h] = lh
    return o, lse


def attn_bwd(q, k, v, do, causal=False, window=0, scale=None, row_chunk=DEFAULT_ROW_CHUNK,
             workers=None, alibi_slopes=None):
    """Backward over full tensors: (dQ [B,N,Hq,d], dK, dV [B,N,Hkv,d], D [B,Hq,N]).

    dK and dV of a KV head are the sums over the query heads of its group (the
    chain rule through the shared K/V).
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    b, n, hq, hkv, d = _check_shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = hq // hkv
    m = _slopes(alibi_slopes, hq)
    tasks = [(q[bi, :, h], k[bi, :, h // g], v[bi, :, h // g], do[bi, :, h], causal, window,
              scale, row_chunk, m[h]) for bi in range(b) for h in range(hq)]
    res = _run(tasks, _bwd_task, workers)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros((b, hq, n))
    for t, (dqh, dkh, dvh, dh) in enumerate(res):
        bi, h = divmod(t, hq)
        dq[bi, :, h] = dqh
        dk[bi, :, h // g] += dkh
        dv[bi, :, h // g] += dvh
        dvec[bi, h] = dh
    return dq, dk, dv, dvec


def attended_pairs(n: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs one head attends, counted one row at a time."""
    total = 0
    for i in range(n):
        lo, hi = allowed_keys(i, n, causal, window)
        total += max(0, hi - lo)
    return total


# ------------------------------------------------------------------ packed sequences
def _check_cu(cu_seqlens, total: int) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing offsets from 0 to total")
    return cu


def attn_fwd_varlen(q, k, v, cu_seqlens, causal=False, window=0, scale=None,
                    row_chunk=DEFAULT_ROW_CHUNK, alibi_slopes=None):
    """Forward over packed sequences: q [T, Hq, d], k, v [T, Hkv, d].

    Sequence s is rows cu_seqlens[s] .. cu_seqlens[s+1]-1 of every tensor.  It is the
    plain attention above applied to each sequence by itself: its queries see only its own
    keys, and the causal / window masks count positions from the sequence's first row.
    (bmjup.com, FAQ Q4, names the variable-length interface; the packing is the reading
    this code takes of it.)  Returns O [T, Hq, dv] and LSE [Hq, T], float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    t, hq, d = q.shape
    hkv = k.shape[1]
    cu = _check_cu(cu_seqlens, t)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = hq // hkv
    m = _slopes(alibi_slopes, hq)
    o = np.zeros((t, hq, v.shape[2]))
    lse = np.zeros((hq, t))
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 == s0:
            continue
        for h in range(hq):
            oh, lh = attn_fwd_head(q[s0:s1, h], k[s0:s1, h // g], v[s0:s1, h // g], causal,
                                   window, scale, row_chunk, m[h])
            o[s0:s1, h] = oh
            lse[h, s0:s1] = lh
    return o, lse


def attn_bwd_varlen(q, k, v, do, cu_seqlens, causal=False, window=0, scale=None,
                    row_chunk=DEFAULT_ROW_CHUNK, alibi_slopes=None):
    """Backward over packed sequences: (dQ [T,Hq,d], dK, dV [T,Hkv,d], D [Hq,T]), each
    sequence on its own as in attn_fwd_varlen; dK, dV of a KV head summed over its group."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    t, hq, d = q.shape
    hkv = k.shape[1]
    cu = _check_cu(cu_seqlens, t)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = hq // hkv
    m = _slopes(alibi_slopes, hq)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros((hq, t))
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 == s0:
            continue
        for h in range(hq):
            dqh, dkh, dvh, dh = attn_bwd_head(q[s0:s1, h], k[s0:s1, h // g], v[s0:s1, h // g],
                                              do[s0:s1, h], causal, window, scale, row_chunk,
                                              m[h])
            dq[s0:s1, h] = dqh
            dk[s0:s1, h // g] += dkh
            dv[s0:s1, h // g] += dvh
            dvec[h, s0:s1] = dh
    return dq, dk, dv, dvec


# ------------------------------------------------------------------ decoding over a cache
def attn_decode(q, k_cache, v_cache, seqlens_k=None, causal=True, window=0, scale=None):
    """Attention of the newest queries of each sequence over its cached keys.

    q [B, Nq, Hq, d]: the Nq newest tokens; k_cache, v_cache [B, Nk, Hkv, d]: the cache,
    of which sequence b uses the first seqlens_k[b] rows (all Nk when None).  Query i of
    sequence b sits at position len_b - Nq + i (the queries are the sequence's last Nq
    positions), and the causal and window masks count from there; without the causal mask
    every query sees all len_b keys (the window still bounds from the left).  This is plain
    attention over the cache for the pages' use in inference (bmjup.com, FAQ on inference:
    streaming generation and large context caches).  Returns O [B, Nq, Hq, dv] and
    LSE [B, Hq, Nq]; a query with no allowed key gets O = 0 and LSE = -inf.
    """
    q, k_cache, v_cache = _as64(q), _as64(k_cache), _as64(v_cache)
    b, nq, hq, d = q.shape
    nk, hkv = k_cache.shape[1], k_cache.shape[2]
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    lens = np.full(b, nk) if seqlens_k is None else np.asarray(seqlens_k, dtype=np.int64)
    if lens.shape != (b,) or np.any(lens < 0) or np.any(lens > nk):
        raise ValueError("seqlens_k must hold one length in [0, Nk] per sequence")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = hq // hkv
    o = np.zeros((b, nq, hq, v_cache.shape[3]))
    lse = np.full((b, hq, nq), -np.inf)
    for bi in range(b):
        n = int(lens[bi])
        pos = n - nq + np.arange(nq)          # positions of the queries
        j = np.arange(n)[None, :]
        ok = np.ones((nq, n), dtype=bool)
        if causal:
            ok &= j <= pos[:, None]
        if window > 0:
            ok &= j >= pos[:, None] - window + 1
        for h in range(hq):
            s = scale * (q[bi, :, h] @ k_cache[bi, :n, h // g].T)
            s = np.where(ok, s, -np.inf)
            m = s.max(axis=1) if n > 0 else np.full(nq, -np.inf)
            fin = np.isfinite(m)
            m0 = np.where(fin, m, 0.0)
            e = np.exp(s - m0[:, None])
            den = e.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                p = np.where(fin[:, None], e / np.where(fin, den, 1.0)[:, None], 0.0)
                lse[bi, h] = np.where(fin, m0 + np.log(np.where(fin, den, 1.0)), -np.inf)
            o[bi, :, h] = p @ v_cache[bi, :n, h // g]
    return o, lse
