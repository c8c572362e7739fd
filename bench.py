#!/usr/bin/env python3
"""One-GPU benchmark of the exact-attention hot path (forward + recompute backward).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one forward (fa_fwd) and one backward (fa_bwd) over one batch of the workload,
with every input already resident in device memory; a packed-sequence workload
(--workload bf16_varlen_...) runs fa_fwd_varlen / fa_bwd_varlen instead and sums the FLOPs
over its sequences.  The timed region is bracketed by
torch.cuda.synchronize(); per-launch kernel durations come from HIP events recorded on the
stream the kernels run on.  Prints ONE JSON line.

FLOP convention (algorithmic, independent of how the kernels schedule the work):
  forward  = 4 * B * Hq * pairs * d, pairs = N^2 (full), N^2 / 2 (causal),
             W (W + 1) / 2 + (N - W) W (causal with a W-key window)
  backward = 2.5 x forward (five products per attended pair: S, dP, dV, dK, dQ)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak (256 CU x 2.4 GHz x 4096)
MFMA_FP8_PEAK_TFLOPS = 5033.2   # MI355X dense fp8 matrix peak (twice the bf16 rate)
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def attended_pairs(N: int, causal: bool, window: int) -> float:
    """(query, key) pairs one head attends, with the metric's convention for causal."""
    if not causal and window <= 0:
        return float(N) * N
    if causal and window <= 0:
        return N * N / 2.0  # the metric's "halved for causal" convention
    if causal:
        W = min(window, N)
        return W * (W + 1) / 2.0 + (N - W) * W
    # left bound only: row i sees keys max(0, i - W + 1) .. N - 1
    return float(sum(N - max(0, i - window + 1) for i in range(N)))


def fwd_flops(w) -> float:
    return 4.0 * w.B * w.Hq * attended_pairs(w.N, w.causal, w.window) * w.d


def _src_sha(name: str) -> str:
    """Hash of a kernel source together with the device-code header every kernel includes and
    the build script that holds the compiler flags."""
    h = hashlib.sha256()
    for rel in (os.path.join("csrc", name), os.path.join("csrc", "fa_common.hpp"), "build.py"):
        with open(os.path.join(ROOT, "exact_io_aware_fa2_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str, source: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None when the
    kernel source changed since the counters were taken."""
    p = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            rec = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != _src_sha(source):
        return None
    return rec.get("bytes_per_launch")


def mfma_probe(fa, torch, dev, stream, blocks: int = 2048, iters: int = 20000, reps: int = 3):
    """Sustained bf16 MFMA throughput of a products-only kernel (TFLOP/s, best of reps)."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    sh = stream.cuda_stream
    if fa.fa_mfma_probe(out, blocks, 100, sh) != fa.FA_OK:
        raise RuntimeError(fa.fa_last_error())
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if fa.fa_mfma_probe(out, blocks, iters, sh) != fa.FA_OK:
            raise RuntimeError(fa.fa_last_error())
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    flop = blocks * 4 * 4 * iters * 32768.0  # waves x chains x iters x flop per product
    return flop / (best * 1e-3) / 1e12


ISSUE_PROBES = {  # kind: (name, params) of fa_issue_probe
    0: ("fma_per_mfma", (0, 2, 4, 6, 8, 12)),
    1: ("exp_per_mfma", (1, 2, 3, 4, 6, 8)),
    2: ("chains", (1, 2, 4, 8)),
    3: ("lds_operands_per_mfma", (0, 1, 2, 10, 11, 12, 20, 21, 22)),
    6: ("global_operand_per_mfma", (1, 2, 3)),
}


def issue_probe(fa, torch, dev, stream, iters: int = 4000, reps: int = 3):
    """Matrix-core throughput (fraction of the 2516.6 TFLOP/s peak, best of reps) with the
    fa_issue_probe variants, one workgroup per CU at one and two waves per SIMD."""
    blocks = 256
    out = torch.zeros(blocks * 512, dtype=torch.float32, device=dev)
    sh = stream.cuda_stream
    res = {}
    for kind, (name, params) in ISSUE_PROBES.items():
        res[name] = {}
        for wps in (1, 2):
            row = {}
            for param in params:
                if fa.fa_issue_probe(out, kind, param, wps, blocks, 20, sh) != fa.FA_OK:
                    raise RuntimeError(fa.fa_last_error())
                best = None
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    if fa.fa_issue_probe(out, kind, param, wps, blocks, iters, sh) != fa.FA_OK:
                        raise RuntimeError(fa.fa_last_error())
                    e1.record(stream)
                    e1.synchronize()
                    ms = e0.elapsed_time(e1)
                    best = ms if best is None else min(best, ms)
                rounds = (iters + (iters & 1) if kind == 3 else
                          (iters + 3) // 4 * 4 if kind == 6 else iters)
                products = 8 if kind == 2 else 4
                flop = blocks * 4 * wps * rounds * products * 32768.0
                row[str(param)] = round(flop / (best * 1e-3) / 1e12 / 2516.6, 4)
            res[name][f"waves_per_simd_{wps}"] = row
    return res


LDS_PROBE_STRIDES = (4, 8, 16, 32, 64, 128, 256)


def lds_probe(fa, torch, dev, stream, iters: int = 2000):
    """Launch the LDS bank probes of fa_issue_probe (kinds 4 and 5) once each, one workgroup
    per CU, in the order returned; the bank-conflict counters of these launches (rocprofv3
    --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS) give cycles per access."""
    blocks = 256
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    sh = stream.cuda_stream
    launches = []
    for kind, access in ((4, "store"), (5, "load")):
        for width in (4, 8, 16):
            for stride in LDS_PROBE_STRIDES:
                if fa.fa_issue_probe(out, kind, width * 10000 + stride, 1, blocks, iters, sh) != fa.FA_OK:
                    raise RuntimeError(fa.fa_last_error())
                launches.append({"access": access, "width_bytes": width, "stride_bytes": stride})
    torch.cuda.synchronize()
    return {"launches_in_order": launches, "workgroups": blocks, "waves_per_workgroup": 4,
            "iters": iters}


def atomic_dq_count(w, bkn: int = 256, bq: int = 32) -> int:
    """float32 atomic adds an atomic accumulation of dQ would issue for a fixed-length
    workload: every key block of `bkn` keys adds, for each 32-row step it visits (the same
    steps the key-block kernel walks) and each query head of its group, one 32 x d tile of
    its contribution summed over its keys."""
    total = 0
    for kb in range((w.N + bkn - 1) // bkn):
        n0 = kb * bkn
        qb_lo = n0 // bq if w.causal else 0
        row_end = min(w.N, n0 + bkn + w.window - 1) if w.window > 0 else w.N
        total += max(0, (row_end + bq - 1) // bq - qb_lo)
    return total * w.B * w.Hq * bq * w.d


def atomic_probe(fa, torch, dev, stream, w, blocks: int = 2048, iters: int = 64):
    """Measured float32 atomic rate (adds/s) in the tile pattern of an atomic dQ, into an
    accumulator of the workload's [B, N, Hq, d] shape (best of 3)."""
    stride = w.Hq * w.d
    row_blocks = (w.B * w.N) // 32
    acc = torch.zeros(row_blocks * 32 * stride, dtype=torch.float32, device=dev)
    sh = stream.cuda_stream
    if fa.fa_atomic_probe(acc, row_blocks, stride, blocks, 4, sh) != fa.FA_OK:
        raise RuntimeError(fa.fa_last_error())
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if fa.fa_atomic_probe(acc, row_blocks, stride, blocks, iters, sh) != fa.FA_OK:
            raise RuntimeError(fa.fa_last_error())
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del acc
    return blocks * iters * 4096 / (best * 1e-3), best


def _head_tasks(w, q, k, v, do, packed):
    """(flop, task maker) per (batch entry or sequence, query head), in an order that
    spreads a prefix over every sequence length: head-major for packed batches."""
    import numpy as np
    import oracle.attention as oa

    g = w.Hq // w.Hkv
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    if packed:
        cu = w.cu_seqlens
        slots = [(h, s) for h in range(w.Hq) for s in range(len(w.lengths)) if w.lengths[s]]
        for h, s in slots:
            a, n = cu[s], w.lengths[s]
            flop = 4.0 * attended_pairs(n, w.causal, w.window) * w.d
            yield flop, lambda a=a, n=n, h=h: (
                f64(q[a:a + n, h]), f64(k[a:a + n, h // g]), f64(v[a:a + n, h // g]),
                None if do is None else f64(do[a:a + n, h]), w.causal, w.window, w.scale,
                oa.DEFAULT_ROW_CHUNK)
    else:
        from exact_io_aware_fa2_amd.workloads import alibi_slopes
        flop = 4.0 * attended_pairs(w.N, w.causal, w.window) * w.d
        # ALiBi: the slope each head's oracle task adds (the float32 value the kernels read)
        slopes = ([float(np.float32(m)) for m in alibi_slopes(w.Hq)]
                  if getattr(w, "alibi", False) else None)
        for i in range(w.B * w.Hq):
            b, h = i // w.Hq, i % w.Hq
            yield flop, lambda b=b, h=h: (
                f64(q[b, :, h]), f64(k[b, :, h // g]), f64(v[b, :, h // g]),
                None if do is None else f64(do[b, :, h]), w.causal, w.window, w.scale,
                oa.DEFAULT_ROW_CHUNK) + ((slopes[h],) if slopes else ())


def cpu_baseline(w, q, k, v, do, packed=False, max_workers: int = 16):
    """Time the float64 oracle on a bounded sample of (batch entry or sequence, head) pairs
    of the same inputs on the host cores; report algorithmic TFLOP/s with the same FLOP
    convention."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    import oracle.attention as oa

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(max_workers, cores))
    bwd = do is not None
    mult = 3.5 if bwd else 1.0
    # about 20 s of wall time at ~25 GFLOP/s per float64 worker, at most the whole workload
    budget = 20.0 * workers * 25e9
    tasks, flop, n_all = [], 0.0, 0
    for f, t in _head_tasks(w, q, k, v, do, packed):
        n_all += 1
        if len(tasks) >= workers and flop >= budget:
            continue
        tasks.append(t())
        flop += f * mult
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=oa._limit_blas_threads) as ex:
        # start every worker before the clock runs
        list(ex.map(oa.default_workers, range(workers)))
        t0 = time.perf_counter()
        list(ex.map(oa._fwd_task, [t[:3] + t[4:] for t in tasks]))
        if bwd:
            list(ex.map(oa._bwd_task, tasks))
        dt = time.perf_counter() - t0
    what = "(sequence, head)" if packed else "(batch, head)"
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s (fwd+bwd, algorithmic)" if bwd else "TFLOP/s (fwd, algorithmic)",
        "cores": workers,
        "host_cores": cores,
        "kind": "oracle",
        "sample": f"{len(tasks)} of {n_all} {what} pairs of {w.name}, "
                  f"{'forward + backward' if bwd else 'forward'}, float64 NumPy, "
                  f"{workers} worker processes x 1 BLAS thread on a host with {cores} "
                  f"cores, {dt:.1f} s wall",
        "seconds": dt,
    }


def _decode_task(args):
    import oracle.attention as oa
    q, k, v, n, causal, window, scale = args
    return oa.attn_decode(q, k, v, [n], causal, window, scale)


def cpu_baseline_decode(w, q, k, v, flop_per_seq, max_workers: int = 16):
    """The float64 oracle's attn_decode, one task per sequence, on the host cores."""
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    import oracle.attention as oa

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(max_workers, cores, w.B))
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    tasks = [(f64(q[b:b + 1]), f64(k[b:b + 1, :n]), f64(v[b:b + 1, :n]), n, w.causal, w.window,
              w.scale) for b, n in enumerate(w.lens)]
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=oa._limit_blas_threads) as ex:
        list(ex.map(oa.default_workers, range(workers)))
        t0 = time.perf_counter()
        list(ex.map(_decode_task, tasks))
        dt = time.perf_counter() - t0
    return {
        "value": sum(flop_per_seq) / dt / 1e12,
        "unit": "TFLOP/s (decode, algorithmic)",
        "cores": workers,
        "host_cores": cores,
        "kind": "oracle",
        "sample": f"all {w.B} sequences of {w.name}, float64 NumPy attn_decode, {workers} worker "
                  f"processes x 1 BLAS thread, {dt:.1f} s wall",
        "seconds": dt,
    }


def decode_bytes_and_flop(w):
    """Algorithmic HBM bytes and flop of one decoding step: each sequence's K and V rows that
    some query may attend, read once per KV head, plus q, o (bf16) and lse (float32)."""
    total_b, flops = 0, []
    for n in w.lens:
        pos = [n - w.Nq + i for i in range(w.Nq)]
        lo = max(0, n - w.Nq - w.window + 1) if w.window > 0 else 0
        keys = max(0, n - lo)
        total_b += keys * w.Hkv * w.d * 2 * 2
        pairs = 0
        for p in pos:
            hi = min(n, p + 1) if w.causal else n
            l0 = max(0, p - w.window + 1) if w.window > 0 else 0
            pairs += max(0, hi - l0)
        flops.append(4.0 * w.d * w.Hq * pairs)
    total_b += w.B * w.Nq * w.Hq * w.d * 2 * 2 + w.B * w.Hq * w.Nq * 4
    return total_b, flops


def run_decode(args, w):
    import torch
    from exact_io_aware_fa2_amd import fa
    from exact_io_aware_fa2_amd.workloads import make_decode_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    q, k, v, sl = make_decode_inputs(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), device=dev, dtype=torch.float32)
    S = fa.fa_decode_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, 0)
    nbytes = fa.fa_decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, S)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def step():
        st = fa.fa_decode(q, k, v, sl, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal,
                          w.window, w.scale, S, ws, nbytes, sh)
        if st != fa.FA_OK:
            raise RuntimeError(fa.fa_last_error())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for e in ev:
        e[2].record(stream)
        e[3].record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(K):
        e = ev[s_]
        fa.fa_bwd_time_main_kernel(e[2], e[3])  # events around the chunk kernel
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [e[0].elapsed_time(e[1]) for e in ev]
    kern_ms = [e[2].elapsed_time(e[3]) for e in ev]
    avg = lambda xs: sum(xs) / len(xs)  # noqa: E731
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    nb, flops = decode_bytes_and_flop(w)
    F = sum(flops)
    ms_step = wall * 1e3 / K
    km = avg(kern_ms)
    out = {
        "metric": "attention fwd & fwd+bwd TFLOPs/s (bf16, d=128, N=8K causal); % of MFMA peak",
        "value": F / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s (decode step, algorithmic)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, 1) draws, rounded to bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "Nk": w.Nk, "d": w.d, "causal": w.causal, "window": w.window,
                   "num_splits": S, "scale": w.scale},
        "tokens_per_s": w.B * w.Nq / (ms_step * 1e-3),
        "decode_call_ms": avg(call_ms),
        "kernel_ms": {"decode_call": {"mean": avg(call_ms), "median": med(call_ms),
                                      "min": min(call_ms)},
                      "decode_kernel": {"mean": km, "median": med(kern_ms), "min": min(kern_ms)}},
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": nb / (km * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nb / (km * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": _traffic("decode_kernel", w.name, "fa_decode.hip"),
                     "algorithmic_bytes": nb, "avg_launch_ms": km},
    }
    if args.probe_issue:
        out["issue_probe_frac_of_peak"] = issue_probe(fa, torch, dev, stream)
    if args.probe_lds:
        out["lds_probe"] = lds_probe(fa, torch, dev, stream)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = src.numel()
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, q, k, v, flops)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, help="workload name (default: bf16_b2_h32_n8192_d128_causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the products-only MFMA throughput probe (profiling runs)")
    ap.add_argument("--probe-atomic-dq", action="store_true",
                    help="also time float32 atomics in the pattern of an atomic dQ and price "
                         "that alternative to the separate dQ pass at this workload")
    ap.add_argument("--probe-issue", action="store_true",
                    help="also run the fa_issue_probe table: matrix-core throughput next to "
                         "FMAs, exp2, LDS operand reads, and over dependent chains")
    ap.add_argument("--probe-lds", action="store_true",
                    help="also launch the LDS bank probes (store and load, 4/8/16 bytes per "
                         "lane, strides 4-256 bytes) for a rocprofv3 counter run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a known-size kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 (the attention kernels "
                          "shard over (batch, head) pairs with no communication; a "
                          "multi-GPU launch is not part of this benchmark)"}))
        return 2

    from exact_io_aware_fa2_amd.workloads import DECODE_WORKLOADS
    if args.workload in DECODE_WORKLOADS:
        return run_decode(args, DECODE_WORKLOADS[args.workload])

    import torch
    from exact_io_aware_fa2_amd import fa
    from exact_io_aware_fa2_amd.workloads import (ALIBI_WORKLOADS, FP8_WORKLOADS, DEFAULT_WORKLOAD,
                                                  VARLEN_WORKLOADS, WORKLOADS, alibi_slopes,
                                                  make_fp8_inputs, make_inputs,
                                                  make_varlen_inputs)

    name = args.workload or DEFAULT_WORKLOAD
    packed = name in VARLEN_WORKLOADS
    fp8 = name in FP8_WORKLOADS
    w = (VARLEN_WORKLOADS[name] if packed else FP8_WORKLOADS[name] if fp8 else
         ALIBI_WORKLOADS[name] if name in ALIBI_WORKLOADS else WORKLOADS[name])
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    if packed:
        q, k, v, do = make_varlen_inputs(w, dev)
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device=dev)
        S, T, M = len(w.lengths), w.total, w.max_seqlen
        lse = torch.empty((w.Hq, T), device=dev, dtype=torch.float32)
        F = sum(4.0 * w.Hq * attended_pairs(n, w.causal, w.window) * w.d for n in w.lengths)
        config = {"workload": w.name, "num_seqs": S, "total": T, "max_seqlen": M,
                  "lengths": list(w.lengths), "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                  "causal": w.causal, "window": w.window, "scale": w.scale}
    elif fp8:
        q, k, v, factors = make_fp8_inputs(w, dev)
        do = None
        lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
        F = fwd_flops(w)
        config = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                  "causal": w.causal, "window": w.window, "scale": w.scale,
                  "inputs": "E4M3 codes, one float32 factor per tensor", "descale": factors}
    else:
        q, k, v, do = make_inputs(w, dev)
        lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
        F = fwd_flops(w)
        config = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                  "causal": w.causal, "window": w.window, "scale": w.scale}
    slopes = None
    if getattr(w, "alibi", False):
        slopes = torch.tensor(alibi_slopes(w.Hq), dtype=torch.float32, device=dev)
        config["alibi_slopes"] = "2^(-8 h / Hq), h = 1 .. Hq"
    o = torch.empty(q.shape, device=dev, dtype=torch.bfloat16) if fp8 else torch.empty_like(q)
    bwd = do is not None and w.dtype == "bf16"
    if bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        if packed:
            ws = fa.workspace_for_varlen(T, w.Hq, w.Hkv, w.d, dev)
        else:
            ws = fa.workspace_for(w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window, dev)
        ws_bytes = ws.numel()
    fwd_fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_fp32

    def run_fwd():
        if packed:
            st = fa.fa_fwd_varlen(q, k, v, o, lse, cu, S, T, M, w.Hq, w.Hkv, w.d, w.causal,
                                  w.window, w.scale, sh)
        elif fp8:
            st = fa.fa_fwd_fp8(q, k, v, o, lse, *factors, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal,
                               w.window, w.scale, sh)
        elif slopes is not None:
            st = fa.fa_fwd_alibi(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window,
                                 w.scale, slopes, sh)
        else:
            st = fwd_fn(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window,
                        w.scale, sh)
        if st != fa.FA_OK:
            raise RuntimeError(fa.fa_last_error())

    def run_bwd():
        if packed:
            st = fa.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, cu, S, T, M, w.Hq, w.Hkv,
                                  w.d, w.causal, w.window, w.scale, ws, ws_bytes, sh)
        elif slopes is not None:
            st = fa.fa_bwd_alibi(q, k, v, o, do, lse, dq, dk, dv, w.B, w.Hq, w.Hkv, w.N, w.d,
                                 w.causal, w.window, w.scale, ws, ws_bytes, slopes, sh)
        else:
            st = fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, w.B, w.Hq, w.Hkv, w.N, w.d,
                           w.causal, w.window, w.scale, ws, ws_bytes, sh)
        if st != fa.FA_OK:
            raise RuntimeError(fa.fa_last_error())

    for _ in range(args.warmup):
        run_fwd()
        if bwd:
            run_bwd()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for e in ev:  # torch creates the HIP event at its first record; the hook needs handles
        e[4].record(stream)
        e[5].record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        run_fwd()
        e[1].record(stream)
        if bwd:
            fa.fa_bwd_time_main_kernel(e[4], e[5])
            e[2].record(stream)
            run_bwd()
            e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    ms_step = wall * 1e3 / K
    total_flop = F * (3.5 if bwd else 1.0)
    out = {
        "metric": "attention fwd & fwd+bwd TFLOPs/s (bf16, d=128, N=8K causal); % of MFMA peak",
        "value": total_flop / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s (fwd+bwd)" if bwd else "TFLOP/s (fwd)",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3"}.get(w.dtype, "f32"),
        "data": "synthetic (seeded N(0, sigma^2) draws, rounded to the compute dtype)",
        "config": config,
    }
    avg = lambda xs: sum(xs) / len(xs)  # noqa: E731
    fwd_avg = avg(fwd_ms)
    out["fwd_ms"] = fwd_avg
    out["fwd_tflops"] = F / (fwd_avg * 1e-3) / 1e12
    peak = MFMA_FP8_PEAK_TFLOPS if fp8 else MFMA_BF16_PEAK_TFLOPS
    out["fwd_frac_of_peak"] = out["fwd_tflops"] / peak
    fwd_name = ("fwd_fp8_kernel" if fp8 else
                "fwd_bf16_kernel" if w.d <= 128 else "fwd_bf16_d256_kernel")
    kernels = {fwd_name: (fwd_avg, F, "fa_fwd_fp8.hip" if fp8 else "fa_fwd.hip")}
    if bwd:
        bwd_ms = [e[2].elapsed_time(e[3]) for e in ev]
        pre_ms = [e[2].elapsed_time(e[4]) for e in ev]   # D = rowsum(dO * O)
        kv_ms = [e[4].elapsed_time(e[5]) for e in ev]    # key-block kernel: dK, dV
        q_ms = [e[5].elapsed_time(e[3]) for e in ev]     # query-block kernel: dQ
        out["bwd_ms"] = avg(bwd_ms)
        out["bwd_pre_ms"] = avg(pre_ms)
        out["bwd_dkdv_kernel_ms"] = avg(kv_ms)
        out["bwd_dq_kernel_ms"] = avg(q_ms)
        out["fwd_bwd_tflops_kernels"] = total_flop / ((fwd_avg + avg(bwd_ms)) * 1e-3) / 1e12
        out["fwd_bwd_frac_of_peak"] = out["value"] / MFMA_BF16_PEAK_TFLOPS
        # Algorithmic work of each kernel (its share of the five products per attended pair,
        # 2.5x the forward): the dK/dV kernel does S, dP, dV and dK (2x the forward); the dQ
        # kernel's own product is dQ (0.5x the forward) -- it also recomputes S and dP, which
        # is work of the method's two-kernel schedule, not of the algorithm, and earns no
        # credit here.  d <= 128 runs the 8-wave key-block kernel, d = 256 the 4-wave one.
        kv_name = "bwd_dkdv8_kernel" if w.d <= 128 else "bwd_dkdv_kernel"
        kernels[kv_name] = (avg(kv_ms), 2.0 * F, "fa_bwd.hip")
        kernels["bwd_dq_kernel"] = (avg(q_ms), 0.5 * F, "fa_bwd.hip")
        out["bwd_dq_kernel_executed_tflops"] = 1.5 * F / (avg(q_ms) * 1e-3) / 1e12
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    stats = {"fwd": fwd_ms}
    if bwd:
        stats.update({"bwd": bwd_ms, "bwd_pre": pre_ms, "bwd_dkdv": kv_ms, "bwd_dq": q_ms})
    out["kernel_ms"] = {n: {"mean": avg(xs), "median": med(xs), "min": min(xs)}
                        for n, xs in stats.items()}
    probe = None
    if w.dtype == "bf16" and not args.no_mfma_probe:
        probe = mfma_probe(fa, torch, dev, stream)
        out["mfma_probe_tflops"] = probe
        # the clock the probe implies: peak is 1024 flop / clock / SIMD x 1024 SIMDs
        out["mfma_probe_implied_sclk_mhz"] = probe * 1e12 / (1024 * 1024) / 1e6
    if w.dtype in ("bf16", "fp8"):
        name = max(kernels, key=lambda n: kernels[n][0])
        ms, flop, src = kernels[name]
        achieved = flop / (ms * 1e-3) / 1e12
        out["roofline"] = {
            "kernel": name,
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": _traffic(name, w.name, src),
            "avg_launch_ms": ms,
            "frac_of_measured_mfma": achieved / probe if probe else None,
        }
        out["fwd_frac_of_measured_mfma"] = out["fwd_tflops"] / probe if probe else None
    if args.probe_atomic_dq and bwd and not packed:
        rate, ms = atomic_probe(fa, torch, dev, stream, w)
        need = atomic_dq_count(w)
        out["atomic_dq"] = {
            "probe_atomics_per_s": rate, "probe_ms": ms,
            "atomics_for_workload": need,
            "atomic_adds_ms_estimate": need / rate * 1e3,
            "separate_dq_pass_ms": out["bwd_dq_kernel_ms"],
            "note": "time of the atomic adds alone, at the probe's rate; an atomic dQ would "
                    "also add the dQ products and a transpose of dS to the key-block kernel, "
                    "and a zeroing and a conversion pass of the float32 accumulator"}
    if args.probe_issue:
        out["issue_probe_frac_of_peak"] = issue_probe(fa, torch, dev, stream)
    if args.probe_lds:
        out["lds_probe"] = lds_probe(fa, torch, dev, stream)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = src.numel()
        del src, dst
    out["context"] = ("pages' A100 figures at 16K tokens (other hardware, not a target): "
                      "~50 TFLOP/s standard PyTorch attention vs >180 TFLOP/s FlashAttention-2")
    if not args.no_cpu_baseline:
        if fp8:  # the oracle runs on the dequantised inputs
            deq = [t.view(torch.float8_e4m3fn).float() * f for t, f in zip((q, k, v), factors)]
            out["cpu_baseline"] = cpu_baseline(w, *deq, None, packed)
        else:
            out["cpu_baseline"] = cpu_baseline(w, q, k, v, do if bwd else None, packed)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
