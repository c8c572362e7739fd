"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m exact_io_aware_fa2_amd.build        # compiles every time it is called

The library lands next to this file as ``libfa.so``; the Python binding loads it from
there.  hipcc cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_decode.hip",
           "fa_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    # keep the compiler away from packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source flags.  The two forward kernels measured 1-3 % faster (interleaved A/B runs)
# with the backend's iterative register-minimising scheduler; the backward kernels are
# fastest with the default one.
# VGPR-form matrix products: a kernel that needs more than 256 registers per lane (the
# head-dim-256 instances, one wave per SIMD) otherwise gets its products in the AGPR form,
# and the backend then moves accumulators and operands between AGPRs and VGPRs around every
# product and every softmax (hundreds of v_accvgpr moves per 32-key piece).  With the VGPR
# form the accumulators stay in VGPRs and AGPRs only hold values spilled out of the loop's
# way.  Kernels within 256 registers compile to identical code either way.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {
    "fa_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"] + VGPR_FORM,
    "fa_fwd_fp8.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"] + VGPR_FORM,
    "fa_bwd.hip": VGPR_FORM,
}


def hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return cand


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source to an object (in parallel) and link libfa.so; returns its path.
    Raises on a compiler error."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="libfa_build_") as tmpdir:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            jobs.append((obj, [cc] + HIPCC_FLAGS + FILE_FLAGS.get(src, []) + (extra_flags or []) +
                         ["-c", os.path.join(CSRC, src), "-o", obj]))
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as pool:
            for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
                f.result()
        tmp = LIB + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for o, _ in jobs] +
             ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
