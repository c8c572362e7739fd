"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m exact_io_aware_fa2_amd.build        # compiles every time it is called

The library lands next to this file as ``libfa.so``; the Python binding loads it from
there.  hipcc cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

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
    "-shared",
    "-munsafe-fp-atomics",
    # keep the compiler away from packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return cand


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile libfa.so; returns its path.  Raises on a compiler error."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + (extra_flags or []) + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
