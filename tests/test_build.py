"""Build checks on the CPU (hipcc cross-compiles for gfx950 without a GPU).

No kernel may use scratch memory (register spills to memory inside an inner loop cost more
than the changes that would cause one save).  The kernels for head dims 64 and 128 must
also compile without any vector-register spill; the head-dim-256 kernels run one wave per
SIMD with up to 512 registers per lane, where a few values parked in AGPRs (counted as
spills by the compiler, but register moves, not memory traffic) are allowed.  The check
uses the flags of the real build (exact_io_aware_fa2_amd/build.py, per-source flags
included).
"""

import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from exact_io_aware_fa2_amd import build as B

SOURCES = ["fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_decode.hip"]


def _resource_usage(src: str, tmpdir: str) -> dict:
    cmd = ([B.hipcc()] + B.HIPCC_FLAGS + B.FILE_FLAGS.get(src, []) +
           ["-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(B.CSRC, src),
            "-o", os.path.join(tmpdir, src + ".o")])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    usage, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|VGPRs Spill|SGPRs Spill|ScratchSize) ?"
                      r"(?:\[bytes/lane\])?: (\d+)", line)
        if m and name:
            usage[name][m.group(1)] = int(m.group(2))
    return usage


@pytest.fixture(scope="module")
def usage():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmpdir:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            parts = list(pool.map(lambda s: _resource_usage(s, tmpdir), SOURCES))
    out = {}
    for p in parts:
        out.update(p)
    return out


def test_every_attention_kernel_is_reported(usage):
    names = " ".join(usage)
    for k in ("fwd_bf16_kernel", "fwd_fp8_kernel", "bwd_dkdv8_kernel", "bwd_dq_kernel",
              "bwd_pre_kernel", "decode_kernel"):
        assert k in names, k


def test_no_vector_register_spills_for_head_dims_up_to_128(usage):
    # (vector spills go to scratch memory; scalar spills stay in VGPR lanes)
    bad = {n: u for n, u in usage.items()
           if ("ILi64E" in n or "ILi128E" in n) and u.get("VGPRs Spill", 0) > 0}
    assert not bad, bad


def test_no_kernel_uses_scratch_memory(usage):
    assert usage, "no kernels reported"
    missing = [n for n, u in usage.items() if "ScratchSize" not in u]
    assert not missing, missing
    bad = {n: u for n, u in usage.items() if u["ScratchSize"] > 0}
    assert not bad, bad


def test_head_dim_256_kernels_are_covered(usage):
    names = " ".join(n for n in usage if "ILi256E" in n)
    for k in ("fwd_bf16_kernel", "fwd_fp8_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
        assert k in names, k
