"""Build checks on the CPU (hipcc cross-compiles for gfx950 without a GPU).

The last two checks read the generated assembly of the head-dim-256 key-block kernel and
the head-dim-256 forward, whose dK/dV and O products are inline assembly with hand-written
wait states (see there).

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
    for k in ("fwd_bf16_kernel", "fwd_bf16_d256_kernel", "fwd_fp8_kernel", "bwd_dkdv8_kernel",
              "bwd_dq_kernel", "bwd_pre_kernel", "decode_kernel"):
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
    for k in ("fwd_fp8_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
        assert k in names, k
    # the bf16 forward has a kernel of its own for d = 256 (templated on the bias only)
    assert sum("fwd_bf16_d256_kernel" in n for n in usage) == 3


# The head-dim-256 key-block kernel accumulates dK and dV in AGPRs through matrix products
# written as inline assembly; the compiler does not see them as matrix instructions, so the
# wait states around them are written out in the source.  These checks read the generated
# gfx950 assembly and pin what those waits rely on: the accumulators are touched by vector
# instructions only before the first product (zeroing, then the short fence) and after the
# long fence that follows the last one, and nothing moves them inside the step loop.
ASM_PRODUCT = re.compile(r"v_mfma_f32_32x32x16_bf16 a\[(\d+):(\d+)\], v\[\d+:\d+\], "
                         r"v\[\d+:\d+\], a\[(\d+):(\d+)\]")


@pytest.fixture(scope="module")
def bwd_asm():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmpdir:
        out = os.path.join(tmpdir, "fa_bwd.s")
        cmd = ([B.hipcc()] + B.HIPCC_FLAGS + B.FILE_FLAGS.get("fa_bwd.hip", []) +
               ["--cuda-device-only", "-S", os.path.join(B.CSRC, "fa_bwd.hip"), "-o", out])
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return f.read()


def _function_bodies(asm: str, prefix: str) -> dict:
    lines = asm.splitlines()
    bodies, i = {}, 0
    while i < len(lines):
        if lines[i].startswith(prefix) and lines[i].split(":")[0] == lines[i].split()[0][:-1]:
            name = lines[i].split(":")[0]
            j = next(k for k in range(i, len(lines)) if lines[k].startswith(".Lfunc_end"))
            bodies[name] = [l.strip() for l in lines[i:j]]
            i = j
        i += 1
    return bodies


def _asm_blocks(body: list) -> list:
    """(line index, text) of every inline-assembly block of a function body."""
    out, i = [], 0
    while i < len(body):
        if body[i].startswith(";;#ASMSTART"):
            j = i + 1
            while not body[j].startswith(";;#ASMEND"):
                j += 1
            out.append((i, "\n".join(body[i + 1:j])))
            i = j
        i += 1
    return out


def test_head_dim_256_key_block_kernel_fences_its_agpr_products(bwd_asm):
    bodies = _function_bodies(bwd_asm, "_ZN2fa15bwd_dkdv_kernelILi256E")
    assert len(bodies) == 3, list(bodies)  # unbiased, causal and general position bias
    for name, body in bodies.items():
        blocks = _asm_blocks(body)
        products = [(i, t) for i, t in blocks if "v_mfma" in t]
        # 8 head-dim tiles x 2 k-steps x (dV, dK) per step, unrolled
        assert len(products) == 32, (name, len(products))
        for _, t in products:
            m = ASM_PRODUCT.search(t)
            assert m and m.group(1, 2) == m.group(3, 4), (name, t)  # acc += a b in AGPRs
        written = [i for i, t in blocks if t.strip() == "s_nop 4"]
        ready = [i for i, t in blocks if t.split() == ["s_nop", "7", "s_nop", "7", "s_nop", "7"]]
        assert len(written) == 2 and len(ready) == 2, (name, len(written), len(ready))
        first, last = products[0][0], products[-1][0]
        assert max(written) < first < last < min(ready), name
        acc_moves = [i for i, l in enumerate(body) if l.startswith("v_accvgpr_")]
        between = [i for i in acc_moves if first < i < max(ready)]
        assert not between, (name, [body[i] for i in between][:4])
        reads = [i for i in acc_moves if body[i].startswith("v_accvgpr_read")]
        assert reads and min(reads) > max(ready), name
        writes = [i for i in acc_moves if not body[i].startswith("v_accvgpr_read")]
        assert writes and max(writes) < min(written), name


@pytest.fixture(scope="module")
def fwd_asm():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmpdir:
        out = os.path.join(tmpdir, "fa_fwd.s")
        cmd = ([B.hipcc()] + B.HIPCC_FLAGS + B.FILE_FLAGS.get("fa_fwd.hip", []) +
               ["--cuda-device-only", "-S", os.path.join(B.CSRC, "fa_fwd.hip"), "-o", out])
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return f.read()


# The head-dim-256 forward keeps O in AGPRs through assembly products too, and touches the
# accumulators with vector instructions in three places: zeroing (before the first
# product), the rare rescale of the running sums (between products) and the epilogue.  In
# the order the code is laid out, every such read must follow a long fence that comes after
# the last product, and every write must be followed by the short fence before the next
# product.
def test_head_dim_256_forward_fences_its_agpr_products(fwd_asm):
    bodies = _function_bodies(fwd_asm, "_ZN2fa20fwd_bf16_d256_kernel")
    assert len(bodies) == 3, list(bodies)  # unbiased, causal and general position bias
    for name, body in bodies.items():
        blocks = dict(_asm_blocks(body))
        n_products = 0
        last_product = ready_after = -1
        pending_write = False
        for i, line in enumerate(body):
            text = blocks.get(i)
            if text is not None and "v_mfma" in text:
                m = ASM_PRODUCT.search(text)
                assert m and m.group(1, 2) == m.group(3, 4), (name, text)
                assert not pending_write, (name, i, "product after an unfenced AGPR write")
                n_products += 1
                last_product = i
            elif text is not None and text.split() == ["s_nop", "7", "s_nop", "7", "s_nop", "7"]:
                ready_after = i
            elif text is not None and text.strip() == "s_nop 4":
                pending_write = False
            elif line.startswith("v_accvgpr_read"):
                assert ready_after > last_product, (name, i, "AGPR read without the long fence")
            elif line.startswith("v_accvgpr_write") or line.startswith("v_accvgpr_mov"):
                pending_write = True
        # 16 O^T products per step; the loop body holds two steps, the odd last step a third
        assert n_products == 48, (name, n_products)
        assert not pending_write, name
