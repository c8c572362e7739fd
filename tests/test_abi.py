"""C-ABI checks that need no GPU: the library loads, exports every declared entry point,
validates arguments before launching anything, and sizes its workspace linearly in N."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from exact_io_aware_fa2_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()),
                                reason="libfa.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.lib_path())
    declared = _declared_functions()
    assert set(declared) == set(fa.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_string():
    assert "gfx950" in fa.fa_version()


BAD_FWD = [
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(window=-2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 12, N=1 << 12, Hq=1 << 4, Hkv=1 << 4, d=128), fa.FA_ERR_INVALID_ARG),
    # exactly 2^31 elements: one row more than the largest accepted size
    (dict(B=2, N=1 << 20, Hq=8, Hkv=2, d=128), fa.FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("bad,status", BAD_FWD)
@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_fp32"])
def test_forward_validation(entry, bad, status):
    args = dict(B=1, Hq=2, Hkv=2, N=16, d=64, causal=0, window=0, scale=0.125)
    args.update(bad)
    fake = 256  # never dereferenced: validation fails before any launch
    fn = getattr(fa, entry)
    st = fn(fake, fake, fake, fake, fake, args["B"], args["Hq"], args["Hkv"], args["N"],
            args["d"], args["causal"], args["window"], args["scale"], stream=0)
    assert st == status
    assert fa.fa_last_error().startswith(entry)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_fp32"])
def test_forward_null_pointer(entry):
    st = getattr(fa, entry)(None, 256, 256, 256, 256, 1, 1, 1, 8, 64, 0, 0, 0.1, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG
    assert "null" in fa.fa_last_error()


def test_backward_validation_and_workspace():
    fake = 256
    base = (1, 4, 2, 128, 128, 1, 0)
    need = fa.fa_bwd_workspace_size(*base)
    assert need > 0
    # too small a workspace is rejected before launch
    st = fa.fa_bwd(fake, fake, fake, fake, fake, fake, fake, fake, fake, 1, 4, 2, 128, 128, 1, 0,
                   0.1, 4096, need - 1, stream=0)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.fa_bwd(fake, fake, fake, fake, fake, fake, fake, fake, fake, 1, 4, 2, 128, 128, 1, 0,
                   0.1, None, need, stream=0)
    assert st == fa.FA_ERR_WORKSPACE
    # misaligned workspace
    st = fa.fa_bwd(fake, fake, fake, fake, fake, fake, fake, fake, fake, 1, 4, 2, 128, 128, 1, 0,
                   0.1, 4096 + 16, need, stream=0)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.fa_bwd(fake, fake, fake, fake, None, fake, fake, fake, fake, 1, 4, 2, 128, 128, 1, 0,
                   0.1, 4096, need, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG
    st = fa.fa_bwd(fake, fake, fake, fake, fake, fake, fake, fake, fake, 1, 4, 3, 128, 128, 1, 0,
                   0.1, 4096, need, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_workspace_size(1, 4, 3, 128, 128, 1, 0) == 0


def test_workspace_linear_in_n():
    sizes = [fa.fa_bwd_workspace_size(2, 8, 2, n, 128, 1, 0) for n in (1024, 2048, 4096)]
    # D only: B*Hq*N float32, rounded up to 256 bytes
    for n, s in zip((1024, 2048, 4096), sizes):
        assert s == ((2 * 8 * n * 4 + 255) // 256) * 256
    assert sizes[2] - sizes[1] == 2 * (sizes[1] - sizes[0])
    assert fa.fa_bwd_workspace_size(1, 1, 1, 3, 64, 0, 0) == 256


def test_mfma_probe_validation():
    # argument checks happen before any launch, so no GPU is touched
    assert fa.fa_mfma_probe(None, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_mfma_probe(1 << 20, 0, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_mfma_probe(1 << 20, 4, -1, stream=0) == fa.FA_ERR_INVALID_ARG


def test_atomic_probe_validation():
    assert fa.fa_atomic_probe(None, 8, 4096, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_atomic_probe(1 << 20, 0, 4096, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_atomic_probe(1 << 20, 8, 64, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_atomic_probe(1 << 20, 8, 4096, 4, 0, stream=0) == fa.FA_ERR_INVALID_ARG
    # 2^31 floats would not be addressable with the kernel's 32-bit row arithmetic
    assert fa.fa_atomic_probe(1 << 20, 1 << 14, 4096, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert "2^31" in fa.fa_last_error()


def test_issue_probe_validation():
    # every rejection happens before a launch (no GPU here)
    assert fa.fa_issue_probe(None, 0, 4, 2, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    for kind, param in ((0, 3), (1, 0), (2, 3), (3, 3), (4, 0), (-1, 0)):
        assert fa.fa_issue_probe(1 << 20, kind, param, 2, 4, 4, stream=0) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_issue_probe(1 << 20, 0, 4, 3, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_issue_probe(1 << 20, 0, 4, 0, 4, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_issue_probe(1 << 20, 0, 4, 2, 0, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_issue_probe(1 << 20, 0, 4, 2, 4, 0, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_last_error().startswith("fa_issue_probe")
    # global-operand probes read a 32 KiB window of `out` per workgroup
    assert fa.fa_issue_probe(1 << 20, 6, 4, 2, 256, 4, stream=0) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_issue_probe(1 << 20, 6, 2, 1, 31, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_issue_probe(1 << 20, 6, 2, 2, 15, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    # LDS bank probes: width * 10000 + stride, width in {4, 8, 16}, stride in [1, 4096]
    for kind in (4, 5):
        for param in (0, 30128, 40000, 44097, 20008, -40004):
            assert fa.fa_issue_probe(1 << 20, kind, param, 1, 4, 4, stream=0) == fa.FA_ERR_UNSUPPORTED


def test_fp8_product_probe_validation():
    good = 1 << 20
    assert fa.fa_fp8_product_probe(None, good, good, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fp8_product_probe(good, None, good, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fp8_product_probe(good, good, None, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fp8_product_probe(good, good, good, 0, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fp8_product_probe(good, good, good, 1 << 20, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fp8_product_probe(good + 8, good, good, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fp8_product_probe(good, good, good + 2, 4, stream=0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_last_error().startswith("fa_fp8_product_probe")


BAD_VARLEN = [
    (dict(cu=None), fa.FA_ERR_INVALID_ARG),
    (dict(num_seqs=0), fa.FA_ERR_INVALID_ARG),
    (dict(total=0), fa.FA_ERR_INVALID_ARG),
    (dict(max_seqlen=0), fa.FA_ERR_INVALID_ARG),
    (dict(max_seqlen=65), fa.FA_ERR_INVALID_ARG),  # longer than the packed rows
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(window=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(num_seqs=1 << 20, total=1 << 20, max_seqlen=1 << 20, Hq=64, Hkv=64),
     fa.FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("bad,status", BAD_VARLEN)
@pytest.mark.parametrize("entry", ["fa_fwd_varlen", "fa_bwd_varlen"])
def test_varlen_validation(entry, bad, status):
    a = dict(cu=256, num_seqs=3, total=64, max_seqlen=40, Hq=4, Hkv=2, d=128, causal=1,
             window=0, scale=0.1)
    a.update(bad)
    fake = 256
    common = (a["cu"], a["num_seqs"], a["total"], a["max_seqlen"], a["Hq"], a["Hkv"], a["d"],
              a["causal"], a["window"], a["scale"])
    if entry == "fa_fwd_varlen":
        st = fa.fa_fwd_varlen(fake, fake, fake, fake, fake, *common, stream=0)
    else:
        st = fa.fa_bwd_varlen(fake, fake, fake, fake, fake, fake, fake, fake, fake, *common,
                              4096, 1 << 30, stream=0)
    assert st == status
    assert fa.fa_last_error().startswith(entry)


def test_varlen_workspace():
    # D only: Hq * total float32, rounded up to 256 bytes
    assert fa.fa_bwd_varlen_workspace_size(1000, 8, 2, 128) == ((8 * 1000 * 4 + 255) // 256) * 256
    assert fa.fa_bwd_varlen_workspace_size(0, 8, 2, 128) == 0
    assert fa.fa_bwd_varlen_workspace_size(64, 6, 4, 128) == 0
    assert fa.fa_bwd_varlen_workspace_size(64, 4, 4, 96) == 0
    fake = 256
    need = fa.fa_bwd_varlen_workspace_size(64, 4, 2, 128)
    args = (fake, 3, 64, 40, 4, 2, 128, 1, 0, 0.1)
    st = fa.fa_bwd_varlen(*([fake] * 9), *args, 4096, need - 1, stream=0)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.fa_bwd_varlen(*([fake] * 9), *args, 4096 + 64, need, stream=0)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.fa_bwd_varlen(*([fake] * 9), *args, None, need, stream=0)
    assert st == fa.FA_ERR_WORKSPACE
    st = fa.fa_fwd_varlen(None, *([fake] * 4), *args, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG and "null" in fa.fa_last_error()


@pytest.mark.parametrize("bad,status", BAD_FWD + [
    (dict(dq=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(dv=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(dq=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(dq=1e30, dk=1e30), fa.FA_ERR_INVALID_ARG),
])
def test_fp8_forward_validation(bad, status):
    a = dict(B=1, Hq=2, Hkv=2, N=16, d=64, causal=0, window=0, scale=0.125, dq=0.1, dk=0.1,
             dv=0.1)
    a.update(bad)
    fake = 256
    st = fa.fa_fwd_fp8(fake, fake, fake, fake, fake, a["dq"], a["dk"], a["dv"], a["B"], a["Hq"],
                       a["Hkv"], a["N"], a["d"], a["causal"], a["window"], a["scale"], stream=0)
    assert st == status
    assert fa.fa_last_error().startswith("fa_fwd_fp8")
    st = fa.fa_fwd_fp8(None, fake, fake, fake, fake, 1.0, 1.0, 1.0, 1, 1, 1, 8, 64, 0, 0, 0.1,
                       stream=0)
    assert st == fa.FA_ERR_INVALID_ARG and "null" in fa.fa_last_error()


def test_decode_validation_and_splits():
    fake = 256
    base = dict(B=2, Hq=8, Hkv=2, Nq=1, Nk=4096, d=128)
    ns = fa.fa_decode_num_splits(*base.values(), 0)
    assert ns >= 1
    assert fa.fa_decode_num_splits(*base.values(), 5) == 5
    assert fa.fa_decode_num_splits(2, 8, 2, 1, 4096, 256, 0) == 0  # d = 256 unsupported
    assert fa.fa_decode_workspace_size(*base.values(), 1) == 0
    need = fa.fa_decode_workspace_size(*base.values(), 4)
    rows = 4 * 2 * 8 * 1
    assert need == ((rows * 128 * 4 + 255) // 256) * 256 + ((rows * 4 + 255) // 256) * 256

    def call(**kw):
        a = dict(base, causal=1, window=0, scale=0.1, num_splits=4, ws=4096, wsb=need)
        a.update(kw)
        return fa.fa_decode(fake, fake, fake, None, fake, fake, a["B"], a["Hq"], a["Hkv"],
                            a["Nq"], a["Nk"], a["d"], a["causal"], a["window"], a["scale"],
                            a["num_splits"], a["ws"], a["wsb"], stream=0)

    assert call(Nq=0) == fa.FA_ERR_INVALID_ARG
    assert call(Hq=6, Hkv=4) == fa.FA_ERR_INVALID_ARG
    assert call(d=256) == fa.FA_ERR_UNSUPPORTED
    assert call(num_splits=-1) == fa.FA_ERR_INVALID_ARG
    assert call(num_splits=257) == fa.FA_ERR_INVALID_ARG
    assert call(wsb=need - 1) == fa.FA_ERR_WORKSPACE
    assert call(ws=4096 + 8) == fa.FA_ERR_WORKSPACE
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(window=-1) == fa.FA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_last_error().startswith("fa_decode")
    st = fa.fa_decode(None, fake, fake, None, fake, fake, 1, 1, 1, 1, 8, 64, 1, 0, 0.1, 1, None,
                      0, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG and "null" in fa.fa_last_error()


# Alignment: tensor pointers 16 bytes, row statistics and side arrays 4 bytes.  Each call
# passes one misaligned pointer (all others aligned fakes, never dereferenced).
_A = 256


def _misaligned_calls(t16, t4):
    A = _A
    return {
        "fa_fwd": lambda: fa.fa_fwd(t16, A, A, A, t4, 1, 2, 2, 16, 64, 0, 0, 0.125, stream=0),
        "fa_fwd_fp32": lambda: fa.fa_fwd_fp32(t16, A, A, A, t4, 1, 2, 2, 16, 64, 0, 0, 0.125,
                                              stream=0),
        "fa_fwd_fp8": lambda: fa.fa_fwd_fp8(A, t16, A, A, t4, 1.0, 1.0, 1.0, 1, 2, 2, 16, 64, 0,
                                            0, 0.125, stream=0),
        "fa_bwd": lambda: fa.fa_bwd(A, A, A, A, A, t4, A, A, t16, 1, 2, 2, 16, 64, 0, 0, 0.125,
                                    A, 1 << 20, stream=0),
        "fa_fwd_alibi": lambda: fa.fa_fwd_alibi(A, t16, A, A, A, 1, 2, 2, 16, 64, 1, 0, 0.125,
                                                t4, stream=0),
        "fa_bwd_alibi": lambda: fa.fa_bwd_alibi(A, A, A, t16, A, A, A, A, A, 1, 2, 2, 16, 64, 1,
                                                0, 0.125, A, 1 << 20, t4, stream=0),
        "fa_fwd_varlen": lambda: fa.fa_fwd_varlen(A, A, t16, A, t4, A, 1, 16, 16, 2, 2, 64, 0, 0,
                                                  0.125, stream=0),
        "fa_fwd_varlen_alibi": lambda: fa.fa_fwd_varlen_alibi(A, A, A, t16, A, A, 1, 16, 16, 2,
                                                              2, 64, 0, 0, 0.125, t4, stream=0),
        "fa_bwd_varlen_alibi": lambda: fa.fa_bwd_varlen_alibi(A, A, A, A, A, A, t16, A, A, t4, 1,
                                                              16, 16, 2, 2, 64, 0, 0, 0.125, A,
                                                              1 << 20, A, stream=0),
        "fa_bwd_varlen": lambda: fa.fa_bwd_varlen(A, A, A, A, t16, t4, A, A, A, A, 1, 16, 16, 2,
                                                  2, 64, 0, 0, 0.125, A, 1 << 20, stream=0),
        "fa_decode": lambda: fa.fa_decode(A, A, t16, None, A, t4, 1, 2, 2, 1, 16, 64, 1, 0, 0.125,
                                          1, None, 0, stream=0),
    }


@pytest.mark.parametrize("entry", sorted(_misaligned_calls(_A, _A)))
@pytest.mark.parametrize("t16,t4", [(_A + 8, _A), (_A, _A + 2)], ids=["tensor+8", "stats+2"])
def test_misaligned_pointers_are_rejected(entry, t16, t4):
    st = _misaligned_calls(t16, t4)[entry]()
    assert st == fa.FA_ERR_INVALID_ARG
    assert "aligned" in fa.fa_last_error()



def test_python_buffer_checks():
    import torch
    t = torch.empty(2, 3, dtype=torch.float32)
    assert fa._expect(t, "x", (2, 3), torch.float32, t.device) is t
    with pytest.raises(ValueError, match="shape"):
        fa._expect(t, "x", (3, 2), torch.float32, t.device)
    with pytest.raises(ValueError):
        fa._expect(t, "x", (2, 3), torch.bfloat16, t.device)
    with pytest.raises(ValueError):
        fa._expect(t.t(), "x", (3, 2), torch.float32, t.device)  # not contiguous
    with pytest.raises(ValueError, match="one dtype"):
        fa._same_dtype_device(t, t.to(torch.bfloat16))


@pytest.mark.parametrize("entry", ["fa_fwd_alibi", "fa_bwd_alibi", "fa_fwd_varlen_alibi",
                                   "fa_bwd_varlen_alibi"])
def test_alibi_entry_points_need_slopes(entry):
    A = _A
    calls = {
        "fa_fwd_alibi": lambda s: fa.fa_fwd_alibi(A, A, A, A, A, 1, 2, 2, 16, 64, 1, 0, 0.125, s,
                                                  stream=0),
        "fa_bwd_alibi": lambda s: fa.fa_bwd_alibi(A, A, A, A, A, A, A, A, A, 1, 2, 2, 16, 64, 1,
                                                  0, 0.125, A, 1 << 20, s, stream=0),
        "fa_fwd_varlen_alibi": lambda s: fa.fa_fwd_varlen_alibi(A, A, A, A, A, A, 1, 16, 16, 2,
                                                                2, 64, 1, 0, 0.125, s, stream=0),
        "fa_bwd_varlen_alibi": lambda s: fa.fa_bwd_varlen_alibi(A, A, A, A, A, A, A, A, A, A, 1,
                                                                16, 16, 2, 2, 64, 1, 0, 0.125, A,
                                                                1 << 20, s, stream=0),
    }
    assert calls[entry](None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_last_error().startswith(entry) and "alibi_slopes" in fa.fa_last_error()
    # the other checks still run first on a call that has its slopes
    assert calls[entry](A + 2) == fa.FA_ERR_INVALID_ARG and "aligned" in fa.fa_last_error()


def test_python_workspace_and_slope_checks():
    """The binding rejects a host workspace (its address would reach the kernels), a
    non-contiguous one, and slopes that are not on the inputs' device."""
    import torch
    dev = torch.device("cuda", 0)  # a device object only: nothing is allocated on it
    host = torch.empty(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace must be a contiguous tensor on cuda:0"):
        fa._device_buffer(host, "workspace", dev)
    with pytest.raises(ValueError, match="non-contiguous"):
        fa._device_buffer(host[::2], "workspace", dev)
    assert fa._slopes(None, 4, dev) is None
    with pytest.raises(ValueError, match="alibi_slopes"):
        fa._slopes(torch.ones(4), 4, dev)


def _cc():
    return shutil.which("gcc") or shutil.which("cc")


@pytest.mark.skipif(_cc() is None, reason="no C compiler")
def test_c_caller_compiled_against_the_header(tmp_path):
    """A plain C program built against include/fa.h: the contract prototypes, written out on
    their own, must accept every library function (a mismatch fails the build), and every
    rejected call returns its status through the C ABI."""
    src = os.path.join(ROOT, "tests", "abi_caller.c")
    pkg = os.path.dirname(fa.lib_path())
    cmd = [_cc(), "-std=c11", "-Wall", "-Werror=incompatible-pointer-types",
           "-I", os.path.join(ROOT, "include"), None, "-L", pkg, "-l:libfa.so",
           f"-Wl,-rpath,{pkg}", "-Wl,-rpath-link,/opt/rocm/lib", "-o", None]
    exe = str(tmp_path / "abi_caller")
    build = subprocess.run([src if c is None and i < 8 else exe if c is None else c
                            for i, c in enumerate(cmd)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "abi_caller ok" in run.stdout, run.stdout + run.stderr
    # the prototype pin bites: a caller that expects the bias argument in fa_fwd does not build
    text = open(src).read()
    bad = text.replace("int, int, int, int, float, void*);\ntypedef fa_status (*fwd_fp32_fn)",
                       "int, int, int, int, float, const float*, void*);\n"
                       "typedef fa_status (*fwd_fp32_fn)", 1)
    assert bad != text
    bad_src = tmp_path / "bad_caller.c"
    bad_src.write_text(bad)
    res = subprocess.run([str(bad_src) if c is None and i < 8 else exe + "_bad" if c is None
                          else c for i, c in enumerate(cmd)], capture_output=True, text=True)
    assert res.returncode != 0 and "incompatible" in res.stderr


def _hipcc():
    c = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return c if os.path.exists(c) else None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_api_layer_under_host_sanitizers(tmp_path):
    """fa_api.hip's validation and argument marshalling built for the host with
    AddressSanitizer and UndefinedBehaviorSanitizer (device code is not built), linked with
    launchers that record their arguments instead of launching: valid calls must derive the
    right launch arguments, rejected calls (including int sizes whose products overflow
    64 bits) must launch nothing, and no sanitizer may fire."""
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    base = [_hipcc(), "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17"]
    objs = []
    for src, extra in ((os.path.join(ROOT, "exact_io_aware_fa2_amd", "csrc", "fa_api.hip"), []),
                       (os.path.join(ROOT, "tests", "native", "stub_launchers.cpp"), ["-x", "hip"]),
                       (os.path.join(ROOT, "tests", "native", "api_sanitize.cpp"), ["-x", "hip"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run(base + extra + san + ["-c", src, "-o", obj], capture_output=True,
                             text=True)
        assert res.returncode == 0, res.stderr
        objs.append(obj)
    exe = str(tmp_path / "api_sanitize")
    res = subprocess.run([_hipcc()] + san + objs + ["-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and "api_sanitize ok" in run.stdout, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr


def test_library_never_allocates_frees_or_synchronises():
    """The memory claim of the boundary (every buffer is the caller's; the backward keeps
    O(N) state in the caller's workspace, ainews.cool "flash-attention transformer
    optimization", technical deep dive, memory table): libfa.so imports no HIP allocation,
    free or synchronisation routine at all."""
    nm = shutil.which("nm") or shutil.which("llvm-nm")
    if nm is None:
        pytest.skip("nm not found")
    out = subprocess.run([nm, "-D", "--undefined-only", fa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    hip = sorted(n for n in imported if n.startswith("hip"))
    assert "hipGetLastError" in hip  # the scan sees the HIP imports at all
    banned = [n for n in hip if re.match(r"hip(Malloc|Free|HostAlloc|HostMalloc|ExtMalloc|"
                                         r"MallocAsync|MemPool|DeviceSynchronize|"
                                         r"StreamSynchronize|EventSynchronize|Memcpy(?!ToSymbol))", n)]
    assert banned == [], banned
