"""Thin ctypes binding of libfa.so (argument marshalling only).

The functions named ``fa_*`` (``fa_fwd``, ``fa_fwd_alibi``, ``fa_fwd_fp32``, ``fa_bwd``,
``fa_bwd_workspace_size``, ...) mirror the C entry points of ``include/fa.h`` one to one,
in the same argument order; they take torch tensors only as carriers of device pointers and
of the current HIP stream.  ``forward`` / ``backward`` (and their packed-sequence and decoding
counterparts) check the tensors and allocate outputs for convenience.  Every step of the
computation runs in the HIP kernels of libfa.so: when the library is missing, loading raises
instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)

EXPORTED = ("fa_fwd", "fa_fwd_alibi", "fa_fwd_fp32", "fa_fwd_fp8", "fa_decode",
            "fa_decode_num_splits", "fa_decode_workspace_size", "fa_bwd", "fa_bwd_alibi",
            "fa_bwd_noalloc", "fa_bwd_workspace_size", "fa_fwd_varlen", "fa_fwd_varlen_alibi",
            "fa_bwd_varlen",
            "fa_bwd_varlen_alibi", "fa_bwd_varlen_workspace_size", "fa_bwd_time_main_kernel",
            "fa_mfma_probe", "fa_atomic_probe", "fa_issue_probe", "fa_fp8_product_probe", "fa_last_error",
            "fa_version")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfa status {status}: {message}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m exact_io_aware_fa2_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_alibi.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp]
    lib.fa_fwd_alibi.restype = i
    lib.fa_fwd_fp32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp32.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, f, f, f, i, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_alibi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp,
                                 sz, vp, vp]
    lib.fa_bwd_alibi.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_varlen_alibi.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, vp]
    lib.fa_fwd_varlen_alibi.restype = i
    lib.fa_bwd_varlen_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_varlen_workspace_size.restype = sz
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                  i, f, vp, sz, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_bwd_varlen_alibi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                        i, i, f, vp, sz, vp, vp]
    lib.fa_bwd_varlen_alibi.restype = i
    lib.fa_decode_num_splits.argtypes = [i, i, i, i, i, i, i]
    lib.fa_decode_num_splits.restype = i
    lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_decode_workspace_size.restype = sz
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode.restype = i
    lib.fa_bwd_time_main_kernel.argtypes = [vp, vp]
    lib.fa_bwd_time_main_kernel.restype = i
    lib.fa_mfma_probe.argtypes = [vp, i, i, vp]
    lib.fa_mfma_probe.restype = i
    lib.fa_atomic_probe.argtypes = [vp, i, i, i, i, vp]
    lib.fa_atomic_probe.restype = i
    lib.fa_issue_probe.argtypes = [vp, i, i, i, i, i, vp]
    lib.fa_issue_probe.restype = i
    lib.fa_fp8_product_probe.argtypes = [vp, vp, vp, i, vp]
    lib.fa_fp8_product_probe.restype = i
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, fa_last_error())


# ------------------------------------------------------------ 1:1 C entry points
def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, stream=None) -> int:
    return load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                         int(causal), int(window), float(scale), _stream(stream))


def fa_fwd_alibi(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, alibi_slopes,
                 stream=None) -> int:
    return load().fa_fwd_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                               int(causal), int(window), float(scale), _ptr(alibi_slopes),
                               _stream(stream))


def fa_fwd_fp8(q, k, v, o, lse, descale_q, descale_k, descale_v, B, Hq, Hkv, N, d, causal,
               window, scale, stream=None) -> int:
    return load().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), float(descale_q),
                             float(descale_k), float(descale_v), B, Hq, Hkv, N, d, int(causal),
                             int(window), float(scale), _stream(stream))


def fa_fwd_fp32(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, stream=None) -> int:
    return load().fa_fwd_fp32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                              int(causal), int(window), float(scale), _stream(stream))


def fa_bwd_workspace_size(B, Hq, Hkv, N, d, causal, window) -> int:
    return load().fa_bwd_workspace_size(B, Hq, Hkv, N, d, int(causal), int(window))


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale,
           workspace, workspace_bytes, stream=None) -> int:
    return load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq),
                         _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(causal), int(window),
                         float(scale), _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_bwd_alibi(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale,
                 workspace, workspace_bytes, alibi_slopes, stream=None) -> int:
    return load().fa_bwd_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(causal),
                               int(window), float(scale), _ptr(workspace),
                               int(workspace_bytes), _ptr(alibi_slopes), _stream(stream))


def fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale,
                   stream=None) -> int:
    return load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(causal),
                                 int(window), float(scale), _stream(stream))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, total, max_seqlen, Hq, Hkv, d, causal,
                  window, scale, stream=None) -> int:
    return load().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                                num_seqs, total, max_seqlen, Hq, Hkv, d, int(causal),
                                int(window), float(scale), _stream(stream))


def fa_fwd_varlen_alibi(q, k, v, o, lse, cu_seqlens, num_seqs, total, max_seqlen, Hq, Hkv, d,
                        causal, window, scale, alibi_slopes, stream=None) -> int:
    return load().fa_fwd_varlen_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _ptr(cu_seqlens), num_seqs, total, max_seqlen, Hq, Hkv, d,
                                      int(causal), int(window), float(scale),
                                      _ptr(alibi_slopes), _stream(stream))


def fa_bwd_varlen_workspace_size(total, Hq, Hkv, d) -> int:
    return load().fa_bwd_varlen_workspace_size(total, Hq, Hkv, d)


def fa_bwd_varlen(q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens, num_seqs, total, max_seqlen, Hq,
                  Hkv, d, causal, window, scale, workspace, workspace_bytes, stream=None) -> int:
    return load().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), num_seqs, total,
                                max_seqlen, Hq, Hkv, d, int(causal), int(window), float(scale),
                                _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa_bwd_varlen_alibi(q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens, num_seqs, total, max_seqlen,
                        Hq, Hkv, d, causal, window, scale, workspace, workspace_bytes,
                        alibi_slopes, stream=None) -> int:
    return load().fa_bwd_varlen_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), num_seqs,
                                      total, max_seqlen, Hq, Hkv, d, int(causal), int(window),
                                      float(scale), _ptr(workspace), int(workspace_bytes),
                                      _ptr(alibi_slopes), _stream(stream))


def fa_decode_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    return load().fa_decode_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    return load().fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fa_decode(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window,
              scale, num_splits, workspace, workspace_bytes, stream=None) -> int:
    return load().fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o),
                            _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal), int(window),
                            float(scale), int(num_splits), _ptr(workspace),
                            int(workspace_bytes), _stream(stream))


def fa_bwd_time_main_kernel(start_event, stop_event) -> int:
    """Ask the next fa_bwd on this thread to record the two torch.cuda.Event objects (or
    raw hipEvent_t handles) around its main kernel."""
    def handle(e):
        if e is None or isinstance(e, int):
            return e
        return e.cuda_event
    return load().fa_bwd_time_main_kernel(handle(start_event), handle(stop_event))


def fa_mfma_probe(out, blocks, iters, stream=None) -> int:
    return load().fa_mfma_probe(_ptr(out), int(blocks), int(iters), _stream(stream))


def fa_atomic_probe(acc, row_blocks, stride, blocks, iters, stream=None) -> int:
    return load().fa_atomic_probe(_ptr(acc), int(row_blocks), int(stride), int(blocks),
                                  int(iters), _stream(stream))


def fa_fp8_product_probe(a, bt, c, sets, stream=None) -> int:
    return load().fa_fp8_product_probe(_ptr(a), _ptr(bt), _ptr(c), int(sets), _stream(stream))


def fa_issue_probe(out, kind, param, waves_per_simd, blocks, iters, stream=None) -> int:
    return load().fa_issue_probe(_ptr(out), int(kind), int(param), int(waves_per_simd),
                                 int(blocks), int(iters), _stream(stream))


def fa_last_error() -> str:
    return load().fa_last_error().decode()


def fa_version() -> str:
    return load().fa_version().decode()


# ------------------------------------------------------------ tensor conveniences
def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [batch, seqlen, heads, headdim]")
    B, N, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k={tuple(k.shape)} v={tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    return B, N, Hq, k.shape[2], d


def _expect(t, name, shape, dtype, device):
    """A caller-supplied tensor must match what the kernels read or write: exact shape and
    dtype, contiguous, on the inputs' device (a smaller buffer would be overrun)."""
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous()
            or t.device != device):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}; got {tuple(t.shape)} {t.dtype} on {t.device}")
    return t


def _same_dtype_device(*ts):
    if any(t.dtype != ts[0].dtype for t in ts) or any(t.device != ts[0].device for t in ts):
        raise ValueError("q, k and v must share one dtype and one device")


def _slopes(alibi_slopes, Hq, device):
    """Check an optional ALiBi slope tensor: float32, contiguous, Hq values, on the inputs'
    device."""
    if alibi_slopes is None:
        return None
    t = alibi_slopes
    if (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()
            or t.numel() != Hq or t.device != device):
        raise ValueError(f"alibi_slopes must be a contiguous float32 tensor of {Hq} slopes "
                         f"(one per query head) on {device}")
    return t


def _device_buffer(t, name, device, nbytes=None):
    """A caller-supplied raw buffer (workspace): contiguous, on the inputs' device, and at
    least ``nbytes`` bytes when given.  The C layer checks only size and alignment, so a host
    tensor here would hand a host address to the kernels."""
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}; got "
                         f"{'contiguous' if t.is_contiguous() else 'non-contiguous'} on {t.device}")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")
    return t


def forward(q, k, v, causal=False, window=0, scale=None, out=None, lse=None, stream=None,
            alibi_slopes=None):
    """O, LSE = attention(q, k, v); bf16 or fp32 tensors in [B, N, H, d] layout."""
    B, N, Hq, Hkv, d = _shapes(q, k, v)
    _same_dtype_device(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.empty_like(q) if out is None else _expect(out, "out", q.shape, q.dtype, q.device)
    lse = (torch.empty((B, Hq, N), device=q.device, dtype=torch.float32) if lse is None
           else _expect(lse, "lse", (B, Hq, N), torch.float32, q.device))
    if q.dtype == torch.bfloat16:
        sl = _slopes(alibi_slopes, Hq, q.device)
        if sl is None:
            _check(fa_fwd(q, k, v, out, lse, B, Hq, Hkv, N, d, causal, window, scale, stream))
        else:
            _check(fa_fwd_alibi(q, k, v, out, lse, B, Hq, Hkv, N, d, causal, window, scale, sl,
                                stream))
    elif q.dtype == torch.float32:
        if alibi_slopes is not None:
            raise ValueError("the float32 forward has no position bias")
        _check(fa_fwd_fp32(q, k, v, out, lse, B, Hq, Hkv, N, d, causal, window, scale, stream))
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return out, lse


def forward_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal=False, window=0,
                scale=None, out=None, lse=None, stream=None):
    """O (bf16), LSE = attention of the dequantised E4M3 inputs [B, N, H, d] (uint8 or
    float8_e4m3fn tensors) with per-tensor factors descale_*."""
    for t in (q8, k8, v8):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"E4M3 codes expected (uint8 or float8_e4m3fn), got {t.dtype}")
    B, N, Hq, Hkv, d = _shapes(q8, k8, v8)
    if any(t.device != q8.device for t in (k8, v8)):
        raise ValueError("q, k and v must be on one device")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = (torch.empty((B, N, Hq, d), device=q8.device, dtype=torch.bfloat16) if out is None
           else _expect(out, "out", (B, N, Hq, d), torch.bfloat16, q8.device))
    lse = (torch.empty((B, Hq, N), device=q8.device, dtype=torch.float32) if lse is None
           else _expect(lse, "lse", (B, Hq, N), torch.float32, q8.device))
    _check(fa_fwd_fp8(q8, k8, v8, out, lse, descale_q, descale_k, descale_v, B, Hq, Hkv, N, d,
                      causal, window, scale, stream))
    return out, lse


def workspace_for(B, Hq, Hkv, N, d, causal, window, device) -> torch.Tensor:
    nbytes = fa_bwd_workspace_size(B, Hq, Hkv, N, d, causal, window)
    if nbytes == 0:
        raise FaError(FA_ERR_INVALID_ARG, fa_last_error())
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def backward(q, k, v, o, dO, lse, causal=False, window=0, scale=None, dq=None, dk=None,
             dv=None, workspace=None, stream=None, alibi_slopes=None):
    """dQ, dK, dV of L = sum(O * dO) for bf16 tensors."""
    B, N, Hq, Hkv, d = _shapes(q, k, v)
    _same_dtype_device(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError(f"the backward takes bfloat16 tensors, got {q.dtype}")
    dev = q.device
    _expect(o, "o", q.shape, q.dtype, dev)
    _expect(dO, "dO", q.shape, q.dtype, dev)
    _expect(lse, "lse", (B, Hq, N), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty_like(q) if dq is None else _expect(dq, "dq", q.shape, q.dtype, dev)
    dk = torch.empty_like(k) if dk is None else _expect(dk, "dk", k.shape, k.dtype, dev)
    dv = torch.empty_like(v) if dv is None else _expect(dv, "dv", v.shape, v.dtype, dev)
    sl = _slopes(alibi_slopes, Hq, dev)
    if workspace is None:
        workspace = workspace_for(B, Hq, Hkv, N, d, causal, window, q.device)
    _device_buffer(workspace, "workspace", dev)
    nbytes = workspace.numel() * workspace.element_size()
    if sl is None:
        _check(fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale,
                      workspace, nbytes, stream))
    else:
        _check(fa_bwd_alibi(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window,
                            scale, workspace, nbytes, sl, stream))
    return dq, dk, dv


def dvec_from_workspace(workspace: torch.Tensor, B: int, Hq: int, N: int) -> torch.Tensor:
    """View of D = rowsum(dO * O) ([B, Hq, N] float32) at the start of the workspace."""
    return workspace[: B * Hq * N * 4].view(torch.float32).view(B, Hq, N)


# ------------------------------------------------------------ packed sequences
def _shapes_varlen(q, k, v, cu_seqlens):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed q, k, v must be [total, heads, headdim]")
    T, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d:
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k={tuple(k.shape)} v={tuple(v.shape)}")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
    for t in (q, k, v, cu_seqlens):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on one device")
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"packed sequences take bfloat16 tensors, got {t.dtype}")
    return T, Hq, k.shape[1], d, cu_seqlens.numel() - 1


def forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, window=0, scale=None,
                   out=None, lse=None, stream=None, alibi_slopes=None):
    """O [total, Hq, d], LSE [Hq, total] for packed bf16 sequences."""
    T, Hq, Hkv, d, S = _shapes_varlen(q, k, v, cu_seqlens)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.empty_like(q) if out is None else _expect(out, "out", q.shape, q.dtype, q.device)
    lse = (torch.empty((Hq, T), device=q.device, dtype=torch.float32) if lse is None
           else _expect(lse, "lse", (Hq, T), torch.float32, q.device))
    sl = _slopes(alibi_slopes, Hq, q.device)
    if sl is None:
        _check(fa_fwd_varlen(q, k, v, out, lse, cu_seqlens, S, T, max_seqlen, Hq, Hkv, d, causal,
                             window, scale, stream))
    else:
        _check(fa_fwd_varlen_alibi(q, k, v, out, lse, cu_seqlens, S, T, max_seqlen, Hq, Hkv, d,
                                   causal, window, scale, sl, stream))
    return out, lse


def workspace_for_varlen(total, Hq, Hkv, d, device) -> torch.Tensor:
    nbytes = fa_bwd_varlen_workspace_size(total, Hq, Hkv, d)
    if nbytes == 0:
        raise FaError(FA_ERR_INVALID_ARG, fa_last_error())
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def backward_varlen(q, k, v, o, dO, lse, cu_seqlens, max_seqlen, causal=False, window=0,
                    scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None,
                    alibi_slopes=None):
    """dQ, dK, dV of L = sum(O * dO) for packed bf16 sequences."""
    T, Hq, Hkv, d, S = _shapes_varlen(q, k, v, cu_seqlens)
    dev = q.device
    _expect(o, "o", q.shape, q.dtype, dev)
    _expect(dO, "dO", q.shape, q.dtype, dev)
    _expect(lse, "lse", (Hq, T), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty_like(q) if dq is None else _expect(dq, "dq", q.shape, q.dtype, dev)
    dk = torch.empty_like(k) if dk is None else _expect(dk, "dk", k.shape, k.dtype, dev)
    dv = torch.empty_like(v) if dv is None else _expect(dv, "dv", v.shape, v.dtype, dev)
    sl = _slopes(alibi_slopes, Hq, dev)
    if workspace is None:
        workspace = workspace_for_varlen(T, Hq, Hkv, d, q.device)
    _device_buffer(workspace, "workspace", dev)
    nbytes = workspace.numel() * workspace.element_size()
    if sl is None:
        _check(fa_bwd_varlen(q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens, S, T, max_seqlen, Hq,
                             Hkv, d, causal, window, scale, workspace, nbytes, stream))
    else:
        _check(fa_bwd_varlen_alibi(q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens, S, T, max_seqlen,
                                   Hq, Hkv, d, causal, window, scale, workspace, nbytes, sl,
                                   stream))
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens_k=None, causal=True, window=0, scale=None,
           num_splits=0, out=None, lse=None, workspace=None, stream=None):
    """O [B, Nq, Hq, d] (bf16), LSE [B, Hq, Nq] of the newest Nq queries over a bf16 KV
    cache [B, Nk, Hkv, d]; seqlens_k: int32 device tensor [B] or None (all Nk)."""
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [B, Nq, Hq, d] and caches [B, Nk, Hkv, d] expected")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"shape mismatch q={tuple(q.shape)} cache={tuple(k_cache.shape)}")
    for t in (q, k_cache, v_cache):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q and the caches must be contiguous bf16 device tensors")
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or seqlens_k.numel() != B
                                  or not seqlens_k.is_cuda or seqlens_k.device != q.device
                                  or not seqlens_k.is_contiguous()):
        raise ValueError(f"seqlens_k must be a contiguous int32 tensor of B lengths on {q.device}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if any(t.device != q.device for t in (k_cache, v_cache)):
        raise ValueError("q and the caches must be on one device")
    out = torch.empty_like(q) if out is None else _expect(out, "out", q.shape, q.dtype, q.device)
    lse = (torch.empty((B, Hq, Nq), device=q.device, dtype=torch.float32) if lse is None
           else _expect(lse, "lse", (B, Hq, Nq), torch.float32, q.device))
    nbytes = fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _device_buffer(workspace, "workspace", q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fa_decode(q, k_cache, v_cache, seqlens_k, out, lse, B, Hq, Hkv, Nq, Nk, d, causal,
                     window, scale, num_splits, workspace, wbytes, stream))
    return out, lse
