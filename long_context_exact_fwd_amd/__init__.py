"""MI355X (gfx950) exact long-context attention: Python binding of libmi355attn.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``. PyTorch supplies
device memory and the current stream. The binding raises if the compiled
library is missing; there is no fallback implementation.

    o, lse = fwd(q, k, v, causal=True)                       # bf16 [B,S,H,D]
    o, lse = fwd_fp8(q8, k8, v8, dq, dk, dv, causal=True)    # uint8 E4M3 codes
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    dq, dk, dv = bwd_fp8(q8, k8, v8, ds_q, ds_k, ds_v, o, lse, do, causal=True)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmi355attn.so")
# Same C ABI, built with -DATTN_DEBUG: LDS accesses bounds-checked on the
# device and a synchronising check after every call (ATTN_ERR_DEBUG_CHECK).
DEBUG_LIB_PATH = os.path.join(_PKG, "libmi355attn_debug.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARGUMENT = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_HIP = 3
ATTN_ERR_SCRATCH_TOO_SMALL = 4
ATTN_ERR_DEBUG_CHECK = 5
NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_NOALLOC_SCRATCH_BYTES in include/attn.h

_lib = None
_lib_path = LIB_PATH  # the library load_library() opens: release, or debug after use_debug_library()


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmi355attn.so and declare the C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _lib_path
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m long_context_exact_fwd_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_fwd.restype = i
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_fwd_fp8.restype = i
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_bwd.restype = i
    lib.attn_bwd_phases.argtypes = [ctypes.c_uint, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i,
                                    f, st]
    lib.attn_bwd_phases.restype = i
    lib.attn_bwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_bwd_fp8.restype = i
    lib.attn_bwd_fp8_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_fp8_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_bwd_noalloc.restype = i
    lib.attn_merge.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, st]
    lib.attn_merge.restype = i
    lib.attn_fwd_merge.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_fwd_merge.restype = i
    lib.attn_fwd_fp8_merge.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_fwd_fp8_merge.restype = i
    lib.attn_bwd_accumulate.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, vp, i, f, st]
    lib.attn_bwd_accumulate.restype = i
    lib.attn_fwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_status_str.argtypes = [i]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = i
    if path is None:
        _lib = lib
    return lib


def use_debug_library(debug: bool = True) -> None:
    """Route every later call of this module through libmi355attn_debug.so (or back to libmi355attn.so).
    The library is loaded by the next call, as the release one is by the first."""
    global _lib, _lib_path
    _lib_path = DEBUG_LIB_PATH if debug else LIB_PATH
    _lib = None


EXPORTED = ("attn_fwd", "attn_fwd_workspace_bytes", "attn_fwd_fp8", "attn_bwd", "attn_bwd_phases",
            "attn_bwd_workspace_bytes", "attn_bwd_fp8", "attn_bwd_fp8_workspace_bytes", "attn_bwd_noalloc",
            "attn_merge", "attn_fwd_merge", "attn_fwd_fp8_merge", "attn_bwd_accumulate", "attn_status_str",
            "attn_last_hip_error")

BWD_DELTA, BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 4, 7


def bf16_from_bits(bits, device="cuda"):
    """Device bfloat16 tensor from a numpy array of bf16 bit patterns (uint16)."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(device)


def _check(status: int, what: str) -> None:
    if status != ATTN_OK:
        lib = load_library()
        name = lib.attn_status_str(status).decode()
        extra = f" (hipError {lib.attn_last_hip_error()})" if status == ATTN_ERR_HIP else ""
        raise AttnError(status, f"{what}: {name}{extra}")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _shape(q, k, v, cu_seqlens):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, S, H, D]")
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError("k/v shape must be [B, S, Hkv, D] with q's B, S, D")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must have the shape of k")
    n = 0
    if cu_seqlens is not None:
        import torch
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
        n = cu_seqlens.numel() - 1
    return B, S, Hq, Hkv, D, n


def _expect(t, shape, dtype, what):
    """A tensor the library reads or writes through a bare pointer: its size is fixed by the call's sizes."""
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous {dtype} device tensor of shape {tuple(shape)}, "
                         f"got {tuple(t.shape)} {t.dtype}")


def _check_descales(*ts):
    for t in ts:
        if t.numel() < 1:
            raise ValueError("descales must hold one float32 element each")


def _check_tensors(*ts, dtype=None):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"expected {dtype}, got {t.dtype}")


def fwd_workspace_bytes(batch: int, hq: int, hkv: int, seqlen: int, head_dim: int) -> int:
    return int(load_library().attn_fwd_workspace_bytes(batch, hq, hkv, seqlen, head_dim))


def fwd(q, k, v, *, causal: bool, cu_seqlens=None, scale: Optional[float] = None, out=None, lse=None,
        workspace=None, split: bool = True):
    """Forward, bf16. Returns (o [B,S,Hq,D] bf16, lse [B,Hq,S] fp32).

    When attn_fwd_workspace_bytes() is above 0 for these sizes, a workspace is
    allocated (or ``workspace`` is used) so the library can split key ranges;
    ``split=False`` passes no workspace.
    """
    import torch
    _check_tensors(q, k, v, dtype=torch.bfloat16)
    B, S, Hq, Hkv, D, n = _shape(q, k, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty_like(q)
    l_ = lse if lse is not None else torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _expect(o, (B, S, Hq, D), torch.bfloat16, "out")
    _expect(l_, (B, Hq, S), torch.float32, "lse")
    ws = _fwd_workspace(B, Hq, Hkv, S, D, q.device, workspace, split)
    st = load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l_), _ptr(ws), B, Hq, Hkv, S, D,
                                 int(bool(causal)), _ptr(cu_seqlens), n, float(scale), _stream())
    _check(st, "attn_fwd")
    return o, l_


def _fwd_workspace(B, Hq, Hkv, S, D, device, workspace, split):
    """The key-split workspace for a forward call, or None (marshalling only)."""
    import torch
    nbytes = fwd_workspace_bytes(B, Hq, Hkv, S, D) if split else 0
    if nbytes == 0:
        return None
    if workspace is None:
        return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device)
    if workspace.is_contiguous() and workspace.numel() * workspace.element_size() >= nbytes \
            and workspace.device == device:
        return workspace
    raise ValueError(f"workspace must be a contiguous tensor of at least {nbytes} bytes on {device}")


def fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, *, causal: bool, cu_seqlens=None,
            scale: Optional[float] = None, out=None, lse=None, workspace=None, split: bool = True):
    """Forward with E4M3FN codes (uint8 tensors) and fp32 device descales (1 element each).

    ``workspace`` and ``split`` work as in fwd().
    """
    import torch
    _check_tensors(q8, k8, v8, dtype=torch.uint8)
    _check_tensors(descale_q, descale_k, descale_v, dtype=torch.float32)
    B, S, Hq, Hkv, D, n = _shape(q8, k8, v8, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_descales(descale_q, descale_k, descale_v)
    o = out if out is not None else torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=q8.device)
    l_ = lse if lse is not None else torch.empty((B, Hq, S), dtype=torch.float32, device=q8.device)
    _expect(o, (B, S, Hq, D), torch.bfloat16, "out")
    _expect(l_, (B, Hq, S), torch.float32, "lse")
    ws = _fwd_workspace(B, Hq, Hkv, S, D, q8.device, workspace, split) if D == 128 else None
    st = load_library().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale_q), _ptr(descale_k),
                                     _ptr(descale_v), _ptr(o), _ptr(l_), _ptr(ws), B, Hq, Hkv, S, D,
                                     int(bool(causal)), _ptr(cu_seqlens), n, float(scale), _stream())
    _check(st, "attn_fwd_fp8")
    return o, l_


def merge(o_acc, lse_acc, o_part, lse_part, *, accumulate: bool = True, o_out=None):
    """Ring-Attention step: merge (o_part bf16, lse_part) into (o_acc fp32, lse_acc) in place.

    o_acc/o_part/o_out [B,S,H,D]; lse_acc/lse_part [B,H,S] fp32. With
    accumulate=False the running result is treated as empty. o_out (bf16) also
    receives the merged output if given. Returns (o_acc, lse_acc).
    """
    import torch
    _check_tensors(o_acc, lse_acc, lse_part, dtype=torch.float32)
    _check_tensors(o_part, dtype=torch.bfloat16)
    if o_acc.dim() != 4 or tuple(o_part.shape) != tuple(o_acc.shape):
        raise ValueError("o_acc and o_part must both be [B, S, H, D]")
    B, S, H, D = o_acc.shape
    for t in (lse_acc, lse_part):
        if tuple(t.shape) != (B, H, S):
            raise ValueError("lse_acc and lse_part must be [B, H, S]")
    if o_out is not None:
        _check_tensors(o_out, dtype=torch.bfloat16)
        if tuple(o_out.shape) != (B, S, H, D):
            raise ValueError("o_out must be [B, S, H, D]")
    st = load_library().attn_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), _ptr(o_out), B, S, H,
                                   D, int(bool(accumulate)), _stream())
    _check(st, "attn_merge")
    return o_acc, lse_acc


def fwd_merge(q, k, v, o_acc, lse_acc, *, causal: bool, accumulate: bool = True, o_out=None, cu_seqlens=None,
              scale: Optional[float] = None, workspace=None, split: bool = True):
    """Ring-Attention step fused into the forward: attention of q over (k, v) merged into (o_acc, lse_acc) in place.

    o_acc [B,S,Hq,D] fp32, lse_acc [B,Hq,S] fp32; accumulate=False treats them
    as empty. o_out (bf16 [B,S,Hq,D]) also receives the merged output if given.
    ``workspace`` and ``split`` work as in fwd(). Returns (o_acc, lse_acc).
    """
    import torch
    _check_tensors(q, k, v, dtype=torch.bfloat16)
    _check_tensors(o_acc, lse_acc, dtype=torch.float32)
    B, S, Hq, Hkv, D, n = _shape(q, k, v, cu_seqlens)
    if tuple(o_acc.shape) != (B, S, Hq, D) or tuple(lse_acc.shape) != (B, Hq, S):
        raise ValueError("o_acc must be [B, S, Hq, D] and lse_acc [B, Hq, S]")
    if o_out is not None:
        _check_tensors(o_out, dtype=torch.bfloat16)
        if tuple(o_out.shape) != (B, S, Hq, D):
            raise ValueError("o_out must be [B, S, Hq, D]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws = _fwd_workspace(B, Hq, Hkv, S, D, q.device, workspace, split)
    st = load_library().attn_fwd_merge(_ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(lse_acc), _ptr(o_out),
                                       int(bool(accumulate)), _ptr(ws), B, Hq, Hkv, S, D, int(bool(causal)),
                                       _ptr(cu_seqlens), n, float(scale), _stream())
    _check(st, "attn_fwd_merge")
    return o_acc, lse_acc


def fwd_fp8_merge(q8, k8, v8, descale_q, descale_k, descale_v, o_acc, lse_acc, *, causal: bool,
                  accumulate: bool = True, o_out=None, cu_seqlens=None, scale: Optional[float] = None, workspace=None,
                  split: bool = True):
    """fwd_merge for the fp8 forward: E4M3 codes (uint8) with fp32 device descales; o_acc, lse_acc updated in place."""
    import torch
    _check_tensors(q8, k8, v8, dtype=torch.uint8)
    _check_tensors(descale_q, descale_k, descale_v, o_acc, lse_acc, dtype=torch.float32)
    _check_descales(descale_q, descale_k, descale_v)
    B, S, Hq, Hkv, D, n = _shape(q8, k8, v8, cu_seqlens)
    if tuple(o_acc.shape) != (B, S, Hq, D) or tuple(lse_acc.shape) != (B, Hq, S):
        raise ValueError("o_acc must be [B, S, Hq, D] and lse_acc [B, Hq, S]")
    if o_out is not None:
        _check_tensors(o_out, dtype=torch.bfloat16)
        if tuple(o_out.shape) != (B, S, Hq, D):
            raise ValueError("o_out must be [B, S, Hq, D]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws = _fwd_workspace(B, Hq, Hkv, S, D, q8.device, workspace, split) if D == 128 else None
    st = load_library().attn_fwd_fp8_merge(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale_q), _ptr(descale_k),
                                           _ptr(descale_v), _ptr(o_acc), _ptr(lse_acc), _ptr(o_out),
                                           int(bool(accumulate)), _ptr(ws), B, Hq, Hkv, S, D, int(bool(causal)),
                                           _ptr(cu_seqlens), n, float(scale), _stream())
    _check(st, "attn_fwd_fp8_merge")
    return o_acc, lse_acc


def bwd_workspace_bytes(batch: int, hq: int, hkv: int, seqlen: int, head_dim: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(batch, hq, hkv, seqlen, head_dim))


def _bwd_operands(o, lse, do, B, S, Hq, D):
    import torch
    _expect(o, (B, S, Hq, D), torch.bfloat16, "o")
    _expect(do, (B, S, Hq, D), torch.bfloat16, "do")
    _expect(lse, (B, Hq, S), torch.float32, "lse")


def _bwd_outputs(dq, dk, dv, B, S, Hq, Hkv, D, dtype):
    _expect(dq, (B, S, Hq, D), dtype, "dq")
    _expect(dk, (B, S, Hkv, D), dtype, "dk")
    _expect(dv, (B, S, Hkv, D), dtype, "dv")


def bwd(q, k, v, o, lse, do, *, causal: bool, cu_seqlens=None, scale: Optional[float] = None, workspace=None,
        dq=None, dk=None, dv=None, phases: Optional[int] = None):
    """Backward, bf16. Returns (dq, dk, dv) shaped like q, k, v.

    ``phases`` (bitmask of BWD_DELTA, BWD_DKDV, BWD_DQ) runs only those kernels
    through attn_bwd_phases; the default runs attn_bwd (all three).
    """
    import torch
    _check_tensors(q, k, v, o, do, dtype=torch.bfloat16)
    _check_tensors(lse, dtype=torch.float32)
    B, S, Hq, Hkv, D, n = _shape(q, k, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _bwd_operands(o, lse, do, B, S, Hq, D)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    _bwd_outputs(dq, dk, dv, B, S, Hq, Hkv, D, torch.bfloat16)
    nbytes = bwd_workspace_bytes(B, Hq, Hkv, S, D)
    if workspace is None:
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=q.device)
    elif not (workspace.is_contiguous() and workspace.numel() * workspace.element_size() >= nbytes
              and workspace.device == q.device):
        raise ValueError(f"workspace must be a contiguous tensor of at least {nbytes} bytes on {q.device}")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            B, Hq, Hkv, S, D, int(bool(causal)), _ptr(cu_seqlens), n, float(scale), _stream())
    if phases is None:
        _check(load_library().attn_bwd(*args), "attn_bwd")
    else:
        _check(load_library().attn_bwd_phases(int(phases), *args), "attn_bwd_phases")
    return dq, dk, dv


def bwd_accumulate(q, k, v, o, lse, do, dq_acc, dk_acc, dv_acc, *, causal: bool, accumulate: bool = True,
                   cu_seqlens=None, scale: Optional[float] = None, workspace=None):
    """Backward with fp32 accumulators: the gradients are added to dq_acc, dk_acc, dv_acc (or written to them with
    accumulate=False). Shapes as q, k, v. Returns (dq_acc, dk_acc, dv_acc)."""
    import torch
    _check_tensors(q, k, v, o, do, dtype=torch.bfloat16)
    _check_tensors(lse, dq_acc, dk_acc, dv_acc, dtype=torch.float32)
    B, S, Hq, Hkv, D, n = _shape(q, k, v, cu_seqlens)
    _bwd_operands(o, lse, do, B, S, Hq, D)
    _bwd_outputs(dq_acc, dk_acc, dv_acc, B, S, Hq, Hkv, D, torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = bwd_workspace_bytes(B, Hq, Hkv, S, D)
    if workspace is None:
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=q.device)
    elif not (workspace.is_contiguous() and workspace.numel() * workspace.element_size() >= nbytes
              and workspace.device == q.device):
        raise ValueError(f"workspace must be a contiguous tensor of at least {nbytes} bytes on {q.device}")
    st = load_library().attn_bwd_accumulate(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq_acc),
                                            _ptr(dk_acc), _ptr(dv_acc), int(bool(accumulate)), _ptr(workspace), B, Hq,
                                            Hkv, S, D, int(bool(causal)), _ptr(cu_seqlens), n, float(scale),
                                            _stream())
    _check(st, "attn_bwd_accumulate")
    return dq_acc, dk_acc, dv_acc


def bwd_noalloc(q, k, v, o, lse, do, *, causal: bool, cu_seqlens=None, scale: Optional[float] = None, dq=None,
                dk=None, dv=None):
    """Backward through attn_bwd_noalloc: no workspace, the library's fixed scratch instead.

    Returns (dq, dk, dv). The call itself allocates nothing on the device;
    outputs not passed in are allocated here, by torch, before it.
    """
    import torch
    _check_tensors(q, k, v, o, do, dtype=torch.bfloat16)
    _check_tensors(lse, dtype=torch.float32)
    B, S, Hq, Hkv, D, n = _shape(q, k, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _bwd_operands(o, lse, do, B, S, Hq, D)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    _bwd_outputs(dq, dk, dv, B, S, Hq, Hkv, D, torch.bfloat16)
    st = load_library().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                         _ptr(dv), B, Hq, Hkv, S, D, int(bool(causal)), _ptr(cu_seqlens), n,
                                         float(scale), _stream())
    _check(st, "attn_bwd_noalloc")
    return dq, dk, dv


def bwd_fp8_workspace_bytes(batch: int, hq: int, hkv: int, seqlen: int, head_dim: int) -> int:
    return int(load_library().attn_bwd_fp8_workspace_bytes(batch, hq, hkv, seqlen, head_dim))


def bwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, o, lse, do, *, causal: bool, cu_seqlens=None,
            scale: Optional[float] = None, workspace=None, dq=None, dk=None, dv=None):
    """Backward of fwd_fp8: bf16 (dq, dk, dv) of attention over the dequantised inputs."""
    import torch
    _check_tensors(q8, k8, v8, dtype=torch.uint8)
    _check_tensors(descale_q, descale_k, descale_v, lse, dtype=torch.float32)
    _check_tensors(o, do, dtype=torch.bfloat16)
    B, S, Hq, Hkv, D, n = _shape(q8, k8, v8, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_descales(descale_q, descale_k, descale_v)
    _bwd_operands(o, lse, do, B, S, Hq, D)
    dq = dq if dq is not None else torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=q8.device)
    dk = dk if dk is not None else torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device=q8.device)
    dv = dv if dv is not None else torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device=q8.device)
    _bwd_outputs(dq, dk, dv, B, S, Hq, Hkv, D, torch.bfloat16)
    nbytes = bwd_fp8_workspace_bytes(B, Hq, Hkv, S, D)
    if workspace is None:
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=q8.device)
    elif not (workspace.is_contiguous() and workspace.numel() * workspace.element_size() >= nbytes
              and workspace.device == q8.device):
        raise ValueError(f"workspace must be a contiguous tensor of at least {nbytes} bytes on {q8.device}")
    st = load_library().attn_bwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale_q), _ptr(descale_k), _ptr(descale_v),
                                     _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                     B, Hq, Hkv, S, D, int(bool(causal)), _ptr(cu_seqlens), n, float(scale), _stream())
    _check(st, "attn_bwd_fp8")
    return dq, dk, dv
