"""Thin ctypes binding of libfa_mi355x.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module only checks
tensor shapes and dtypes, allocates outputs and workspaces with PyTorch, and
passes raw device pointers plus the current HIP stream.  Importing it fails
loudly when the library has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

from .build import LIB_PATH

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -m exact_attention_80_amd.build)")


_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGS = {
    "fa_abi_version": ([], _i),
    "fa_status_string": ([_i], ctypes.c_char_p),
    "fa_last_error": ([], ctypes.c_char_p),
    "fa_fwd_workspace_size": ([_i] * 6, _sz),
    "fa_fwd": ([_p] * 5 + [_i] * 5 + [_f, _i, _p, _sz, _p], _i),
    "fa_fwd_fp8": ([_p] * 5 + [_i] * 5 + [_f, _f, _f, _i, _p], _i),
    "fa_bwd_workspace_size": ([_i] * 7, _sz),
    "fa_bwd": ([_p] * 9 + [_i] * 5 + [_f, _i, _i, _p, _sz, _p], _i),
    "fa_varlen_fwd_workspace_size": ([_i] * 6, _sz),
    "fa_varlen_fwd": ([_p] * 6 + [_i] * 6 + [_f, _i, _p, _sz, _p], _i),
    "fa_varlen_bwd_workspace_size": ([_i] * 7, _sz),
    "fa_varlen_bwd": ([_p] * 10 + [_i] * 6 + [_f, _i, _i, _p, _sz, _p], _i),
    "fa_varlen_qk_fwd_workspace_size": ([_i] * 7, _sz),
    "fa_varlen_qk_fwd": ([_p] * 7 + [_i] * 8 + [_f, _i, _p, _sz, _p], _i),
    "fa_varlen_qk_fwd_fp8": ([_p] * 7 + [_i] * 8 + [_f, _f, _f, _i, _p, _sz, _p], _i),
    "fa_varlen_qk_fwd_noalloc": ([_p] * 7 + [_i] * 8 + [_f, _i, _p], _i),
    "fa_varlen_qk_bwd_workspace_size": ([_i] * 8, _sz),
    "fa_varlen_qk_bwd": ([_p] * 11 + [_i] * 8 + [_f, _i, _i, _p, _sz, _p], _i),
    "fa_workspace_error": ([_p, _sz, _p, ctypes.POINTER(ctypes.c_uint32)], _i),
    "fa_probe_dq_reduction": ([_p, _i, _i, _i, _i, _i, _p], _i),
    "fa_timing_begin": ([], _i),
    "fa_timing_end": ([ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)], _i),
}


def _load(path: str):
    lib = ctypes.CDLL(path)
    for name, (args, ret) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ret
    return lib


_lib = _load(LIB_PATH)


def load_variant(name: str):
    """The ctypes handle of a test variant built beside the library (see
    build.VARIANTS), for the ``lib`` argument of fwd."""
    from .build import variant_path
    path = variant_path(name)
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -m exact_attention_80_amd.build)")
    return _load(path)

FA_OK = 0


class FAError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        self.status = status
        L = _lib if lib is None else lib
        name = L.fa_status_string(status).decode()
        detail = L.fa_last_error().decode()
        super().__init__(f"{where}: {name}: {detail}")


def _check(status: int, where: str, lib=None) -> None:
    """Raise FAError for a failed call; lib is the library that was called
    (its own last-error text), default this package's."""
    if status != FA_OK:
        raise FAError(status, where, lib)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, shape, dtype=torch.bfloat16):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _scale(d, softmax_scale):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def fwd(q, k, v, causal: bool = False, softmax_scale: float | None = None, lib=None):
    """Dense forward: q [B,N,Hq,d], k/v [B,N,Hkv,d] bf16 -> (o [B,N,Hq,d] bf16, lse [B,Hq,N] fp32).

    lib: another build of the library (load_variant), default this package's."""
    L = _lib if lib is None else lib
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    _need(q, "q", (B, N, Hq, d))
    _need(k, "k", (B, N, Hkv, d))
    _need(v, "v", (B, N, Hkv, d))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    ws_n = L.fa_fwd_workspace_size(B, N, Hq, Hkv, d, int(causal))
    ws = _workspace(ws_n, q.device)
    _check(L.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, N, Hq, Hkv, d, _scale(d, softmax_scale), int(causal),
                       _ptr(ws), ws_n, _stream()), "fa_fwd", L)
    return o, lse


def _e4m3_bytes(t, name, shape):
    """fp8 operands travel as their raw e4m3 bytes (uint8 or float8_e4m3fn tensors)."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _need(t, name, shape, torch.uint8)
    return t


def fwd_fp8(q8, k8, v, q_descale: float, k_descale: float, causal: bool = False,
            softmax_scale: float | None = None, lib=None):
    """Dense forward with fp8 scores: q8 [B,N,Hq,d], k8 [B,N,Hkv,d] OCP e4m3 bytes
    (uint8 or float8_e4m3fn) standing for q_descale * q8 and k_descale * k8, v
    [B,N,Hkv,d] bf16 -> (o [B,N,Hq,d] bf16, lse [B,Hq,N] fp32).  d = 64 or 128.
    lib: another build of the library (load_variant), default this package's."""
    L = _lib if lib is None else lib
    B, N, Hq, d = q8.shape
    Hkv = k8.shape[2]
    q8 = _e4m3_bytes(q8, "q8", (B, N, Hq, d))
    k8 = _e4m3_bytes(k8, "k8", (B, N, Hkv, d))
    _need(v, "v", (B, N, Hkv, d))
    o = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=v.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=v.device)
    _check(L.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), o.data_ptr(),
                        lse.data_ptr(), B, N, Hq, Hkv, d, _scale(d, softmax_scale),
                        float(q_descale), float(k_descale), int(causal), _stream()),
           "fa_fwd_fp8", L)
    return o, lse


def bwd_workspace(q, k, causal: bool, deterministic: int | bool) -> torch.Tensor:
    B, N, Hq, d = q.shape
    n = _lib.fa_bwd_workspace_size(B, N, Hq, k.shape[2], d, int(causal), int(deterministic))
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def bwd(q, k, v, o, lse, do, causal: bool = False, softmax_scale: float | None = None,
        deterministic: int | bool = False, workspace: torch.Tensor | None = None, lib=None):
    """Dense backward -> (dq [B,N,Hq,d], dk [B,N,Hkv,d], dv [B,N,Hkv,d]) bf16.

    deterministic selects the dQ reduction across key tiles: 0 (False) fp32
    atomics, 1 (True) semaphore-ordered adds, 2 partial tiles summed in a fixed
    order by a second kernel, 3 partial tiles summed in a fixed order by the
    last workgroup to contribute to each query tile, 4 int32 fixed-point
    atomics (per-row scale from a bound on the row's dQ; exact sums in any
    order, the fastest mode); 1 to 4 are bit-reproducible.  Mode 1 bounds its waits: one that expires leaves dQ
    correct but unordered and sets a bit that workspace_error(workspace)
    reports (check it after the call when reproducibility matters).  lib:
    another build of the library (load_variant), default this package's."""
    L = _lib if lib is None else lib
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    _need(q, "q", (B, N, Hq, d))
    _need(k, "k", (B, N, Hkv, d))
    _need(v, "v", (B, N, Hkv, d))
    _need(o, "o", (B, N, Hq, d))
    _need(do, "do", (B, N, Hq, d))
    _need(lse, "lse", (B, Hq, N), torch.float32)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if workspace is None:
        n = L.fa_bwd_workspace_size(B, N, Hq, Hkv, d, int(causal), int(deterministic))
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    else:
        ws = workspace
    _check(L.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    B, N, Hq, Hkv, d, _scale(d, softmax_scale), int(causal), int(deterministic),
                    ws.data_ptr(), ws.numel(), _stream()), "fa_bwd", L)
    return dq, dk, dv


def _cu(cu_seqlens, T):
    _need(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32)
    return cu_seqlens.shape[0] - 1


def varlen_fwd_workspace(nseq: int, T: int, Hq: int, Hkv: int, d: int, causal: bool,
                         device) -> torch.Tensor | None:
    return _workspace(_lib.fa_varlen_fwd_workspace_size(nseq, T, Hq, Hkv, d, int(causal)), device)


def varlen_bwd_workspace(nseq: int, T: int, Hq: int, Hkv: int, d: int, causal: bool,
                         deterministic: bool, device) -> torch.Tensor:
    n = _lib.fa_varlen_bwd_workspace_size(nseq, T, Hq, Hkv, d, int(causal), int(deterministic))
    return torch.empty(n, dtype=torch.uint8, device=device)


def varlen_fwd(q, k, v, cu_seqlens, causal: bool = False, softmax_scale: float | None = None,
               max_seqlen: int = 0, workspace: torch.Tensor | None = None, lib=None):
    """Packed forward: q [T,Hq,d], k/v [T,Hkv,d], cu_seqlens int32 [nseq+1] on the device
    -> (o [T,Hq,d], lse [Hq,T]).  lib: another build of the library (load_variant)."""
    L = _lib if lib is None else lib
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", (T, Hq, d))
    _need(k, "k", (T, Hkv, d))
    _need(v, "v", (T, Hkv, d))
    nseq = _cu(cu_seqlens, T)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    ws = workspace
    if ws is None:
        ws = _workspace(L.fa_varlen_fwd_workspace_size(nseq, T, Hq, Hkv, d, int(causal)), q.device)
    _check(L.fa_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), cu_seqlens.data_ptr(), nseq, T, int(max_seqlen),
                           Hq, Hkv, d, _scale(d, softmax_scale), int(causal),
                           _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
           "fa_varlen_fwd", L)
    return o, lse


def varlen_bwd(q, k, v, o, lse, do, cu_seqlens, causal: bool = False,
               softmax_scale: float | None = None, deterministic: bool = False,
               max_seqlen: int = 0, workspace: torch.Tensor | None = None, lib=None):
    """Packed backward -> (dq [T,Hq,d], dk [T,Hkv,d], dv [T,Hkv,d]); deterministic
    0, 1 or 4 as in bwd.  lib: another build of the library (load_variant)."""
    L = _lib if lib is None else lib
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", (T, Hq, d))
    _need(k, "k", (T, Hkv, d))
    _need(v, "v", (T, Hkv, d))
    _need(o, "o", (T, Hq, d))
    _need(do, "do", (T, Hq, d))
    _need(lse, "lse", (Hq, T), torch.float32)
    nseq = _cu(cu_seqlens, T)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = workspace
    if ws is None:
        n = L.fa_varlen_bwd_workspace_size(nseq, T, Hq, Hkv, d, int(causal), int(deterministic))
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(L.fa_varlen_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), cu_seqlens.data_ptr(), nseq, T, int(max_seqlen),
                           Hq, Hkv, d, _scale(d, softmax_scale), int(causal),
                           int(deterministic), ws.data_ptr(), ws.numel(), _stream()),
           "fa_varlen_bwd", L)
    return dq, dk, dv


def varlen_qk_fwd_workspace(nseq: int, Tq: int, Tk: int, Hq: int, Hkv: int, d: int,
                            causal: bool, device) -> torch.Tensor | None:
    return _workspace(_lib.fa_varlen_qk_fwd_workspace_size(nseq, Tq, Tk, Hq, Hkv, d, int(causal)),
                      device)


def varlen_qk_bwd_workspace(nseq: int, Tq: int, Tk: int, Hq: int, Hkv: int, d: int, causal: bool,
                            deterministic: int | bool, device) -> torch.Tensor:
    n = _lib.fa_varlen_qk_bwd_workspace_size(nseq, Tq, Tk, Hq, Hkv, d, int(causal),
                                             int(deterministic))
    return torch.empty(n, dtype=torch.uint8, device=device)


def _cu_pair(cu_q, cu_k):
    nseq = _cu(cu_q, 0)
    _need(cu_k, "cu_seqlens_k", (nseq + 1,), torch.int32)
    return nseq


def varlen_qk_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool = False,
                  softmax_scale: float | None = None, max_seqlen_q: int = 0,
                  max_seqlen_k: int = 0, workspace: torch.Tensor | None = None, lib=None):
    """Packed forward with separate query and key lengths per sequence:
    q [Tq,Hq,d], k/v [Tk,Hkv,d], cu_seqlens_q / cu_seqlens_k int32 [nseq+1] on
    the device -> (o [Tq,Hq,d], lse [Hq,Tq]).  Causal masks are aligned
    bottom-right (query i sees key j iff j <= i + Lk - Lq).  lib: another
    build of the library (load_variant), default this package's."""
    L = _lib if lib is None else lib
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    _need(q, "q", (Tq, Hq, d))
    _need(k, "k", (Tk, Hkv, d))
    _need(v, "v", (Tk, Hkv, d))
    nseq = _cu_pair(cu_seqlens_q, cu_seqlens_k)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    ws = workspace
    if ws is None:
        ws = _workspace(L.fa_varlen_qk_fwd_workspace_size(nseq, Tq, Tk, Hq, Hkv, d, int(causal)),
                        q.device)
    _check(L.fa_varlen_qk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                 nseq, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d,
                                 _scale(d, softmax_scale), int(causal), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream()),
           "fa_varlen_qk_fwd", L)
    return o, lse



NOALLOC_SCRATCH_BYTES = 64 << 20  # FA_NOALLOC_SCRATCH_BYTES


def varlen_qk_fwd_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool = False,
                          softmax_scale: float | None = None, max_seqlen_q: int = 0,
                          max_seqlen_k: int = 0, out=None):
    """varlen_qk_fwd through the entry point that allocates nothing on the
    device: the library's static per-GPU scratch array (NOALLOC_SCRATCH_BYTES)
    replaces the workspace, and larger problems are rejected.  out=(o, lse)
    writes into caller-provided tensors, so that nothing is allocated at all.
    Calls that overlap in time on one GPU share the scratch and must not be
    issued concurrently."""
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    _need(q, "q", (Tq, Hq, d))
    _need(k, "k", (Tk, Hkv, d))
    _need(v, "v", (Tk, Hkv, d))
    nseq = _cu_pair(cu_seqlens_q, cu_seqlens_k)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (Tq, Hq, d))
        _need(lse, "lse", (Hq, Tq), torch.float32)
    _check(_lib.fa_varlen_qk_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), cu_seqlens_q.data_ptr(),
                                         cu_seqlens_k.data_ptr(), nseq, Tq, Tk,
                                         int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d,
                                         _scale(d, softmax_scale), int(causal), _stream()),
           "fa_varlen_qk_fwd_noalloc")
    return o, lse


def varlen_qk_fwd_fp8(q8, k8, v, cu_seqlens_q, cu_seqlens_k, q_descale: float, k_descale: float,
                      causal: bool = False, softmax_scale: float | None = None,
                      max_seqlen_q: int = 0, max_seqlen_k: int = 0,
                      workspace: torch.Tensor | None = None):
    """varlen_qk_fwd with fp8 scores: q8 [Tq,Hq,d], k8 [Tk,Hkv,d] OCP e4m3 bytes
    (uint8 or float8_e4m3fn) standing for q_descale * q8 and k_descale * k8, v
    [Tk,Hkv,d] bf16 -> (o [Tq,Hq,d] bf16, lse [Hq,Tq] fp32).  d = 64 or 128."""
    Tq, Hq, d = q8.shape
    Tk, Hkv = k8.shape[0], k8.shape[1]
    q8 = _e4m3_bytes(q8, "q8", (Tq, Hq, d))
    k8 = _e4m3_bytes(k8, "k8", (Tk, Hkv, d))
    _need(v, "v", (Tk, Hkv, d))
    nseq = _cu_pair(cu_seqlens_q, cu_seqlens_k)
    o = torch.empty((Tq, Hq, d), dtype=torch.bfloat16, device=v.device)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=v.device)
    ws = workspace
    if ws is None:
        ws = varlen_qk_fwd_workspace(nseq, Tq, Tk, Hq, Hkv, d, causal, v.device)
    ws_n = 0 if ws is None else ws.numel()
    _check(_lib.fa_varlen_qk_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), cu_seqlens_q.data_ptr(),
                                     cu_seqlens_k.data_ptr(), nseq, Tq, Tk, int(max_seqlen_q),
                                     int(max_seqlen_k), Hq, Hkv, d, _scale(d, softmax_scale),
                                     float(q_descale), float(k_descale), int(causal), _ptr(ws),
                                     ws_n, _stream()), "fa_varlen_qk_fwd_fp8")
    return o, lse


def varlen_qk_bwd(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, causal: bool = False,
                  softmax_scale: float | None = None, deterministic: int | bool = False,
                  max_seqlen_q: int = 0, max_seqlen_k: int = 0,
                  workspace: torch.Tensor | None = None, lib=None):
    """Packed backward with separate query and key lengths
    -> (dq [Tq,Hq,d], dk [Tk,Hkv,d], dv [Tk,Hkv,d]); deterministic 0, 1 or 4.
    lib: another build of the library (load_variant)."""
    L = _lib if lib is None else lib
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    _need(q, "q", (Tq, Hq, d))
    _need(k, "k", (Tk, Hkv, d))
    _need(v, "v", (Tk, Hkv, d))
    _need(o, "o", (Tq, Hq, d))
    _need(do, "do", (Tq, Hq, d))
    _need(lse, "lse", (Hq, Tq), torch.float32)
    nseq = _cu_pair(cu_seqlens_q, cu_seqlens_k)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = workspace
    if ws is None:
        n = L.fa_varlen_qk_bwd_workspace_size(nseq, Tq, Tk, Hq, Hkv, d, int(causal),
                                              int(deterministic))
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(L.fa_varlen_qk_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                              nseq, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d,
                              _scale(d, softmax_scale), int(causal), int(deterministic),
                              ws.data_ptr(), ws.numel(), _stream()),
           "fa_varlen_qk_bwd", L)
    return dq, dk, dv


def workspace_error(ws: torch.Tensor) -> int:
    """Synchronise and return the device error word a varlen/backward call left in ``ws``."""
    bits = ctypes.c_uint32(0)
    st = _lib.fa_workspace_error(ws.data_ptr(), ws.numel(), _stream(), ctypes.byref(bits))
    if st not in (FA_OK, 6):
        _check(st, "fa_workspace_error")
    return int(bits.value)


TIMING_KINDS = ("fwd", "bwd_main", "bwd_pre", "bwd_post", "sched", "fwd_combine")


def timing_begin(lib=None) -> None:
    """Start recording HIP events around every kernel this thread launches
    (through lib, a variant from load_variant, or this package's library)."""
    L = _lib if lib is None else lib
    _check(L.fa_timing_begin(), "fa_timing_begin", L)


def timing_end(lib=None) -> dict:
    """Stop recording; returns {kind: (launches, total_ms)} for the kernels launched since."""
    L = _lib if lib is None else lib
    n = len(TIMING_KINDS)
    counts = (ctypes.c_int * n)()
    ms = (ctypes.c_float * n)()
    _check(L.fa_timing_end(counts, ms), "fa_timing_end", L)
    return {k: (int(counts[i]), float(ms[i])) for i, k in enumerate(TIMING_KINDS)}


def probe_dq_reduction(buf, blocks: int, items: int, store: int | bool = False) -> int:
    """Launch the dQ-reduction measurement kernel on buf [rows, row_floats]
    fp32 (rows % 32 == 0, row_floats % 128 == 0): store 0 (False) fp32 atomic
    adds, 1 (True) plain stores, 2 int32 atomic adds (buf holds int32 bits);
    returns the bytes it moves."""
    _need(buf, "buf", tuple(buf.shape), torch.float32)
    rows, row_floats = buf.shape
    _check(_lib.fa_probe_dq_reduction(buf.data_ptr(), rows, row_floats, blocks, items, int(store),
                                      _stream()), "fa_probe_dq_reduction")
    return blocks * items * 16384


def lib_path() -> str:
    return LIB_PATH


def raw():
    """The ctypes handle of the library (for ABI tests)."""
    return _lib
