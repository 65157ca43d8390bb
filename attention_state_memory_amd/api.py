"""Python binding of libasm_amd.so (the attention-state-memory HIP library).

Argument marshalling only: each function checks that the torch tensors it
receives live on the GPU with the layout the C ABI expects, allocates the
workspace and outputs with torch, and calls the matching entry point of
include/asm_memory.h on torch's current stream.  Every step of the method
runs in the library's kernels.  There is no fallback: if the library is not
built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libasm_amd.so")

BF16, F32 = 0, 1

_c_int, _c_float, _c_i64, _c_size, _vp = (ctypes.c_int, ctypes.c_float, ctypes.c_int64,
                                          ctypes.c_size_t, ctypes.c_void_p)

# name -> (restype, argtypes); the C declarations are in include/asm_memory.h
SIGNATURES = {
    "asm_abi_version": (_c_int, []),
    "asm_status_str": (ctypes.c_char_p, [_c_int]),
    "asm_last_error": (ctypes.c_char_p, []),
    "asm_centroid_inv_norms": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "asm_decode_step_ws": (_c_size, [_c_int] * 7),
    "asm_decode_step": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int,
                                 _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_decode_step_begin": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int,
                                       _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_decode_step_finish": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int,
                                        _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_decode_step_noalloc": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int,
                                         _vp, _vp, _vp, _vp]),
    "asm_attend_step_ws": (_c_size, [_c_int] * 6),
    "asm_attend_step": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp,
                                 _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int, _vp, _vp, _vp, _c_size,
                                 _vp]),
    "asm_whiten_fit_ws": (_c_size, [_c_int] * 4),
    "asm_whiten_fit": (_c_int, [_c_int] * 4 + [_vp, ctypes.c_double, _vp, _vp, _vp, _vp, _c_size,
                                               _vp]),
    "asm_whiten_rows": (_c_int, [_c_int, _c_int, _c_i64, _c_int, _vp, _c_i64, _c_i64, _vp, _vp,
                                 _vp, _vp]),
    "asm_decode_step_whitened_ws": (_c_size, [_c_int] * 7),
    "asm_decode_step_whitened": (_c_int, [_c_int] * 6 + [_c_float, _vp, _vp, _vp, _vp, _vp, _vp,
                                                          _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                                          _vp, _vp, _c_int, _vp, _vp, _vp, _vp,
                                                          _c_size, _vp]),
    "asm_build_states_ws": (_c_size, [_c_int] * 7),
    "asm_build_states": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_size, _vp]),
    "asm_kmeans_assign_ws": (_c_size, [_c_int] * 5),
    "asm_kmeans_assign": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_aggregate_ws": (_c_size, [_c_int] * 5),
    "asm_aggregate": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_build_states_streamed_ws": (_c_size, [_c_int] * 6),
    "asm_build_states_streamed": (_c_int, [_c_int] * 7 + [_c_float, _vp, _vp, _vp, _vp, _vp,
                                                          _c_int, _vp, _c_size, _vp, _vp]),
    "asm_build_memory_ws": (_c_size, [_c_int] * 5),
    "asm_build_memory": (_c_int, [_c_int] * 6 + [_vp] * 9 + [_vp, _c_size, _vp]),
    "asm_build_index_ws": (_c_size, [_c_int] * 5),
    "asm_build_index": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_decode_step_hier_ws": (_c_size, [_c_int] * 9),
    "asm_decode_step_hier": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int,
                                      _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "asm_index_group_rows": (_c_int, [_c_int] * 4 + [_vp] * 6),
}

_lib: Optional[ctypes.CDLL] = None


class AsmError(RuntimeError):
    """A library call returned a negative status."""


def lib() -> ctypes.CDLL:
    """Load libasm_amd.so (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m attention_state_memory_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(name: str, status: int) -> None:
    if status != 0:
        L = lib()
        raise AsmError(f"{name}: {L.asm_status_str(status).decode()} "
                       f"({L.asm_last_error().decode()})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """The caller's workspace if large enough, else a new one."""
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes and ws.is_cuda:
        return ws
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def abi_version() -> int:
    return lib().asm_abi_version()


# ---------------------------------------------------------------------------

def centroid_inv_norms(C: torch.Tensor, cinv: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cinv[h, k] = 1/|C[h, k]| (0 for a zero row).  C [H, K, d]."""
    _dev(C, "C")
    H, K, d = C.shape
    if cinv is None:
        cinv = torch.empty((H, K), dtype=torch.float32, device=C.device)
    _dev(cinv, "cinv", torch.float32)
    _check("asm_centroid_inv_norms",
           lib().asm_centroid_inv_norms(_dtype_code(C), H, K, d, _ptr(C), _ptr(cinv),
                                        _stream(C.device)))
    return cinv


def decode_step_ws(dtype_code: int, B, Hq, Hkv, d, K, max_kv_len) -> int:
    return int(lib().asm_decode_step_ws(dtype_code, B, Hq, Hkv, d, K, max_kv_len))


def _decode_operands(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len):
    for t, n in ((q, "q"), (C, "C")):
        _dev(t, n)
    _dev(cinv, "cinv", torch.float32)
    _dev(Abar, "Abar", torch.float32)
    _dev(LSEbar, "LSEbar", torch.float32)
    _dev(kv_start, "kv_start", torch.int32)
    _dev(kv_len, "kv_len", torch.int32)
    code = _dtype_code(q)
    if C.dtype != q.dtype or Kl.dtype != q.dtype or Vl.dtype != q.dtype:
        raise TypeError("q, C, Kl and Vl must share one dtype")
    for t, n in ((Kl, "Kl"), (Vl, "Vl")):
        if not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{n} must be a [Hkv, capacity, d] CUDA tensor with d contiguous")
    if Kl.stride() != Vl.stride() or Kl.shape != Vl.shape:
        raise ValueError("Kl and Vl must share shape and strides")
    return code


def decode_step(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len, max_kv_len: int,
                scale: float, *, out=None, out_lse=None, out_idx=None, workspace=None,
                want_lse: bool = True, want_idx: bool = True):
    """One decode step.  q [B, Hq, d]; C [Hq, K, d]; cinv, LSEbar [Hq, K];
    Abar [Hq, K, d]; Kl, Vl [Hkv, capacity, d] (any strides with d
    contiguous); kv_start, kv_len [B] int32 token slots.
    Returns (out [B, Hq, d] f32, out_lse [B, Hq] f32 | None, idx [B, Hq] i32 | None)."""
    code = _decode_operands(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len)
    B, Hq, d = q.shape
    K = C.shape[1]
    Hkv, cap, _ = Kl.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if out_lse is None and want_lse:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if out_idx is None and want_idx:
        out_idx = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    nbytes = decode_step_ws(code, B, Hq, Hkv, d, K, max_kv_len)
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_decode_step", lib().asm_decode_step(
        code, B, Hq, Hkv, d, K, float(scale), _ptr(q), _ptr(C), _ptr(cinv), _ptr(Abar),
        _ptr(LSEbar), _ptr(Kl), _ptr(Vl), Kl.stride(0), Kl.stride(1), cap,
        _ptr(kv_start), _ptr(kv_len), int(max_kv_len), _ptr(out), _ptr(out_lse), _ptr(out_idx),
        _ptr(ws), nbytes, _stream(dev)))
    return out, out_lse, out_idx


def _decode_phase(name, q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len, max_kv_len, scale,
                  out, out_lse, out_idx, workspace):
    code = _decode_operands(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len)
    B, Hq, d = q.shape
    K = C.shape[1]
    Hkv, cap, _ = Kl.shape
    _dev(out, "out", torch.float32)
    for t, n, dt in ((out_lse, "out_lse", torch.float32), (out_idx, "out_idx", torch.int32)):
        if t is not None:
            _dev(t, n, dt)
    _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(
        code, B, Hq, Hkv, d, K, float(scale), _ptr(q), _ptr(C), _ptr(cinv), _ptr(Abar),
        _ptr(LSEbar), _ptr(Kl), _ptr(Vl), Kl.stride(0), Kl.stride(1), cap,
        _ptr(kv_start), _ptr(kv_len), int(max_kv_len), _ptr(out), _ptr(out_lse), _ptr(out_idx),
        _ptr(workspace), nbytes, _stream(q.device)))
    return out, out_lse, out_idx


def decode_step_begin(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len, max_kv_len: int,
                      scale: float, *, out, out_lse=None, out_idx=None, workspace):
    """First launch of decode_step (scoring and local attention into the
    workspace).  decode_step_finish with the same arguments and workspace,
    on the same stream, completes the step.  The workspace is required
    (decode_step_ws bytes) and shared by the two calls."""
    return _decode_phase("asm_decode_step_begin", q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start,
                         kv_len, max_kv_len, scale, out, out_lse, out_idx, workspace)


def decode_step_finish(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len, max_kv_len: int,
                       scale: float, *, out, out_lse=None, out_idx=None, workspace):
    """Second launch of decode_step (index, gather and merge into out,
    out_lse, out_idx), after decode_step_begin with the same arguments and
    workspace.  Returns (out, out_lse, out_idx)."""
    return _decode_phase("asm_decode_step_finish", q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start,
                         kv_len, max_kv_len, scale, out, out_lse, out_idx, workspace)


def decode_step_noalloc(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len, max_kv_len: int,
                        scale: float, *, out, out_lse=None, out_idx=None):
    """decode_step through the entry point that allocates nothing: the
    library's fixed per-GPU scratch replaces the workspace, and this binding
    allocates nothing either (out is required; out_lse and out_idx are
    written when given).  Returns (out, out_lse, out_idx)."""
    code = _decode_operands(q, C, cinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len)
    B, Hq, d = q.shape
    K = C.shape[1]
    Hkv, cap, _ = Kl.shape
    _dev(out, "out", torch.float32)
    for t, n, dt in ((out_lse, "out_lse", torch.float32), (out_idx, "out_idx", torch.int32)):
        if t is not None:
            _dev(t, n, dt)
    _check("asm_decode_step_noalloc", lib().asm_decode_step_noalloc(
        code, B, Hq, Hkv, d, K, float(scale), _ptr(q), _ptr(C), _ptr(cinv), _ptr(Abar),
        _ptr(LSEbar), _ptr(Kl), _ptr(Vl), Kl.stride(0), Kl.stride(1), cap,
        _ptr(kv_start), _ptr(kv_len), int(max_kv_len), _ptr(out), _ptr(out_lse), _ptr(out_idx),
        _stream(q.device)))
    return out, out_lse, out_idx


def whiten_fit(X, ridge: float = 1e-6, *, want_resid: bool = False, workspace=None):
    """Whitening transforms of the calibration queries X [H, N, d]: returns
    (mu [H, d] f64, W [H, d, d] f64, resid [H] f64 | None)."""
    _dev(X, "X")
    code = _dtype_code(X)
    H, N, d = X.shape
    dev = X.device
    mu = torch.empty((H, d), dtype=torch.float64, device=dev)
    W = torch.empty((H, d, d), dtype=torch.float64, device=dev)
    resid = torch.empty((H,), dtype=torch.float64, device=dev) if want_resid else None
    nbytes = int(lib().asm_whiten_fit_ws(code, H, N, d))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_whiten_fit", lib().asm_whiten_fit(
        code, H, N, d, _ptr(X), float(ridge), _ptr(mu), _ptr(W), _ptr(resid), _ptr(ws), nbytes,
        _stream(dev)))
    return mu, W, resid


def whiten_rows(Y, mu, W, *, out=None):
    """Whitened rows of a head-major table Y [H, M, d]: round(W[h] (y - mu[h]))."""
    _dev(Y, "Y")
    _dev(mu, "mu", torch.float64)
    _dev(W, "W", torch.float64)
    H, M, d = Y.shape
    if out is None:
        out = torch.empty_like(Y)
    _dev(out, "out", Y.dtype)
    _check("asm_whiten_rows", lib().asm_whiten_rows(
        _dtype_code(Y), H, M, d, _ptr(Y), M * d, d, _ptr(mu), _ptr(W), _ptr(out),
        _stream(Y.device)))
    return out


def attend_step(q, Kc, Vc, kv_start, kv_len, max_kv_len: int, scale: float, *, out=None,
                out_lse=None, workspace=None):
    """Full attention of one decode step (no memory).  q [B, Hq, d];
    Kc, Vc [Hkv, capacity, d] (any strides with d contiguous) holding each
    sequence's whole context; kv_start, kv_len [B] int32 token slots.
    Returns (out [B, Hq, d] f32, out_lse [B, Hq] f32)."""
    _dev(q, "q")
    _dev(kv_start, "kv_start", torch.int32)
    _dev(kv_len, "kv_len", torch.int32)
    code = _dtype_code(q)
    if Kc.dtype != q.dtype or Vc.dtype != q.dtype:
        raise TypeError("q, Kc and Vc must share one dtype")
    for t, n in ((Kc, "Kc"), (Vc, "Vc")):
        if not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{n} must be a [Hkv, capacity, d] CUDA tensor with d contiguous")
    if Kc.stride() != Vc.stride() or Kc.shape != Vc.shape:
        raise ValueError("Kc and Vc must share shape and strides")
    B, Hq, d = q.shape
    Hkv, cap, _ = Kc.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    nbytes = int(lib().asm_attend_step_ws(code, B, Hq, Hkv, d, int(max_kv_len)))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_attend_step", lib().asm_attend_step(
        code, B, Hq, Hkv, d, float(scale), _ptr(q), _ptr(Kc), _ptr(Vc), Kc.stride(0), Kc.stride(1),
        cap, _ptr(kv_start), _ptr(kv_len), int(max_kv_len), _ptr(out), _ptr(out_lse), _ptr(ws),
        nbytes, _stream(dev)))
    return out, out_lse


def decode_step_whitened(q, mu, W, Cw, cwinv, Abar, LSEbar, Kl, Vl, kv_start, kv_len,
                         max_kv_len: int, scale: float, *, out=None, out_lse=None, out_idx=None,
                         workspace=None):
    """decode_step with the lookup on whitened queries against the whitened
    table Cw (cwinv its inverse norms).  Returns (out, out_lse, idx)."""
    for t, n in ((q, "q"), (Cw, "Cw")):
        _dev(t, n)
    _dev(mu, "mu", torch.float64)
    _dev(W, "W", torch.float64)
    _dev(cwinv, "cwinv", torch.float32)
    _dev(Abar, "Abar", torch.float32)
    _dev(LSEbar, "LSEbar", torch.float32)
    _dev(kv_start, "kv_start", torch.int32)
    _dev(kv_len, "kv_len", torch.int32)
    code = _dtype_code(q)
    if Cw.dtype != q.dtype or Kl.dtype != q.dtype or Vl.dtype != q.dtype:
        raise TypeError("q, Cw, Kl and Vl must share one dtype")
    for t, n in ((Kl, "Kl"), (Vl, "Vl")):
        if not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{n} must be a [Hkv, capacity, d] CUDA tensor with d contiguous")
    if Kl.stride() != Vl.stride() or Kl.shape != Vl.shape:
        raise ValueError("Kl and Vl must share shape and strides")
    B, Hq, d = q.shape
    K = Cw.shape[1]
    Hkv, cap, _ = Kl.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    nbytes = int(lib().asm_decode_step_whitened_ws(code, B, Hq, Hkv, d, K, int(max_kv_len)))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_decode_step_whitened", lib().asm_decode_step_whitened(
        code, B, Hq, Hkv, d, K, float(scale), _ptr(q), _ptr(mu), _ptr(W), _ptr(Cw), _ptr(cwinv),
        _ptr(Abar), _ptr(LSEbar), _ptr(Kl), _ptr(Vl), Kl.stride(0), Kl.stride(1), cap,
        _ptr(kv_start), _ptr(kv_len), int(max_kv_len), _ptr(out), _ptr(out_lse), _ptr(out_idx),
        _ptr(ws), nbytes, _stream(dev)))
    return out, out_lse, out_idx


def build_states(Q, Kp, Vp, chunk: int, scale: float, *, A=None, LSE=None,
                 accumulate: bool = False, keep_chunks: bool = False, workspace=None):
    """Prefix states.  Q [Hq, N, d]; Kp, Vp [Hkv, L, d].  Returns
    (A [Hq, N, d], LSE [Hq, N], A_chunks [nc, Hq, N, d] | None,
    LSE_chunks [nc, Hq, N] | None)."""
    _dev(Q, "Q")
    _dev(Kp, "Kp")
    _dev(Vp, "Vp")
    code = _dtype_code(Q)
    if Kp.dtype != Q.dtype or Vp.dtype != Q.dtype:
        raise TypeError("Q, Kp and Vp must share one dtype")
    Hq, N, d = Q.shape
    Hkv, L, _ = Kp.shape
    dev = Q.device
    nc = -(-L // chunk) if L > 0 else 0
    if A is None:
        A = torch.empty((Hq, N, d), dtype=torch.float32, device=dev)
    if LSE is None:
        LSE = torch.empty((Hq, N), dtype=torch.float32, device=dev)
    _dev(A, "A", torch.float32)
    _dev(LSE, "LSE", torch.float32)
    Ac = Lc = None
    if keep_chunks:
        Ac = torch.empty((nc, Hq, N, d), dtype=torch.float32, device=dev)
        Lc = torch.empty((nc, Hq, N), dtype=torch.float32, device=dev)
    nbytes = int(lib().asm_build_states_ws(code, Hq, Hkv, N, L, d, chunk))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_build_states", lib().asm_build_states(
        code, Hq, Hkv, N, L, d, int(chunk), float(scale), _ptr(Q), _ptr(Kp), _ptr(Vp),
        _ptr(Ac), _ptr(Lc), _ptr(A), _ptr(LSE), int(bool(accumulate)), _ptr(ws), nbytes,
        _stream(dev)))
    return A, LSE, Ac, Lc


def build_states_streamed(Q, Kp_host, Vp_host, chunk: int, scale: float, *, A=None, LSE=None,
                          accumulate: bool = False, workspace=None, copy_stream=None):
    """Prefix states for a prefix in host memory.  Q [Hq, N, d] on the GPU;
    Kp_host, Vp_host [Hkv, L, d] CPU tensors (pinned for overlap).  The
    copies run on `copy_stream` (a new default-priority stream if None)
    while the current stream encodes.  Returns (A [Hq, N, d], LSE [Hq, N])."""
    _dev(Q, "Q")
    for t, name in ((Kp_host, "Kp_host"), (Vp_host, "Vp_host")):
        if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous CPU tensor")
        if t.dtype != Q.dtype:
            raise TypeError("Q, Kp_host and Vp_host must share one dtype")
    code = _dtype_code(Q)
    Hq, N, d = Q.shape
    Hkv, L, _ = Kp_host.shape
    dev = Q.device
    if A is None:
        A = torch.empty((Hq, N, d), dtype=torch.float32, device=dev)
    if LSE is None:
        LSE = torch.empty((Hq, N), dtype=torch.float32, device=dev)
    _dev(A, "A", torch.float32)
    _dev(LSE, "LSE", torch.float32)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=dev)
    nbytes = int(lib().asm_build_states_streamed_ws(code, Hq, Hkv, N, d, int(chunk)))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_build_states_streamed", lib().asm_build_states_streamed(
        code, Hq, Hkv, N, L, d, int(chunk), float(scale), _ptr(Q), Kp_host.data_ptr(),
        Vp_host.data_ptr(), _ptr(A), _ptr(LSE), int(bool(accumulate)), _ptr(ws), nbytes,
        _stream(dev), ctypes.c_void_p(copy_stream.cuda_stream)))
    return A, LSE


def kmeans_assign(X, C, cinv, *, idx=None, best=None, want_best: bool = False, workspace=None):
    """Nearest centroid by cosine.  X [H, N, d]; C [H, K, d]; cinv [H, K].
    Returns (idx [H, N] int32, best [H, N] float32 | None)."""
    _dev(X, "X")
    _dev(C, "C")
    _dev(cinv, "cinv", torch.float32)
    code = _dtype_code(X)
    if C.dtype != X.dtype:
        raise TypeError("X and C must share one dtype")
    H, N, d = X.shape
    K = C.shape[1]
    dev = X.device
    if idx is None:
        idx = torch.empty((H, N), dtype=torch.int32, device=dev)
    if best is None and want_best:
        best = torch.empty((H, N), dtype=torch.float32, device=dev)
    nbytes = int(lib().asm_kmeans_assign_ws(code, H, N, K, d))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_kmeans_assign", lib().asm_kmeans_assign(
        code, H, N, K, d, _ptr(X), _ptr(C), _ptr(cinv), _ptr(idx), _ptr(best), _ptr(ws),
        nbytes, _stream(dev)))
    return idx, best


def aggregate(X, idx, C, *, A=None, LSE=None, cinv=None, count=None, Abar=None, LSEbar=None,
              with_states: bool = True, workspace=None):
    """Memory-table update from an assignment.  X [H, N, d]; idx [H, N]
    int32; C [H, K, d] updated in place.  With with_states, A [H, N, d] and
    LSE [H, N] are aggregated into Abar [H, K, d], LSEbar [H, K].
    Returns (C, cinv, count, Abar | None, LSEbar | None)."""
    _dev(X, "X")
    _dev(idx, "idx", torch.int32)
    _dev(C, "C")
    code = _dtype_code(X)
    if C.dtype != X.dtype:
        raise TypeError("X and C must share one dtype")
    H, N, d = X.shape
    K = C.shape[1]
    dev = X.device
    if cinv is None:
        cinv = torch.empty((H, K), dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty((H, K), dtype=torch.int32, device=dev)
    if with_states:
        _dev(A, "A", torch.float32)
        _dev(LSE, "LSE", torch.float32)
        if Abar is None:
            Abar = torch.empty((H, K, d), dtype=torch.float32, device=dev)
        if LSEbar is None:
            LSEbar = torch.empty((H, K), dtype=torch.float32, device=dev)
    else:
        A = LSE = Abar = LSEbar = None
    nbytes = int(lib().asm_aggregate_ws(code, H, N, K, d))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_aggregate", lib().asm_aggregate(
        code, H, N, K, d, _ptr(X), _ptr(idx), _ptr(A), _ptr(LSE), _ptr(C), _ptr(cinv),
        _ptr(count), _ptr(Abar), _ptr(LSEbar), _ptr(ws), nbytes, _stream(dev)))
    return C, cinv, count, Abar, LSEbar


def build_memory(X, K: int, iters: int, A=None, LSE=None, *, workspace=None):
    """Cosine k-means with first-K initialisation followed by the state
    aggregation of the final partition (asm_build_memory): `iters` >= 1
    rounds of assignment and mean; the last round also merges the states
    (A, LSE) when they are given.  Returns (C, cinv, count, idx, Abar, LSEbar)."""
    _dev(X, "X")
    code = _dtype_code(X)
    H, N, d = X.shape
    dev = X.device
    C = torch.empty((H, K, d), dtype=X.dtype, device=dev)
    cinv = torch.empty((H, K), dtype=torch.float32, device=dev)
    idx = torch.empty((H, N), dtype=torch.int32, device=dev)
    count = torch.empty((H, K), dtype=torch.int32, device=dev)
    Abar = LSEbar = None
    if A is not None:
        _dev(A, "A", torch.float32)
        _dev(LSE, "LSE", torch.float32)
        Abar = torch.empty((H, K, d), dtype=torch.float32, device=dev)
        LSEbar = torch.empty((H, K), dtype=torch.float32, device=dev)
    nbytes = int(lib().asm_build_memory_ws(code, H, N, int(K), d))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_build_memory", lib().asm_build_memory(
        code, H, N, int(K), d, int(iters), _ptr(X), _ptr(A), _ptr(LSE), _ptr(C), _ptr(cinv),
        _ptr(Abar), _ptr(LSEbar), _ptr(count), _ptr(idx), _ptr(ws), nbytes, _stream(dev)))
    return C, cinv, count, idx, Abar, LSEbar


def build_index(C, S: int, iters: int, *, workspace=None):
    """Two-level index over each head's entries.  C [H, K, d].  Returns
    (SC [H, S, d], scinv [H, S], counts [H, S], offsets [H, S+1],
    members [H, K])."""
    _dev(C, "C")
    code = _dtype_code(C)
    H, K, d = C.shape
    dev = C.device
    SC = torch.empty((H, S, d), dtype=C.dtype, device=dev)
    scinv = torch.empty((H, S), dtype=torch.float32, device=dev)
    counts = torch.empty((H, S), dtype=torch.int32, device=dev)
    offsets = torch.empty((H, S + 1), dtype=torch.int32, device=dev)
    members = torch.empty((H, K), dtype=torch.int32, device=dev)
    nbytes = int(lib().asm_build_index_ws(code, H, K, S, d))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_build_index", lib().asm_build_index(
        code, H, K, int(S), d, int(iters), _ptr(C), _ptr(SC), _ptr(scinv), _ptr(counts),
        _ptr(offsets), _ptr(members), _ptr(ws), nbytes, _stream(dev)))
    return SC, scinv, counts, offsets, members


def group_index_rows(C, cinv, index):
    """The entry table grouped by super: (Cg [H, K, d], cginv [H, K]) with
    row i of head h the entry index[4][h, i] (the members of build_index)."""
    members = index[4]
    _dev(C, "C")
    _dev(cinv, "cinv", torch.float32)
    _dev(members, "members", torch.int32)
    code = _dtype_code(C)
    H, K, d = C.shape
    Cg = torch.empty_like(C)
    cginv = torch.empty((H, K), dtype=torch.float32, device=C.device)
    _check("asm_index_group_rows", lib().asm_index_group_rows(
        code, H, K, d, _ptr(C), _ptr(cinv), _ptr(members), _ptr(Cg), _ptr(cginv), _stream(C.device)))
    return Cg, cginv


def decode_step_hier(q, C, cinv, index, p: int, Abar, LSEbar, Kl, Vl, kv_start, kv_len,
                     max_kv_len: int, scale: float, *, grouped=None, out=None, out_lse=None,
                     out_idx=None, want_probes: bool = False, workspace=None):
    """Decode step with the two-level lookup.  `index` is the tuple returned
    by build_index; `grouped` (optional) the pair returned by
    group_index_rows.  Returns (out, out_lse, out_idx, probes | None)."""
    SC, scinv, _, offsets, members = index
    Cg, cginv = grouped if grouped is not None else (None, None)
    if Cg is not None:
        _dev(Cg, "Cg")
        _dev(cginv, "cginv", torch.float32)
    for t, n in ((q, "q"), (C, "C"), (SC, "SC"), (Kl, "Kl"), (Vl, "Vl")):
        _dev(t, n)
    _dev(cinv, "cinv", torch.float32)
    _dev(scinv, "scinv", torch.float32)
    _dev(offsets, "offsets", torch.int32)
    _dev(members, "members", torch.int32)
    _dev(Abar, "Abar", torch.float32)
    _dev(LSEbar, "LSEbar", torch.float32)
    _dev(kv_start, "kv_start", torch.int32)
    _dev(kv_len, "kv_len", torch.int32)
    code = _dtype_code(q)
    if Kl.stride() != Vl.stride() or Kl.shape != Vl.shape or Kl.stride(2) != 1:
        raise ValueError("Kl and Vl must share shape and strides, d contiguous")
    B, Hq, d = q.shape
    K = C.shape[1]
    S = SC.shape[1]
    Hkv, cap, _ = Kl.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    probes = torch.empty((B, Hq, p), dtype=torch.int32, device=dev) if want_probes else None
    nbytes = int(lib().asm_decode_step_hier_ws(code, B, Hq, Hkv, d, K, S, int(p), int(max_kv_len)))
    ws = _workspace(nbytes, dev, workspace)
    _check("asm_decode_step_hier", lib().asm_decode_step_hier(
        code, B, Hq, Hkv, d, K, S, int(p), float(scale), _ptr(q), _ptr(C), _ptr(cinv), _ptr(SC),
        _ptr(scinv), _ptr(offsets), _ptr(members), _ptr(Cg), _ptr(cginv), _ptr(Abar), _ptr(LSEbar),
        _ptr(Kl), _ptr(Vl),
        Kl.stride(0), Kl.stride(1), cap, _ptr(kv_start), _ptr(kv_len), int(max_kv_len), _ptr(out),
        _ptr(out_lse), _ptr(out_idx), _ptr(probes), _ptr(ws), nbytes, _stream(dev)))
    return out, out_lse, out_idx, probes

