"""ctypes marshalling for libkda (see ``include/kda.h`` for the contract)."""
from __future__ import annotations

import ctypes
import os

import torch

from .build import library_path

KDA_F32 = 0
KDA_BF16 = 1
KDA_CHUNK = 16
KDA_MAX_DECODE_TOKENS = 16

_STATUS = ["KDA_OK", "KDA_ERR_NULL_POINTER", "KDA_ERR_INVALID_SHAPE", "KDA_ERR_INVALID_VALUE",
           "KDA_ERR_UNSUPPORTED", "KDA_ERR_MISALIGNED", "KDA_ERR_WORKSPACE_TOO_SMALL",
           "KDA_ERR_ALIASING", "KDA_ERR_HIP"]


class KdaLibraryMissing(RuntimeError):
    """libkda.so is not built; there is no fallback implementation."""


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str, where: str):
        self.status = status
        name = _STATUS[status] if 0 <= status < len(_STATUS) else f"status {status}"
        super().__init__(f"{where}: {name}: {detail}")


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int

_SIGNATURES = {
    "kda_abi_version": ([], ctypes.c_int),
    "kda_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "kda_last_error": ([], ctypes.c_char_p),
    "kda_chunk_prefill_workspace_bytes": ([_i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "kda_chunk_prefill_segments": ([_i, _i, _i, _i, _i, _i], _i),
    "kda_chunk_prefill": ([_vp] * 6 + [ctypes.c_float, _vp, _vp, _vp] + [_i] * 6
                          + [_vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "kda_decode_step": ([_vp] * 6 + [ctypes.c_float, _vp, _vp] + [_i] * 5 + [_vp], ctypes.c_int),
    "kda_decode_tokens": ([_vp] * 6 + [ctypes.c_float, _vp, _vp, _vp] + [_i] * 6 + [_vp],
                          ctypes.c_int),
    "kda_chunk_prefill_paged": ([_vp] * 6 + [ctypes.c_float, _vp, _i, _vp, _vp, _vp] + [_i] * 6
                                + [_vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "kda_decode_step_paged": ([_vp] * 6 + [ctypes.c_float, _vp, _i, _vp, _vp] + [_i] * 5 + [_vp],
                              ctypes.c_int),
    "kda_decode_tokens_paged": ([_vp] * 6 + [ctypes.c_float, _vp, _i, _vp, _vp, _vp] + [_i] * 6
                                + [_vp], ctypes.c_int),
    "kda_chunk_prefill_segmented_workspace_bytes": ([_i] * 7, ctypes.c_size_t),
    "kda_chunk_prefill_segmented": ([_vp] * 6 + [ctypes.c_float, _vp, _vp, _vp] + [_i] * 7
                                    + [_vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "kda_chunk_backward_workspace_bytes": ([_i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "kda_chunk_backward": ([_vp] * 6 + [ctypes.c_float] + [_vp] * 10 + [_i] * 6
                           + [_vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "kda_gate_chunk_cumsum": ([_vp, _vp, ctypes.c_float, _vp] + [_i] * 5 + [_vp], ctypes.c_int),
    "kda_intra_chunk": ([_vp] * 5 + [ctypes.c_float, _vp, _vp, _vp] + [_i] * 5 + [_vp],
                        ctypes.c_int),
}


def lib():
    """The loaded libkda (raises KdaLibraryMissing if it was never built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise KdaLibraryMissing(
                f"{path} not found: build it with `python -m linear_attention_recurrence_05_amd.build`")
        L = ctypes.CDLL(path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().kda_abi_version())


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise KdaError(status, lib().kda_last_error().decode(), where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v/z/o must be bfloat16 or float32, got {t.dtype}")


def _require_contiguous(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def kda_chunk_prefill_workspace_bytes(B, T, H, d_k, d_v, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (KDA_BF16 if dtype == torch.bfloat16 else KDA_F32)
    return int(lib().kda_chunk_prefill_workspace_bytes(B, T, H, d_k, d_v, code))


def kda_chunk_prefill_segments(B, T, H, d_k, d_v, dtype) -> int:
    """C entry point kda_chunk_prefill_segments (1: a direct plan)."""
    code = dtype if isinstance(dtype, int) else (KDA_BF16 if dtype == torch.bfloat16 else KDA_F32)
    return int(lib().kda_chunk_prefill_segments(B, T, H, d_k, d_v, code))


def kda_chunk_prefill(q, k, v, z, beta, A, g_min, S0, o, S_T, workspace=None, stream=None):
    """C entry point kda_chunk_prefill on torch tensors (layouts of kda.h)."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, S0=S0, o=o, S_T=S_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kda_chunk_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                 float(g_min), _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv,
                                 _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "kda_chunk_prefill")


def kda_decode_step(q, k, v, z, beta, A, g_min, S, o, stream=None):
    """C entry point kda_decode_step on torch tensors; S is updated in place."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, S=S, o=o)
    B, H, dk = q.shape
    dv = v.shape[-1]
    st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                               float(g_min), _ptr(S), _ptr(o), B, H, dk, dv, _dtype_code(q),
                               _stream(stream))
    _check(st, "kda_decode_step")


def kda_decode_tokens(q, k, v, z, beta, A, g_min, S, S_out, o, stream=None):
    """C entry point kda_decode_tokens on torch tensors: T = q.shape[1] steps from
    the state S; the state after them goes to S_out (which may be S)."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, S=S, S_out=S_out, o=o)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    st = lib().kda_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                 float(g_min), _ptr(S), _ptr(S_out), _ptr(o), B, T, H, dk, dv,
                                 _dtype_code(q), _stream(stream))
    _check(st, "kda_decode_tokens")


def _slots(t, B):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.numel() != B:
        raise ValueError("a slot table is an int32 tensor of B entries")
    return t


def kda_chunk_prefill_paged(q, k, v, z, beta, A, g_min, pool, slots_in, slots_out, o,
                            workspace=None, stream=None):
    """C entry point kda_chunk_prefill_paged: states from pool[slots_in[b]] into
    pool[slots_out[b]] (either table may be None)."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, pool=pool, slots_in=slots_in,
                        slots_out=slots_out, o=o)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kda_chunk_prefill_paged(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                       float(g_min), _ptr(pool), pool.shape[0],
                                       _ptr(_slots(slots_in, B)), _ptr(_slots(slots_out, B)),
                                       _ptr(o), B, T, H, dk, dv, _dtype_code(q), _ptr(workspace),
                                       ws_bytes, _stream(stream))
    _check(st, "kda_chunk_prefill_paged")


def kda_decode_step_paged(q, k, v, z, beta, A, g_min, pool, slots, o, stream=None):
    """C entry point kda_decode_step_paged: pool[slots[b]] updated in place."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, pool=pool, slots=slots, o=o)
    B, H, dk = q.shape
    dv = v.shape[-1]
    st = lib().kda_decode_step_paged(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                     float(g_min), _ptr(pool), pool.shape[0],
                                     _ptr(_slots(slots, B)), _ptr(o), B, H, dk, dv,
                                     _dtype_code(q), _stream(stream))
    _check(st, "kda_decode_step_paged")


def kda_decode_tokens_paged(q, k, v, z, beta, A, g_min, pool, slots_in, slots_out, o,
                            stream=None):
    """C entry point kda_decode_tokens_paged: T steps from pool[slots_in[b]] into
    pool[slots_out[b]]."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, pool=pool, slots_in=slots_in,
                        slots_out=slots_out, o=o)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    st = lib().kda_decode_tokens_paged(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                       float(g_min), _ptr(pool), pool.shape[0],
                                       _ptr(_slots(slots_in, B)), _ptr(_slots(slots_out, B)),
                                       _ptr(o), B, T, H, dk, dv, _dtype_code(q), _stream(stream))
    _check(st, "kda_decode_tokens_paged")


def kda_gate_chunk_cumsum(z, A, g_min, G, stream=None):
    _require_contiguous(z=z, A=A, G=G)
    B, T, H, dk = z.shape
    st = lib().kda_gate_chunk_cumsum(_ptr(z), _ptr(A), float(g_min), _ptr(G), B, T, H, dk,
                                     _dtype_code(z), _stream(stream))
    _check(st, "kda_gate_chunk_cumsum")


def kda_intra_chunk(q, k, z, beta, A, g_min, Tm, Aqk, gamma, stream=None):
    _require_contiguous(q=q, k=k, z=z, beta=beta, A=A, Tm=Tm, Aqk=Aqk, gamma=gamma)
    B, T, H, dk = q.shape
    st = lib().kda_intra_chunk(_ptr(q), _ptr(k), _ptr(z), _ptr(beta), _ptr(A), float(g_min),
                               _ptr(Tm), _ptr(Aqk), _ptr(gamma), B, T, H, dk, _dtype_code(q),
                               _stream(stream))
    _check(st, "kda_intra_chunk")


# ----------------------------------------------------------------- allocating helpers

def chunk_prefill(q, k, v, z, beta, A, g_min=-5.0, S0=None, want_state=True, stream=None):
    """Allocate o (and S_T, workspace) with torch.empty and run kda_chunk_prefill.

    Returns (o, S_T or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if want_state else None
    nbytes = kda_chunk_prefill_workspace_bytes(B, T, H, dk, dv, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    kda_chunk_prefill(q, k, v, z, beta, A, g_min, S0, o, S_T, ws, stream)
    return o, S_T


def kda_chunk_prefill_segmented_workspace_bytes(B, T, H, d_k, d_v, n_seg, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (KDA_BF16 if dtype == torch.bfloat16 else KDA_F32)
    return int(lib().kda_chunk_prefill_segmented_workspace_bytes(B, T, H, d_k, d_v, n_seg, code))


def kda_chunk_prefill_segmented(q, k, v, z, beta, A, g_min, S0, o, S_T, n_seg, workspace,
                                stream=None):
    """C entry point kda_chunk_prefill_segmented on torch tensors (layouts of kda.h)."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, S0=S0, o=o, S_T=S_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kda_chunk_prefill_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta),
                                           _ptr(A), float(g_min), _ptr(S0), _ptr(o), _ptr(S_T),
                                           B, T, H, dk, dv, int(n_seg), _dtype_code(q),
                                           _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "kda_chunk_prefill_segmented")


def chunk_prefill_segmented(q, k, v, z, beta, A, n_seg, g_min=-5.0, S0=None, want_state=True,
                            stream=None):
    """Allocate o (and S_T, workspace) with torch.empty and run
    kda_chunk_prefill_segmented.  Returns (o, S_T or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if want_state else None
    nbytes = kda_chunk_prefill_segmented_workspace_bytes(B, T, H, dk, dv, n_seg, q.dtype)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    kda_chunk_prefill_segmented(q, k, v, z, beta, A, g_min, S0, o, S_T, n_seg, ws, stream)
    return o, S_T


def kda_chunk_backward_workspace_bytes(B, T, H, d_k, d_v, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (KDA_BF16 if dtype == torch.bfloat16 else KDA_F32)
    return int(lib().kda_chunk_backward_workspace_bytes(B, T, H, d_k, d_v, code))


def kda_chunk_backward(q, k, v, z, beta, A, g_min, S0, dO, dS_T, dq, dk, dv, dz, dbeta, dA, dS0,
                       workspace, stream=None):
    """C entry point kda_chunk_backward on torch tensors (layouts of kda.h)."""
    _require_contiguous(q=q, k=k, v=v, z=z, beta=beta, A=A, S0=S0, dO=dO, dS_T=dS_T, dq=dq,
                        dk=dk, dv=dv, dz=dz, dbeta=dbeta, dA=dA, dS0=dS0)
    B, T, H, dkk = q.shape
    dvv = v.shape[-1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kda_chunk_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                  float(g_min), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(dz), _ptr(dbeta), _ptr(dA), _ptr(dS0),
                                  B, T, H, dkk, dvv, _dtype_code(q), _ptr(workspace), ws_bytes,
                                  _stream(stream))
    _check(st, "kda_chunk_backward")


def chunk_backward(q, k, v, z, beta, A, dO, g_min=-5.0, S0=None, dS_T=None, want_dS0=True,
                   stream=None):
    """Allocate the gradients (and the workspace) with torch.empty and run
    kda_chunk_backward.  Returns a dict with dq, dk, dv, dz, dbeta, dA, dS0."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
             dz=torch.empty_like(z),
             dbeta=torch.empty((B, T, H), dtype=torch.float32, device=q.device),
             dA=torch.empty((H,), dtype=torch.float32, device=q.device),
             dS0=(torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
                  if want_dS0 else None))
    nbytes = kda_chunk_backward_workspace_bytes(B, T, H, dk, dv, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    kda_chunk_backward(q, k, v, z, beta, A, g_min, S0, dO, dS_T, g["dq"], g["dk"], g["dv"],
                       g["dz"], g["dbeta"], g["dA"], g["dS0"], ws, stream)
    return g


def decode_tokens(q, k, v, z, beta, A, S, S_out=None, g_min=-5.0, stream=None):
    """Allocate o (and S_out unless given) and run kda_decode_tokens.
    Returns (o, S_out)."""
    B, T, H, dk = q.shape
    o = torch.empty((B, T, H, v.shape[-1]), dtype=q.dtype, device=q.device)
    if S_out is None:
        S_out = torch.empty_like(S)
    kda_decode_tokens(q, k, v, z, beta, A, g_min, S, S_out, o, stream)
    return o, S_out


def decode_step(q, k, v, z, beta, A, S, g_min=-5.0, stream=None):
    """Allocate o and run kda_decode_step (S updated in place).  Returns o."""
    o = torch.empty((q.shape[0], q.shape[1], v.shape[-1]), dtype=q.dtype, device=q.device)
    kda_decode_step(q, k, v, z, beta, A, g_min, S, o, stream)
    return o
