"""fp64 CPU oracle for the KDA gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and the GPU library never calls it.

* ``kda_oracle.c``  -- token-by-token recurrence in C, fp64 (``liboracle.so``),
  and its exact gradients by a reverse sweep over the stored states
* ``chunkwise.py``  -- an independent chunkwise form in numpy, fp64

The C library is built with gcc by :func:`build` (``oracle/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build, library_path

__all__ = ["Oracle", "build", "library_path", "default", "gate",
           "gate_chunk_cumsum", "prefill", "decode", "backward", "max_threads"]

_dbl_p = ctypes.POINTER(ctypes.c_double)
_flt_p = ctypes.POINTER(ctypes.c_float)


def _f32(x):
    """Contiguous float32 numpy copy of a numpy array or torch tensor.

    bf16 and fp32 values widen to float32 exactly."""
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu")
        if x.dtype != torch.float32:
            x = x.float()
        x = x.contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _fp(a):
    return a.ctypes.data_as(_flt_p)


def _dp(a):
    return a.ctypes.data_as(_dbl_p)


class Oracle:
    """ctypes wrapper around one build of ``kda_oracle.c``."""

    def __init__(self, path: str | None = None):
        # KDA_ORACLE_LIB: another build of the same source (the sanitizer
        # test runs the pins against one)
        path = path or os.environ.get("KDA_ORACLE_LIB") or library_path()
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        L = ctypes.c_long
        lib.kda_oracle_gate.argtypes = [_flt_p, _flt_p, ctypes.c_double, L, L, L, L, _dbl_p]
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_gate_chunk_cumsum.argtypes = [_flt_p, _flt_p, ctypes.c_double,
                                                     L, L, L, L, L, _dbl_p]
        lib.kda_oracle_gate_chunk_cumsum.restype = None
        lib.kda_oracle_prefill.argtypes = ([_flt_p] * 6 + [ctypes.c_double, _flt_p, _dbl_p,
                                                           _dbl_p, L, L, L, L, L, ctypes.c_int])
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = ([_flt_p] * 6 + [ctypes.c_double, _dbl_p, _dbl_p,
                                                          L, L, L, L, ctypes.c_int])
        lib.kda_oracle_decode.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = ([_flt_p] * 6 + [ctypes.c_double] + [_flt_p] * 3
                                            + [_dbl_p] * 7 + [L, L, L, L, L, ctypes.c_int])
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_max_threads.argtypes = []
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.kda_oracle_max_threads())

    def gate(self, z, A, g_min):
        """g = g_min * Sigmoid(e^{A_h} z) for z [B,T,H,dk] -> fp64 same shape."""
        z, A = _f32(z), _f32(A)
        B, T, H, dk = z.shape
        g = np.empty(z.shape, dtype=np.float64)
        self.lib.kda_oracle_gate(_fp(z), _fp(A), float(g_min), B, T, H, dk, _dp(g))
        return g

    def gate_chunk_cumsum(self, z, A, g_min, chunk=16):
        """Chunk-local inclusive cumulative log-decay, z [B,T,H,dk] -> fp64."""
        z, A = _f32(z), _f32(A)
        B, T, H, dk = z.shape
        G = np.empty(z.shape, dtype=np.float64)
        self.lib.kda_oracle_gate_chunk_cumsum(_fp(z), _fp(A), float(g_min), B, T, H,
                                              dk, int(chunk), _dp(G))
        return G

    def prefill(self, q, k, v, z, beta, A, g_min, S0=None, nthreads=0,
                want_state=True):
        """Token-by-token fp64 prefill.

        q,k,z [B,T,H,dk], v [B,T,H,dv], beta [B,T,H], A [H], S0 [B,H,dk,dv] or
        None.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv] or None), fp64 numpy."""
        q, k, v, z, beta, A = (_f32(x) for x in (q, k, v, z, beta, A))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        s0 = None if S0 is None else _f32(S0)
        o = np.empty((B, T, H, dv), dtype=np.float64)
        ST = np.empty((B, H, dk, dv), dtype=np.float64) if want_state else None
        rc = self.lib.kda_oracle_prefill(
            _fp(q), _fp(k), _fp(v), _fp(z), _fp(beta), _fp(A), float(g_min),
            None if s0 is None else _fp(s0), _dp(o), None if ST is None else _dp(ST),
            B, T, H, dk, dv, int(nthreads))
        if rc != 0:
            raise MemoryError("oracle prefill: allocation failed")
        return o, ST

    def decode(self, q, k, v, z, beta, A, g_min, S, nthreads=0):
        """One fp64 decode step.  q,k,z [B,H,dk], v [B,H,dv], beta [B,H];
        S [B,H,dk,dv] fp64 numpy array, updated in place.  Returns o [B,H,dv]."""
        q, k, v, z, beta, A = (_f32(x) for x in (q, k, v, z, beta, A))
        B, H, dk = k.shape
        dv = v.shape[-1]
        if not (isinstance(S, np.ndarray) and S.dtype == np.float64
                and S.flags.c_contiguous and S.shape == (B, H, dk, dv)):
            raise TypeError("S must be a C-contiguous float64 array [B,H,dk,dv]")
        o = np.empty((B, H, dv), dtype=np.float64)
        rc = self.lib.kda_oracle_decode(_fp(q), _fp(k), _fp(v), _fp(z), _fp(beta), _fp(A),
                                        float(g_min), _dp(S), _dp(o), B, H, dk, dv,
                                        int(nthreads))
        if rc != 0:
            raise MemoryError("oracle decode: allocation failed")
        return o

    def backward(self, q, k, v, z, beta, A, g_min, S0, dO, dST=None, nthreads=0):
        """fp64 gradients of L = sum(dO * o) + sum(dST * S_T) through the
        token-by-token prefill.  Shapes as in :meth:`prefill`; dO [B,T,H,dv],
        dST [B,H,dk,dv] or None.  Returns a dict of fp64 arrays dq, dk, dv,
        dz, dbeta, dA, dS0."""
        q, k, v, z, beta, A, dO = (_f32(x) for x in (q, k, v, z, beta, A, dO))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        s0 = None if S0 is None else _f32(S0)
        dst = None if dST is None else _f32(dST)
        out = dict(dq=np.empty((B, T, H, dk)), dk=np.empty((B, T, H, dk)),
                   dv=np.empty((B, T, H, dv)), dz=np.empty((B, T, H, dk)),
                   dbeta=np.empty((B, T, H)), dA=np.empty((H,)),
                   dS0=np.empty((B, H, dk, dv)))
        rc = self.lib.kda_oracle_backward(
            _fp(q), _fp(k), _fp(v), _fp(z), _fp(beta), _fp(A), float(g_min),
            None if s0 is None else _fp(s0), _fp(dO), None if dst is None else _fp(dst),
            *(_dp(out[n]) for n in ("dq", "dk", "dv", "dz", "dbeta", "dA", "dS0")),
            B, T, H, dk, dv, int(nthreads))
        if rc != 0:
            raise MemoryError("oracle backward: allocation failed")
        return out


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from the committed ``kda_oracle.c``."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads() -> int:
    return default().max_threads()


def gate(z, A, g_min):
    return default().gate(z, A, g_min)


def gate_chunk_cumsum(z, A, g_min, chunk=16):
    return default().gate_chunk_cumsum(z, A, g_min, chunk)


def prefill(q, k, v, z, beta, A, g_min, S0=None, nthreads=0, want_state=True):
    return default().prefill(q, k, v, z, beta, A, g_min, S0, nthreads, want_state)


def decode(q, k, v, z, beta, A, g_min, S, nthreads=0):
    return default().decode(q, k, v, z, beta, A, g_min, S, nthreads)


def backward(q, k, v, z, beta, A, g_min, S0, dO, dST=None, nthreads=0):
    return default().backward(q, k, v, z, beta, A, g_min, S0, dO, dST, nthreads)
