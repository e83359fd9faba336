"""CPU chunkwise form of the KDA recurrence, fp64 numpy.

TEST INFRASTRUCTURE ONLY: imported by the tests (and nothing on the product
path).  It exists for two reasons:

* as an independent second algorithm whose agreement with the token-by-token
  oracle (``kda_oracle.c``) on tiny inputs pins both of them (brute-force
  equivalence for several chunk sizes), and
* to expose the per-chunk intermediates (cumulative log-decay, the masked
  key-key and query-key tiles, the triangular-solve result, the decay factor of
  the whole chunk) that the GPU's intra-chunk stage produces.

Source: the dev.to page "Kimi K3 Architecture: Scaling 2.8T Parameters ...",
section "The Sequence Bottleneck: Hybrid KDA and Gated MLA": chunkwise parallel
execution over 16-token tiles whose cumulative log-decay stays in (-80, 0),
so that the diagonal (within-chunk) and off-diagonal (state) tiles become
dense matrix products.  The pages give no chunk equations; the ones below are
derived from the recurrence S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T,
o_t = S_t^T q_t, with the state written as
    S_r = Diag(e^{G_r}) (S_0 + sum_{i<=r} Diag(e^{-G_i}) k_i u_i^T)
inside a chunk (G_r = inclusive chunk-local cumulative log-decay, u_i = the
delta-rule correction).  Chunks start at t = 0, C, 2C, ... and the last one may
be short.

Library primitives used as steps: ``@`` (matmul), ``np.cumsum``, ``np.tril``,
``scipy.linalg.solve_triangular`` (forward substitution).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

__all__ = ["gate_fp64", "chunk_head", "chunk_prefill"]


def gate_fp64(z: np.ndarray, a_h: float, g_min: float) -> np.ndarray:
    """g = g_min * Sigmoid(e^{A_h} z) in fp64 (dev.to page, gate equation).

    The logistic function is taken in the form that does not overflow."""
    x = np.exp(np.float64(a_h)) * np.asarray(z, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return np.float64(g_min) * out


def chunk_head(q, k, v, g, beta, S0, C, want_intermediates=False):
    """One head: q,k,g [T,dk], v [T,dv], beta [T], S0 [dk,dv] (fp64).

    Returns (o [T,dv], S_T [dk,dv]) and, if asked, a list with one dict per
    chunk holding G (cumulative log-decay), Akk (masked, beta-scaled key-key
    tile), Tm = (I + Akk)^{-1} Diag(beta), Aqk (masked query-key tile), gamma
    (e^{G_last}) -- all fp64, shapes for the chunk's own length."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    T, dk = k.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    inter = []
    for s in range(0, T, C):
        e = min(s + C, T)
        L = e - s
        G = np.cumsum(g[s:e], axis=0)                  # [L, dk]
        Kt = k[s:e] * np.exp(G)                        # k_r e^{G_r}
        Kh = k[s:e] * np.exp(-G)                       # k_i e^{-G_i}
        Qt = q[s:e] * np.exp(G)                        # q_r e^{G_r}
        Kdec = k[s:e] * np.exp(G[-1] - G)              # k_i e^{G_L - G_i}
        b = beta[s:e]
        Akk = np.tril(b[:, None] * (Kt @ Kh.T), -1)    # strictly lower
        Aqk = np.tril(Qt @ Kh.T, 0)                    # lower incl. diagonal
        Tm = solve_triangular(np.eye(L) + Akk, np.diag(b), lower=True,
                              unit_diagonal=True)
        # U = Tm (V - Kt S): the delta-rule corrections of the chunk
        U = Tm @ (v[s:e] - Kt @ S)
        o[s:e] = Qt @ S + Aqk @ U
        S = np.exp(G[-1])[:, None] * S + Kdec.T @ U
        if want_intermediates:
            inter.append(dict(G=G, Akk=Akk, Tm=Tm, Aqk=Aqk,
                              gamma=np.exp(G[-1])))
    if want_intermediates:
        return o, S, inter
    return o, S


def chunk_prefill(q, k, v, z, beta, A, g_min, S0, C):
    """Batched chunkwise prefill over [B,T,H,*] inputs (any float dtype).

    Returns o [B,T,H,dv], S_T [B,H,dk,dv] in fp64."""
    q, k, v, z = (np.asarray(x, dtype=np.float64) for x in (q, k, v, z))
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            g = gate_fp64(z[b, :, h], float(A[h]), g_min)
            s0 = np.zeros((dk, dv)) if S0 is None else S0[b, h]
            o[b, :, h], ST[b, h] = chunk_head(q[b, :, h], k[b, :, h],
                                              v[b, :, h], g, beta[b, :, h],
                                              s0, C)
    return o, ST
