"""CPU chunkwise form of the KDA recurrence, fp64 numpy.

TEST INFRASTRUCTURE ONLY: imported by the tests (and nothing on the product
path).  It exists for two reasons:

* as an independent second algorithm whose agreement with the token-by-token
  oracle (``kda_oracle.c``) on tiny inputs pins both of them (brute-force
  equivalence for several chunk sizes), and
* to expose the per-chunk intermediates (cumulative log-decay, the masked
  key-key and query-key tiles, the triangular-solve result, the decay factor of
  the whole chunk) that the GPU's intra-chunk stage produces, and
* to differentiate those chunk equations (:func:`chunk_head_backward`), an
  independent algorithm for the gradients whose agreement with the
  token-by-token reverse sweep pins both, and the chunk-level form of the
  backward (a chain of state gradients over chunks, the rest parallel per
  chunk).

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

__all__ = ["gate_fp64", "chunk_head", "chunk_prefill", "chunk_head_backward"]


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


def chunk_head_backward(q, k, v, g, beta, S0, dO, dST, C):
    """Gradients of one head's chunkwise prefill, chunk by chunk in reverse.

    Same inputs as :func:`chunk_head` plus dO [T,dv] and dST [dk,dv] (the
    incoming gradients of o and S_T).  Returns dq, dk, dv, dg [T,*], dbeta [T]
    and dS0, all fp64.  The pages give no backward pass; this differentiates
    the chunk equations above step by step (reverse order of the forward):
      O = Qt S + Aqk U,  S' = Diag(gamma) S + Kdec^T U,  U = Tm (V - Kt S),
      Tm = (I + Akk)^{-1} Diag(beta),  Akk = tril_-1(Diag(beta) Kt Kh^T),
      Aqk = tril_0(Qt Kh^T),  Kt = K e^G,  Kh = K e^-G,  Qt = Q e^G,
      Kdec = K e^{G_L - G},  gamma = e^{G_L},  G = cumsum of g in the chunk.
    """
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T, dk = k.shape
    # forward, keeping each chunk's start state
    S = np.array(S0, dtype=np.float64, copy=True)
    starts = []
    for s in range(0, T, C):
        e = min(s + C, T)
        starts.append(S.copy())
        G = np.cumsum(g[s:e], axis=0)
        Kt, Kh = k[s:e] * np.exp(G), k[s:e] * np.exp(-G)
        Kdec = k[s:e] * np.exp(G[-1] - G)
        b = beta[s:e]
        Akk = np.tril(b[:, None] * (Kt @ Kh.T), -1)
        Tm = solve_triangular(np.eye(e - s) + Akk, np.diag(b), lower=True, unit_diagonal=True)
        U = Tm @ (v[s:e] - Kt @ S)
        S = np.exp(G[-1])[:, None] * S + Kdec.T @ U
    dq, dkk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    dbeta = np.zeros_like(beta)
    dS = np.array(dST, dtype=np.float64, copy=True)          # gradient of the chunk's end state
    for n, s in reversed(list(enumerate(range(0, T, C)))):
        e = min(s + C, T)
        L = e - s
        S = starts[n]
        G = np.cumsum(g[s:e], axis=0)
        Ex = np.exp(G)
        Kt, Kh, Qt = k[s:e] * Ex, k[s:e] / Ex, q[s:e] * Ex
        gam = np.exp(G[-1])
        Kdec = k[s:e] * (gam / Ex)
        b = beta[s:e]
        P = Kt @ Kh.T
        Akk = np.tril(b[:, None] * P, -1)
        M = np.eye(L) + Akk
        Ninv = solve_triangular(M, np.eye(L), lower=True, unit_diagonal=True)
        Tm = Ninv * b[None, :]
        W = v[s:e] - Kt @ S
        U = Tm @ W
        Aqk = np.tril(Qt @ Kh.T, 0)
        dOc = dO[s:e]
        # S' = Diag(gam) S + Kdec^T U
        dgam = np.sum(dS * S, axis=1)
        dS_prev = gam[:, None] * dS
        dKdec = U @ dS.T
        dU = Kdec @ dS
        # O = Qt S + Aqk U
        dQt = dOc @ S.T
        dS_prev += Qt.T @ dOc
        dAqk = np.tril(dOc @ U.T, 0)
        dU += Aqk.T @ dOc
        dQt += dAqk @ Kh
        dKh = dAqk.T @ Qt
        # U = Tm W,  W = V - Kt S
        dTm = dU @ W.T
        dW = Tm.T @ dU
        dv[s:e] = dW
        dKt = -dW @ S.T
        dS_prev += -Kt.T @ dW
        # Tm = M^{-1} Diag(beta),  M = I + tril_-1(Diag(beta) P)
        dbeta[s:e] += np.sum(dTm * Ninv, axis=0)
        dN = dTm * b[None, :]
        dM = -Ninv.T @ dN @ Ninv.T
        dA = np.tril(dM, -1)
        dbeta[s:e] += np.sum(dA * P, axis=1)
        dP = b[:, None] * dA
        dKt += dP @ Kh
        dKh += dP.T @ Kt
        # decay factors: Kt = K e^G, Kh = K e^-G, Qt = Q e^G, Kdec = K e^{G_L - G}, gam = e^{G_L}
        dkk[s:e] = dKt * Ex + dKh / Ex + dKdec * (gam / Ex)
        dq[s:e] = dQt * Ex
        dG = dKt * Kt - dKh * Kh + dQt * Qt - dKdec * Kdec
        dG[-1] += np.sum(dKdec * Kdec, axis=0) + dgam * gam
        dg[s:e] = np.cumsum(dG[::-1], axis=0)[::-1]          # G_r = sum_{i<=r} g_i
        dS = dS_prev
    return dict(dq=dq, dk=dkk, dv=dv, dg=dg, dbeta=dbeta, dS0=dS)
