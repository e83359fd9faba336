"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` if the oracle disagrees with:

* numbers the pages print (``golden/gate_bounds.json``);
* closed forms (gate at z = 0, beta = 0, the scalar exponential moving
  average of ``golden/scalar_ema.json``);
* reductions to textbook forms (exact retrieval with beta = 1 and unit keys;
  causal linear attention with alpha = 1 and orthonormal keys);
* a library routine (``scipy.special.expit`` for the logistic function,
  ``np.cumsum``);
* an independent algorithm (the numpy chunkwise form) on tiny inputs, for
  several chunk sizes; and
* structural invariants (continuation, linearity, permutation equivariance,
  head and batch independence, decode = one-token prefill).

``test_oracle_pins.py`` runs them on the committed oracle;
``test_oracle_mutants.py`` runs them on deliberately broken builds and expects
each break to trip at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

from oracle.chunkwise import chunk_head_backward, chunk_prefill, gate_fp64

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _unit(x):
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


def _inputs(rng, B, T, H, dk, dv, s0=True):
    q = _unit(rng.standard_normal((B, T, H, dk)))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    z = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    beta = expit(rng.standard_normal((B, T, H))).astype(np.float32)
    A = rng.uniform(-1, 1, H).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if s0 else None
    return q, k, v, z, beta, A, S0


def _hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


# --------------------------------------------------------------------------- gate

def pin_gate_at_zero(orc):
    """z = 0: Sigmoid(0) = 1/2, so g = g_min / 2 whatever A is."""
    z = np.zeros((1, 3, 4, 8), np.float32)
    A = np.array([-1.0, -0.25, 0.5, 1.0], np.float32)
    for g_min in (-5.0, -1.3, 0.0):
        g = orc.gate(z, A, g_min)
        np.testing.assert_allclose(g, g_min / 2.0, rtol=0, atol=1e-15)
    # the value a = e^{-2.5} = 0.0820849986238988 for g_min = -5
    a = math.exp(orc.gate(z, A, -5.0)[0, 0, 0, 0])
    assert abs(a - 0.0820849986238988) < 1e-15


def pin_gate_library(orc):
    """g = g_min * expit(e^{A_h} z), expit from scipy."""
    rng = np.random.default_rng(11)
    z = (3.0 * rng.standard_normal((2, 5, 3, 16))).astype(np.float32)
    A = rng.uniform(-1, 1, 3).astype(np.float32)
    g = orc.gate(z, A, -5.0)
    ref = -5.0 * expit(np.exp(A.astype(np.float64))[None, None, :, None] * z.astype(np.float64))
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-300)


def pin_gate_bounds_printed(orc):
    """The page's numbers: g in (g_min, 0), a in (e^{g_min}, 1), e^{-5} ~ 6.7e-3;
    g decreasing in z for g_min < 0."""
    gb = _golden("gate_bounds.json")
    g_min = gb["g_min"]
    assert round(math.exp(g_min), 4) == gb["alpha_lower_bound_printed"]
    rng = np.random.default_rng(12)
    z = rng.uniform(-10, 10, (1, 64, 2, 32)).astype(np.float32)
    A = np.array([-1.0, 1.0], np.float32)
    g = orc.gate(z, A, g_min)
    a = np.exp(g)
    assert np.all(g > g_min) and np.all(g < 0.0)
    assert np.all(a > gb["alpha_lower_bound_printed"] * 0.99) and np.all(a < 1.0)
    assert np.all(a > math.exp(g_min))
    zs = np.sort(z.reshape(-1)).reshape(1, -1, 1, 1)
    gs = orc.gate(zs, np.array([0.3], np.float32), g_min).reshape(-1)
    assert np.all(np.diff(gs) <= 0.0) and gs[0] > gs[-1]


def pin_chunk_cumsum(orc):
    """Chunk-local cumulative log-decay = per-chunk np.cumsum of the gate, reset
    at t = 0, 16, 32, ...; over 16-token tiles it stays inside (-80, 0)."""
    gb = _golden("gate_bounds.json")
    C = gb["tile_tokens"]
    lo, hi = gb["tile_cumulative_log_decay_open_interval"]
    rng = np.random.default_rng(13)
    T = 3 * C + 5
    z = rng.uniform(-8, 8, (2, T, 2, 8)).astype(np.float32)
    A = np.array([-0.5, 1.0], np.float32)
    G = orc.gate_chunk_cumsum(z, A, gb["g_min"], C)
    g = gb["g_min"] * expit(np.exp(A.astype(np.float64))[None, None, :, None] * z)
    for s in range(0, T, C):
        ref = np.cumsum(g[:, s:s + C], axis=1)
        np.testing.assert_allclose(G[:, s:s + C], ref, rtol=1e-13, atol=1e-13)
    assert np.all(G > lo) and np.all(G < hi)
    # near the extreme: every z large and positive drives each g towards g_min
    zmax = np.full((1, C, 1, 4), 20.0, np.float32)
    Gm = orc.gate_chunk_cumsum(zmax, np.array([0.0], np.float32), gb["g_min"], C)
    assert np.all(Gm[:, -1] > lo) and np.all(Gm[:, -1] < lo + 1e-6)


# --------------------------------------------------------------------------- recurrence

def pin_scalar_ema(orc):
    """d_k = d_v = 1, k = +-1: the hand-worked moving average."""
    ema = _golden("scalar_ema.json")
    g_min = -2.0 * math.log(2.0)
    T = len(ema["v"])
    for case in ema["cases"]:
        shape = (1, T, 1, 1)
        q = np.full(shape, case["q"], np.float32)
        k = np.full(shape, case["k"], np.float32)
        v = np.array(ema["v"], np.float32).reshape(shape)
        z = np.full(shape, ema["z"], np.float32)
        beta = np.full((1, T, 1), ema["beta"], np.float32)
        A = np.array([ema["A"]], np.float32)
        S0 = np.full((1, 1, 1, 1), case["s0"], np.float32)
        o, ST = orc.prefill(q, k, v, z, beta, A, g_min, S0)
        np.testing.assert_allclose(o.reshape(-1), case["o"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ST.reshape(-1), [case["s_T"]], rtol=0, atol=1e-13)


def pin_beta_zero(orc):
    """beta = 0: nothing is written, S_T = Diag(e^{sum g}) S0 and
    o_t = S0^T (e^{G_t} * q_t) with G_t the running sum from the start."""
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 2, 21, 2, 6, 4
    q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
    beta = np.zeros_like(beta)
    o, ST = orc.prefill(q, k, v, z, beta, A, -5.0, S0)
    g = -5.0 * expit(np.exp(A.astype(np.float64))[None, None, :, None] * z)
    Gt = np.cumsum(g, axis=1)                          # [B,T,H,dk]
    ST_ref = np.exp(Gt[:, -1])[..., None] * S0         # [B,H,dk,dv]
    np.testing.assert_allclose(ST, ST_ref, rtol=1e-12, atol=1e-14)
    o_ref = np.einsum("bthc,bhcj->bthj", np.exp(Gt) * q, S0.astype(np.float64))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    o0, ST0 = orc.prefill(q, k, v, z, beta, A, -5.0, None)
    assert np.all(o0 == 0.0) and np.all(ST0 == 0.0)


def pin_exact_retrieval(orc):
    """beta = 1 and |k_t| = 1: S_t^T k_t = v_t for any retention and any
    earlier state, so o_t = v_t when q_t = k_t."""
    rng = np.random.default_rng(15)
    B, T, H, d = 1, 24, 2, 16
    Hd = (_hadamard(d) / 4.0).astype(np.float32)      # rows: exact unit vectors
    idx = rng.integers(0, d, (B, T, H))
    sign = rng.choice([-1.0, 1.0], (B, T, H, 1)).astype(np.float32)
    k = Hd[idx] * sign
    _, _, v, z, _, A, S0 = _inputs(rng, B, T, H, d, d)
    beta = np.ones((B, T, H), np.float32)
    o, _ = orc.prefill(k, k, v, z, beta, A, -5.0, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def pin_linear_attention(orc):
    """alpha = 1 (g_min = 0), S0 = 0 and mutually orthonormal keys: the erase
    term vanishes and o_t = sum_{i<=t} beta_i (q_t . k_i) v_i, i.e. causal
    linear attention O = tril(Q K^T) Diag(beta) V."""
    rng = np.random.default_rng(16)
    d, T, dv = 16, 16, 8
    Hd = (_hadamard(d) / 4.0).astype(np.float32)
    k = Hd[rng.permutation(d)][:T].reshape(1, T, 1, d)
    q = _unit(rng.standard_normal((1, T, 1, d)))
    v = rng.standard_normal((1, T, 1, dv)).astype(np.float32)
    z = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    beta = expit(rng.standard_normal((1, T, 1))).astype(np.float32)
    A = np.array([0.3], np.float32)
    o, ST = orc.prefill(q, k, v, z, beta, A, 0.0, None)
    Q, K, V = (x[0, :, 0].astype(np.float64) for x in (q, k, v))
    bt = beta[0, :, 0].astype(np.float64)
    O_ref = np.tril(Q @ K.T) @ (bt[:, None] * V)
    np.testing.assert_allclose(o[0, :, 0], O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST[0, 0], K.T @ (bt[:, None] * V), rtol=0, atol=1e-12)


def pin_alpha_one_beta_zero(orc):
    """The literal alpha = 1, beta = 0 case: the state never changes,
    S_T = S0 and o_t = S0^T q_t."""
    rng = np.random.default_rng(17)
    q, k, v, z, beta, A, S0 = _inputs(rng, 1, 9, 2, 8, 5)
    beta = np.zeros_like(beta)
    o, ST = orc.prefill(q, k, v, z, beta, A, 0.0, S0)
    np.testing.assert_array_equal(ST, S0.astype(np.float64))
    np.testing.assert_allclose(o, np.einsum("bthc,bhcj->bthj", q.astype(np.float64),
                                            S0.astype(np.float64)), rtol=1e-13, atol=1e-15)


def pin_chunkwise_equivalence(orc):
    """Token-by-token recurrence == independent chunkwise form, C in
    {1, 5, 7, 16, T}, ragged T, nonzero S0, g_min = -5."""
    rng = np.random.default_rng(18)
    B, T, H, dk, dv = 2, 37, 2, 8, 6
    q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
    o, ST = orc.prefill(q, k, v, z, beta, A, -5.0, S0)
    for C in (1, 5, 7, 16, T):
        o2, ST2 = chunk_prefill(q, k, v, z, beta, A, -5.0, S0, C)
        np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ST, ST2, rtol=0, atol=1e-12)


def pin_continuation(orc):
    """prefill(T1) then prefill(T2, S0 = S_T1) == prefill(T1 + T2), bitwise."""
    rng = np.random.default_rng(19)
    q, k, v, z, beta, A, S0 = _inputs(rng, 2, 30, 2, 8, 8)
    o, ST = orc.prefill(q, k, v, z, beta, A, -5.0, S0)
    cut = 13
    oa, Sa = orc.prefill(q[:, :cut], k[:, :cut], v[:, :cut], z[:, :cut], beta[:, :cut],
                         A, -5.0, S0)
    # the state handed over is the fp64 state rounded to float32 by the
    # interface; rerun the full sequence from the same point for a bitwise check
    Sa32 = Sa.astype(np.float32)
    ob, Sb = orc.prefill(q[:, cut:], k[:, cut:], v[:, cut:], z[:, cut:], beta[:, cut:],
                         A, -5.0, Sa32)
    np.testing.assert_array_equal(oa, o[:, :cut])
    np.testing.assert_allclose(ob, o[:, cut:], rtol=0, atol=1e-6)
    np.testing.assert_allclose(Sb, ST, rtol=0, atol=1e-6)
    # exact (no rounding of the handed-over state) via the chunkwise form
    o2, S2 = chunk_prefill(q[:, cut:], k[:, cut:], v[:, cut:], z[:, cut:], beta[:, cut:],
                           A, -5.0, Sa, 16)
    np.testing.assert_allclose(o2, o[:, cut:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, ST, rtol=0, atol=1e-12)


def pin_linearity(orc):
    """(V, S0) -> (O, S_T) is linear for fixed q, k, z, beta, A."""
    rng = np.random.default_rng(20)
    q, k, _, z, beta, A, _ = _inputs(rng, 1, 19, 2, 8, 8)

    def coarse(shape):  # values on a 2^-10 grid, so a*x + b*y below is exact in fp32
        return (np.round(rng.standard_normal(shape) * 1024.0) / 1024.0).astype(np.float32)

    v1, v2 = coarse((1, 19, 2, 8)), coarse((1, 19, 2, 8))
    S1, S2 = coarse((1, 2, 8, 8)), coarse((1, 2, 8, 8))
    a, b = 0.75, -2.5
    o1, T1 = orc.prefill(q, k, v1, z, beta, A, -5.0, S1)
    o2, T2 = orc.prefill(q, k, v2, z, beta, A, -5.0, S2)
    o3, T3 = orc.prefill(q, k, (a * v1 + b * v2).astype(np.float32), z, beta, A, -5.0,
                         (a * S1 + b * S2).astype(np.float32))
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-11)
    np.testing.assert_allclose(T3, a * T1 + b * T2, rtol=0, atol=1e-11)


def pin_structure(orc):
    """Permuting value channels permutes outputs; heads and batch rows are
    independent (batched run == per-slice runs)."""
    rng = np.random.default_rng(21)
    B, T, H, dk, dv = 2, 17, 3, 8, 6
    q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
    o, ST = orc.prefill(q, k, v, z, beta, A, -5.0, S0)
    perm = rng.permutation(dv)
    op, STp = orc.prefill(q, k, v[..., perm], z, beta, A, -5.0, S0[..., perm])
    np.testing.assert_array_equal(op, o[..., perm])
    np.testing.assert_array_equal(STp, ST[..., perm])
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            o1, S1 = orc.prefill(q[sl], k[sl], v[sl], z[sl], beta[b:b + 1, :, h:h + 1],
                                 A[h:h + 1], -5.0, S0[b:b + 1, h:h + 1])
            np.testing.assert_array_equal(o1[0, :, 0], o[b, :, h])
            np.testing.assert_array_equal(S1[0, 0], ST[b, h])


def pin_decode_matches_prefill(orc):
    """T decode steps from S0 == a T-token prefill from S0 (bitwise)."""
    rng = np.random.default_rng(22)
    B, T, H, dk, dv = 3, 5, 2, 8, 4
    q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
    o, ST = orc.prefill(q, k, v, z, beta, A, -5.0, S0)
    S = S0.astype(np.float64).copy()
    for t in range(T):
        ot = orc.decode(q[:, t], k[:, t], v[:, t], z[:, t], beta[:, t], A, -5.0, S)
        np.testing.assert_array_equal(ot, o[:, t])
    np.testing.assert_array_equal(S, ST)


# --------------------------------------------------------------------------- gradients

def _loss_fd(x, dO, dST, g_min, C):
    """L = sum(dO o) + sum(dST S_T) through the fp64 chunkwise form."""
    o, ST = chunk_prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], g_min,
                          x["S0"], C)
    return float(np.sum(dO * o) + np.sum(dST * ST))


def pin_backward_finite_difference(orc):
    """Gradients of L = sum(dO o) + sum(dST S_T) against Richardson-extrapolated
    central differences of L through the independent fp64 chunkwise form, along
    random directions, for every input (q, k, v, z, beta, A, S0)."""
    rng = np.random.default_rng(31)
    B, T, H, dk, dv = 2, 11, 2, 4, 3
    for g_min in (-5.0, -1.3):
        q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
        dO = rng.standard_normal((B, T, H, dv))
        dST = rng.standard_normal((B, H, dk, dv))
        gr = orc.backward(q, k, v, z, beta, A, g_min, S0, dO.astype(np.float32),
                          dST.astype(np.float32))
        dO = dO.astype(np.float32).astype(np.float64)
        dST = dST.astype(np.float32).astype(np.float64)
        x0 = {n: a.astype(np.float64) for n, a in
              dict(q=q, k=k, v=v, z=z, beta=beta, A=A, S0=S0).items()}
        names = dict(q="dq", k="dk", v="dv", z="dz", beta="dbeta", A="dA", S0="dS0")
        for n, gname in names.items():
            for _ in range(2):
                d = rng.standard_normal(x0[n].shape)

                def D(h):
                    xp = dict(x0)
                    xm = dict(x0)
                    xp[n] = x0[n] + h * d
                    xm[n] = x0[n] - h * d
                    return (_loss_fd(xp, dO, dST, g_min, 4) - _loss_fd(xm, dO, dST, g_min, 4)) / (2 * h)

                h = 1e-3
                fd = (4.0 * D(h / 2) - D(h)) / 3.0
                an = float(np.sum(gr[gname] * d))
                scale = max(abs(fd), float(np.linalg.norm(gr[gname]) * np.linalg.norm(d)), 1e-3)
                assert abs(an - fd) <= 1e-8 * scale, (n, g_min, an, fd)


def pin_backward_beta_zero(orc):
    """beta = 0 closed form: o_t = S0^T (e^{cumsum g} q_t), S_T = Diag(e^{sum g}) S0,
    so dq_t = e^{cumsum g} (S0 dO_t), dk = dv = 0 and
    dS0 = sum_t (e^{cumsum g} q_t) dO_t^T + Diag(e^{sum g}) dST."""
    rng = np.random.default_rng(32)
    B, T, H, dk, dv = 2, 9, 3, 5, 4
    q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
    beta = np.zeros_like(beta)
    dO = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    dST = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    gr = orc.backward(q, k, v, z, beta, A, -5.0, S0, dO, dST)
    g = -5.0 * expit(np.exp(A.astype(np.float64))[None, None, :, None] * z.astype(np.float64))
    Gam = np.exp(np.cumsum(g, axis=1))                                   # [B,T,H,dk]
    S0d = S0.astype(np.float64)
    dq_ref = Gam * np.einsum("bhcj,bthj->bthc", S0d, dO.astype(np.float64))
    dS0_ref = (np.einsum("bthc,bthj->bhcj", Gam * q, dO.astype(np.float64))
               + Gam[:, -1][..., None] * dST)
    np.testing.assert_allclose(gr["dq"], dq_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gr["dS0"], dS0_ref, rtol=1e-12, atol=1e-13)
    assert np.all(gr["dk"] == 0.0) and np.all(gr["dv"] == 0.0)


def pin_backward_chunkwise_equivalence(orc):
    """The token-by-token gradients equal those of the independent chunkwise
    backward (oracle/chunkwise.py, the chunk equations differentiated step by
    step) for chunk sizes 1, 5, 16 and T, including dz through the gate."""
    rng = np.random.default_rng(33)
    B, T, H, dk, dv = 2, 21, 2, 5, 4
    q, k, v, z, beta, A, S0 = _inputs(rng, B, T, H, dk, dv)
    dO = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    dST = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    g_min = -5.0
    ref = orc.backward(q, k, v, z, beta, A, g_min, S0, dO, dST)
    for b in range(B):
        for h in range(H):
            g = gate_fp64(z[b, :, h], float(A[h]), g_min)
            x = np.exp(np.float64(A[h])) * z[b, :, h].astype(np.float64)
            s = expit(x)
            for C in (1, 5, 16, T):
                c = chunk_head_backward(q[b, :, h], k[b, :, h], v[b, :, h], g, beta[b, :, h],
                                        S0[b, h], dO[b, :, h], dST[b, h], C)
                np.testing.assert_allclose(c["dq"], ref["dq"][b, :, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(c["dk"], ref["dk"][b, :, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(c["dv"], ref["dv"][b, :, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(c["dbeta"], ref["dbeta"][b, :, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(c["dS0"], ref["dS0"][b, h], rtol=0, atol=1e-12)
                dz = c["dg"] * g_min * s * (1.0 - s) * np.exp(np.float64(A[h]))
                np.testing.assert_allclose(dz, ref["dz"][b, :, h], rtol=0, atol=1e-12)


PINS = [pin_gate_at_zero, pin_gate_library, pin_gate_bounds_printed, pin_chunk_cumsum,
        pin_scalar_ema, pin_beta_zero, pin_exact_retrieval, pin_linear_attention,
        pin_alpha_one_beta_zero, pin_chunkwise_equivalence, pin_continuation,
        pin_linearity, pin_structure, pin_decode_matches_prefill,
        pin_backward_finite_difference, pin_backward_beta_zero,
        pin_backward_chunkwise_equivalence]


def failing_pins(orc):
    """Names of the pins the given oracle build fails (crashes count)."""
    bad = []
    for pin in PINS:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001 -- any failure trips the pin
            bad.append(pin.__name__)
    return bad
