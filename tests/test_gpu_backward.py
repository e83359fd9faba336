"""GPU parity of kda_chunk_backward (gradients of the prefill) against the
fp64 oracle's reverse sweep, on the same seeded inputs: every gradient tensor
compared element by element, normwise, at the bf16 / fp32 tolerances."""
from __future__ import annotations

import pytest
import torch

import linear_attention_recurrence_05_amd as kda
from linear_attention_recurrence_05_amd.inputs import backward_grads, config_inputs, prefill_inputs
import oracle

from gpu_common import TOL, need_gpu, rel_err, say

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
NAMES = ("dq", "dk", "dv", "dz", "dbeta", "dA", "dS0")


def run(x, gr):
    g = kda.chunk_backward(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], gr["dO"],
                           g_min=x["g_min"], S0=x["S0"], dS_T=gr["dST"])
    torch.cuda.synchronize()
    return g


def compare(x, gr, g, tol, what, nthreads=0):
    ref = oracle.backward(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                          x["S0"], gr["dO"], gr["dST"], nthreads=nthreads)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    say(what + ": " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e < tol, (n, e)


@pytest.mark.parametrize("d,dt", [(32, "f32"), (128, "f32"), (32, "bf16"), (128, "bf16")])
@pytest.mark.parametrize("T", [1, 15, 17, 64, 100])
def test_backward_small(d, dt, T):
    dev = need_gpu()
    with_s0 = T % 2 == 1
    x = prefill_inputs(2, T, 3, d, d, DT[dt], seed=500 + T + d, s0_std=0.1 if with_s0 else None,
                       device=dev)
    gr = backward_grads(2, T, 3, d, d, DT[dt], seed=500 + T + d, with_dST=not with_s0, device=dev)
    g = run(x, gr)
    compare(x, gr, g, TOL[DT[dt]], f"backward d={d} {dt} T={T} S0={with_s0}")


def test_backward_many_segments():
    """B2 H96, d = 128: the partial sums of one launch cover 128 tokens, so
    T = 200 runs as two reverse-sweep launches carrying the state gradient."""
    dev = need_gpu()
    x = prefill_inputs(2, 200, 96, 128, 128, torch.bfloat16, seed=77, s0_std=0.1, device=dev)
    gr = backward_grads(2, 200, 96, 128, 128, torch.bfloat16, seed=77, device=dev)
    g = run(x, gr)
    compare(x, gr, g, TOL[torch.bfloat16], "backward B2 H96 T200 (2 launches)", nthreads=16)


def test_backward_workload_0():
    """The tiny fp32 workload (B1 H2 T64 d32), every gradient at 1e-4."""
    dev = need_gpu()
    x = config_inputs(0, device=dev)
    B, T, H, d = x["q"].shape
    gr = backward_grads(B, T, H, d, d, torch.float32, seed=0, device=dev)
    g = run(x, gr)
    compare(x, gr, g, 1e-4, "backward workload 0")


def test_backward_workload_1():
    """The mid workload (B1 H32 T4096 d128 bf16), every gradient in full."""
    dev = need_gpu()
    x = config_inputs(1, device=dev)
    B, T, H, d = x["q"].shape
    gr = backward_grads(B, T, H, d, d, torch.bfloat16, seed=1, device=dev)
    g = run(x, gr)
    compare(x, gr, g, TOL[torch.bfloat16], "backward workload 1", nthreads=16)


def test_backward_deterministic_and_optional_args():
    dev = need_gpu()
    x = prefill_inputs(2, 70, 4, 128, 128, torch.bfloat16, seed=9, s0_std=0.1, device=dev)
    gr = backward_grads(2, 70, 4, 128, 128, torch.bfloat16, seed=9, device=dev)
    g1, g2 = run(x, gr), run(x, gr)
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n
    # dS0 not requested: the other gradients are unchanged
    g3 = kda.chunk_backward(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], gr["dO"],
                            g_min=x["g_min"], S0=x["S0"], dS_T=gr["dST"], want_dS0=False)
    torch.cuda.synchronize()
    for n in NAMES[:-1]:
        assert torch.equal(g1[n], g3[n]), n


def test_backward_decay_free_gate():
    """g_min = 0 (retention 1, a pure delta rule): dz and dA vanish exactly,
    the rest matches the oracle."""
    dev = need_gpu()
    x = prefill_inputs(1, 40, 2, 32, 32, torch.float32, seed=13, s0_std=0.1, device=dev)
    x["g_min"] = 0.0
    gr = backward_grads(1, 40, 2, 32, 32, torch.float32, seed=13, device=dev)
    g = run(x, gr)
    assert torch.count_nonzero(g["dz"]) == 0 and torch.count_nonzero(g["dA"]) == 0
    ref = oracle.backward(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], 0.0, x["S0"],
                          gr["dO"], gr["dST"])
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert rel_err(g[n], ref[n]) < 1e-4, n


@pytest.mark.parametrize("B,d,dt,T,s0", [(1, 32, "f32", 768, True), (1, 128, "f32", 1024, True),
                                          (1, 128, "bf16", 2048, True), (2, 128, "bf16", 1024, False),
                                          (2, 32, "f32", 2080, False)])
def test_backward_segmented_forward_sweep(B, d, dt, T, s0):
    """T splits into whole-chunk segments of >= 256 tokens (2, 4 and 8 of
    them here; 2 x 65 chunks for T = 2080): the forward sweep runs the
    segments side by side from start states given by a segment scan of the
    chunkwise forward."""
    dev = need_gpu()
    x = prefill_inputs(B, T, 4, d, d, DT[dt], seed=700 + T, s0_std=0.1 if s0 else None, device=dev)
    gr = backward_grads(B, T, 4, d, d, DT[dt], seed=700 + T, device=dev)
    g = run(x, gr)
    compare(x, gr, g, TOL[DT[dt]], f"backward B={B} d={d} {dt} T={T} S0={s0} (segmented forward sweep)",
            nthreads=16)


@pytest.mark.parametrize("bplan", ["sweep", "chain"])
@pytest.mark.parametrize("d,dt,T", [(32, "f32", 100), (128, "f32", 300), (128, "bf16", 520)])
def test_backward_plans(bplan, d, dt, T):
    """Both reverse-sweep plans against the oracle: one token-level sweep per
    (b, h, column block) over the sequence, and the chunk-level chain of end-
    state gradients followed by every chunk's sweep at once."""
    dev = need_gpu()
    x = prefill_inputs(2, T, 3, d, d, DT[dt], seed=800 + T, s0_std=0.1, device=dev)
    gr = backward_grads(2, T, 3, d, d, DT[dt], seed=800 + T, device=dev)
    import os
    old = os.environ.get("KDA_BACKWARD_PLAN")
    os.environ["KDA_BACKWARD_PLAN"] = bplan
    try:
        g = run(x, gr)
    finally:
        if old is None:
            os.environ.pop("KDA_BACKWARD_PLAN", None)
        else:
            os.environ["KDA_BACKWARD_PLAN"] = old
    compare(x, gr, g, TOL[DT[dt]], f"backward plan {bplan} d={d} {dt} T={T}")
