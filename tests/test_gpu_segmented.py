"""GPU parity of kda_chunk_prefill_segmented (the prefill as a scan over
segments of the sequence) against the fp64 oracle's token-by-token prefill,
and against the direct chunkwise prefill on the GPU."""
from __future__ import annotations

import pytest
import torch

import linear_attention_recurrence_05_amd as kda
from linear_attention_recurrence_05_amd.inputs import config_inputs, prefill_inputs
import oracle

from gpu_common import TOL, need_gpu, plan, rel_err, say

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def seg(x, n_seg, S0="given"):
    s0 = x["S0"] if S0 == "given" else S0
    o, ST = kda.chunk_prefill_segmented(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], n_seg,
                                        g_min=x["g_min"], S0=s0)
    torch.cuda.synchronize()
    return o, ST


@pytest.mark.parametrize("d,dt", [(32, "f32"), (128, "f32"), (32, "bf16"), (128, "bf16")])
@pytest.mark.parametrize("T,n_seg", [(96, 1), (96, 2), (96, 3), (96, 6), (100, 4), (48, 48)])
def test_segmented_vs_oracle(d, dt, T, n_seg):
    dev = need_gpu()
    x = prefill_inputs(2, T, 3, d, d, DT[dt], seed=900 + T + n_seg + d, s0_std=0.1, device=dev)
    o, ST = seg(x, n_seg)
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                  x["S0"])
    eo, es = rel_err(o, o_ref), rel_err(ST, S_ref)
    say(f"segmented d={d} {dt} T={T} n_seg={n_seg}: o {eo:.2e} S_T {es:.2e}")
    assert eo < TOL[DT[dt]] and es < TOL[DT[dt]]


def test_segmented_slow_decay():
    """g_min = -0.05: the state remembers across many chunks, so every
    segment's start state (the scan) matters for its outputs."""
    dev = need_gpu()
    x = prefill_inputs(1, 512, 4, 128, 128, torch.float32, seed=31, s0_std=0.1, device=dev)
    x["g_min"] = -0.05
    o, ST = seg(x, 8)
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], -0.05,
                                  x["S0"])
    eo, es = rel_err(o, o_ref), rel_err(ST, S_ref)
    say(f"segmented slow decay: o {eo:.2e} S_T {es:.2e}")
    assert eo < 1e-4 and es < 1e-4


def test_segmented_state_alias_and_no_state():
    dev = need_gpu()
    x = prefill_inputs(2, 64, 3, 128, 128, torch.bfloat16, seed=5, s0_std=0.1, device=dev)
    o1, S1 = seg(x, 4)
    S = x["S0"].clone()
    nb = kda.kda_chunk_prefill_segmented_workspace_bytes(2, 64, 3, 128, 128, 4, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    o2 = torch.empty_like(o1)
    kda.kda_chunk_prefill_segmented(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                    S, o2, S, 4, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S)
    o3, S3 = kda.chunk_prefill_segmented(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], 4,
                                         g_min=x["g_min"], S0=x["S0"], want_state=False)
    torch.cuda.synchronize()
    assert S3 is None and torch.equal(o1, o3)


def test_segmented_mid_workload():
    """The mid workload (B1 H32 T4096 bf16) in 8 segments, in full against the
    oracle and against the direct prefill."""
    dev = need_gpu()
    x = config_inputs(1, device=dev)
    o, ST = seg(x, 8)
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                  x["S0"], nthreads=16)
    od, Sd = kda.chunk_prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                               x["S0"])
    torch.cuda.synchronize()
    eo, es = rel_err(o, o_ref), rel_err(ST, S_ref)
    say(f"segmented mid workload n_seg=8: o {eo:.2e} S_T {es:.2e}; "
        f"vs direct o {rel_err(o, od.float().cpu().numpy()):.2e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16]


def _np(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("H,R", [(32, 8), (24, 8), (16, 16)])
def test_prefill_chooses_segment_scan_for_long_sequences_of_few_heads(H, R):
    """kda_chunk_prefill runs the segment scan by itself for T = 65,536 with
    few heads (fused state-only passes with 128 columns per workgroup at
    B * R * H = 256, 64 at 192): bit-identical to the explicit segmented call,
    within tolerance of the direct plan and of the oracle."""
    dev = need_gpu()
    T = 65536
    assert kda.kda_chunk_prefill_segments(1, T, H, 128, 128, torch.bfloat16) == R
    x = prefill_inputs(1, T, H, 128, 128, torch.bfloat16, seed=77 + H, s0_std=0.1, device=dev)
    args = (x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"])
    o, ST = kda.chunk_prefill(*args, g_min=x["g_min"], S0=x["S0"])
    o_s, S_s = seg(x, R)
    assert torch.equal(o, o_s) and torch.equal(ST, S_s)
    with plan("split"):
        o_d, S_d = kda.chunk_prefill(*args, g_min=x["g_min"], S0=x["S0"])
    torch.cuda.synchronize()
    ed_o, ed_s = rel_err(o, _np(o_d)), rel_err(ST, _np(S_d))
    # the oracle from token 0 over the first two segments and 512 tokens of
    # the third: outputs inside segment 0 and after the first two segment
    # boundaries (which depend on the scanned start states)
    Tseg = T // R
    P = 2 * Tseg + 512
    o_ref, _ = oracle.prefill(*(t[:, :P] for t in (x["q"], x["k"], x["v"], x["z"], x["beta"])),
                              x["A"], x["g_min"], x["S0"], want_state=False, nthreads=16)
    eo = rel_err(o[:, :P], o_ref)
    eb = [rel_err(o[:, r * Tseg:r * Tseg + 512], o_ref[:, r * Tseg:r * Tseg + 512]) for r in (1, 2)]
    say(f"auto segments H={H} R={R}: vs direct o {ed_o:.2e} S_T {ed_s:.2e}; "
        f"vs oracle on tokens 0..{P - 1} {eo:.2e} (after boundaries 1, 2: {eb[0]:.2e}, "
        f"{eb[1]:.2e})")
    assert ed_o < TOL[torch.bfloat16] and ed_s < TOL[torch.bfloat16]
    assert eo < TOL[torch.bfloat16] and max(eb) < TOL[torch.bfloat16]
    if H == 32:
        # in place (S_T aliases S0) and without S_T, through the plain entry point
        S = x["S0"].clone()
        o2 = torch.empty_like(o)
        ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(1, T, H, 128, 128, torch.bfloat16),
                         dtype=torch.uint8, device=dev)
        kda.kda_chunk_prefill(*args, x["g_min"], S, o2, S, ws)
        o3 = torch.empty_like(o)
        kda.kda_chunk_prefill(*args, x["g_min"], x["S0"], o3, None, ws)
        torch.cuda.synchronize()
        assert torch.equal(S, ST) and torch.equal(o2, o) and torch.equal(o3, o)


@pytest.mark.parametrize("dt,H,decay", [("bf16", 32, "fast"), ("bf16", 32, "slow"),
                                        ("bf16", 32, "mixed"), ("bf16", 24, "mixed"),
                                        ("f32", 32, "fast"), ("f32", 32, "mixed")])
def test_segmented_fused_map_early_exit(dt, H, decay):
    """Segments of the fused plan (B * R * H >= 128 units at d = 128): the M_r
    pass stops once a segment's map is exactly zero, the outputs come from a
    zero-start pass and the first chunks of every segment are redone from its
    scanned start state.  Fast decay (g_min = -5: every map vanishes within a
    few chunks), slow decay (g_min = -0.05: no map vanishes, the redo covers
    whole segments) and a mix (half the heads with z shifted by -12, so that
    their gate stays near 0 and their maps do not vanish), with S0 given;
    against the oracle and bit for bit from run to run."""
    dev = need_gpu()
    T, R = (2048, 8) if dt == "bf16" else (1024, 8)
    x = prefill_inputs(1, T, H, 128, 128, DT[dt], seed=1300 + H + len(decay), s0_std=0.1,
                       device=dev)
    if decay == "slow":
        x["g_min"] = -0.05
    elif decay == "mixed":
        zf = x["z"].float()
        zf[:, :, ::2] -= 12.0
        x["z"] = zf.to(x["z"].dtype)
    o, ST = seg(x, R)
    o2, ST2 = seg(x, R)
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                  x["S0"], nthreads=16)
    eo, es = rel_err(o, o_ref), rel_err(ST, S_ref)
    Tseg = T // R
    eb = max(rel_err(o[:, r * Tseg:r * Tseg + 64], o_ref[:, r * Tseg:r * Tseg + 64])
             for r in range(1, R))
    say(f"segmented fused {dt} H={H} {decay} decay: o {eo:.2e} S_T {es:.2e}; "
        f"first 64 tokens after each boundary {eb:.2e}")
    assert eo < TOL[DT[dt]] and es < TOL[DT[dt]] and eb < TOL[DT[dt]]
