"""GPU tests of the ring plan (pair producers and state chains in one launch,
pair blocks handed over through an XCD's L2): the fp64 oracle on unit counts
that leave XCD groups partly empty, equality with the split plan (the same
pair arithmetic) over thousands of ring-slot reuses, and slot-addressed
states with a skipped sequence."""
from __future__ import annotations

import pytest
import torch

import linear_attention_recurrence_05_amd as kda
from linear_attention_recurrence_05_amd.inputs import prefill_inputs
import oracle

from gpu_common import TOL, need_gpu, plan, rel_err, say

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def run(x, s0="keep"):
    s0 = x["S0"] if isinstance(s0, str) else s0
    o, ST = kda.chunk_prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"], s0)
    torch.cuda.synchronize()
    return o, ST


@pytest.mark.parametrize("B,T,H", [(3, 300, 3), (1, 1, 1), (2, 47, 16), (4, 129, 5)])
def test_ring_against_oracle(B, T, H):
    """B * H in {9, 1, 32, 20}: one to four units per XCD group, groups with
    empty places; T with an empty second chunk in the last pair (47, 129) and
    a single token (1)."""
    dev = need_gpu()
    x = prefill_inputs(B, T, H, 128, 128, BF, seed=B * 100 + T + H, s0_std=0.1, device=dev)
    with plan("ring"):
        o, ST = run(x)
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"], x["S0"])
    eo, es = rel_err(o, o_ref), rel_err(ST, S_ref)
    say(f"ring B{B} T{T} H{H}: o {eo:.2e} S_T {es:.2e}")
    assert eo < TOL[BF] and es < TOL[BF]


def test_ring_equals_split_over_many_slot_reuses():
    """B1 H32, 65,000 tokens (2,032 pairs: every ring slot reused ~200 times),
    with S0: the ring plan and the split plan run the same pair arithmetic;
    a stale or torn pair block would show as a large difference."""
    dev = need_gpu()
    x = prefill_inputs(1, 65000, 32, 128, 128, BF, seed=31, s0_std=0.1, device=dev)
    with plan("ring"):
        o_r, S_r = run(x)
    with plan("split"):
        o_s, S_s = run(x)
    d_o = float((o_r.float() - o_s.float()).abs().max()) / float(o_s.float().abs().max())
    d_s = float((S_r - S_s).abs().max()) / float(S_s.abs().max())
    say(f"ring vs split, B1 H32 T65000: o {d_o:.2e} S_T {d_s:.2e} "
        f"(bit-identical: {bool(torch.equal(o_r, o_s) and torch.equal(S_r, S_s))})")
    assert torch.isfinite(o_r.float()).all() and torch.isfinite(S_r).all()
    assert d_o < 1e-6 and d_s < 1e-6


def test_ring_workspace():
    """The ring plan's workspace is 256 bytes of flags and 10 pair blocks
    (ring slots) per unit.  A pair block at bf16, d = 128 is 28,160 bytes: four 16 x 128 bf16
    operands (16,384), the 32 x 128 state-update operand (8,192), four
    16 x 16 and one 16 x 32 small operand (3,072) and gam_a gam_b in fp32
    (512)."""
    need_gpu()
    for (B, H) in [(1, 32), (2, 3)]:
        with plan("ring"):
            nbytes = kda.kda_chunk_prefill_workspace_bytes(B, 4096, H, 128, 128, BF)
        units = B * H
        say(f"ring workspace B{B} H{H} T4096: {nbytes} bytes")
        assert nbytes == units * 256 + units * 10 * 28160


def test_ring_paged_with_skipped_sequence():
    """States from pool rows into other pool rows; sequence 1's slot is out of
    range (skipped: its outputs and every pool row stay); the others match
    the oracle, and rows no table names are untouched."""
    dev = need_gpu()
    B, T, H, d, n_slots = 4, 90, 5, 128, 11
    g = torch.Generator(device="cpu").manual_seed(33)
    pool = (torch.randn(n_slots, H, d, d, generator=g) * 0.1).to(dev)
    perm = torch.randperm(n_slots, generator=g)
    s_in = perm[:B].to(torch.int32).to(dev)
    s_out = perm[B:2 * B].to(torch.int32).to(dev)
    s_in[1] = n_slots
    pool0 = pool.clone()
    x = prefill_inputs(B, T, H, d, d, BF, seed=34, device=dev)
    o = torch.full_like(x["v"], 3.0)
    with plan("ring"):
        nbytes = kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, BF)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        kda.kda_chunk_prefill_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                    pool, s_in, s_out, o, ws)
        torch.cuda.synchronize()
    live = [0, 2, 3]
    S0 = pool0[s_in[live].long()]
    sub = {kk: x[kk][live].contiguous() for kk in ("q", "k", "v", "z", "beta")}
    o_ref, S_ref = oracle.prefill(sub["q"], sub["k"], sub["v"], sub["z"], sub["beta"], x["A"], x["g_min"], S0)
    eo, es = rel_err(o[live], o_ref), rel_err(pool[s_out[live].long()], S_ref)
    say(f"ring paged, sequence 1 skipped: o {eo:.2e} S_T {es:.2e}")
    assert eo < TOL[BF] and es < TOL[BF]
    assert torch.all(o[1] == 3.0)
    named = set(int(t) for t in s_out[live].cpu().tolist())
    rest = [r for r in range(n_slots) if r not in named]
    assert torch.equal(pool[rest], pool0[rest])
