"""GPU tests of the paged entry points: with the states in a pool addressed by
an int32 slot table, every result equals the dense call on the gathered
states bit for bit (the same kernels run on the same values), rows of the
pool no sequence names are untouched, and a sequence whose slot is out of
range is skipped (its outputs and every pool row stay as they were)."""
from __future__ import annotations

import pytest
import torch

import linear_attention_recurrence_05_amd as kda
from linear_attention_recurrence_05_amd.inputs import decode_state, decode_step_inputs, prefill_inputs
import oracle

from gpu_common import TOL, need_gpu, plan, rel_err, say

pytestmark = pytest.mark.gpu


def pool_and_slots(B, H, d, n_slots, dev, seed=7):
    g = torch.Generator(device="cpu").manual_seed(seed)
    pool = (torch.randn(n_slots, H, d, d, generator=g) * 0.1).to(dev)
    perm = torch.randperm(n_slots, generator=g)
    slots_in = perm[:B].to(torch.int32).to(dev)
    slots_out = perm[B:2 * B].to(torch.int32).to(dev) if 2 * B <= n_slots else slots_in.clone()
    return pool, slots_in, slots_out


def untouched_rows(n_slots, *tables):
    used = set()
    for t in tables:
        used |= set(int(x) for x in t.cpu().tolist())
    return [r for r in range(n_slots) if r not in used]


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (32, torch.float32)])
def test_decode_paged_equals_dense(d, dt):
    dev = need_gpu()
    B, H, n_slots = 5, 3, 9
    pool, slots, _ = pool_and_slots(B, H, d, n_slots, dev)
    pool0 = pool.clone()
    gen, A, _ = decode_state(B, H, d, d, seed=11, device=dev)
    x = decode_step_inputs(gen, B, H, d, d, dt, dev)
    S = pool[slots.long()].clone()
    o_dense = kda.decode_step(x["q"], x["k"], x["v"], x["z"], x["beta"], A, S)
    o = torch.empty_like(o_dense)
    kda.kda_decode_step_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], A, -5.0, pool, slots, o)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dense)
    assert torch.equal(pool[slots.long()], S)
    rest = untouched_rows(n_slots, slots)
    assert torch.equal(pool[rest], pool0[rest])


def test_tokens_paged_snapshot_equals_dense():
    dev = need_gpu()
    B, T, H, d, n_slots = 4, 6, 3, 128, 10
    pool, s_in, s_out = pool_and_slots(B, H, d, n_slots, dev, seed=8)
    pool0 = pool.clone()
    x = prefill_inputs(B, T, H, d, d, torch.bfloat16, seed=12, device=dev)
    o_dense, S_dense = kda.decode_tokens(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"],
                                         pool[s_in.long()].clone())
    o = torch.empty_like(o_dense)
    kda.kda_decode_tokens_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], -5.0, pool,
                                s_in, s_out, o)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dense)
    assert torch.equal(pool[s_out.long()], S_dense)
    assert torch.equal(pool[s_in.long()], pool0[s_in.long()])   # the snapshot rows stay
    rest = untouched_rows(n_slots, s_in, s_out)
    assert torch.equal(pool[rest], pool0[rest])


@pytest.mark.parametrize("p", ["split", "fused:32"])
@pytest.mark.parametrize("tables", ["in_out", "out_only", "in_only", "same"])
def test_prefill_paged_equals_dense(p, tables):
    dev = need_gpu()
    B, T, H, d, n_slots = 3, 100, 2, 32, 8
    pool, s_in, s_out = pool_and_slots(B, H, d, n_slots, dev, seed=9)
    if tables == "same":
        s_out = s_in
    t_in = None if tables == "out_only" else s_in
    t_out = None if tables == "in_only" else s_out
    pool0 = pool.clone()
    x = prefill_inputs(B, T, H, d, d, torch.float32, seed=13, device=dev)
    with plan(p):
        S0 = pool[t_in.long()].clone() if t_in is not None else None
        o_dense, S_dense = kda.chunk_prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"],
                                             x["g_min"], S0)
        o = torch.empty_like(o_dense)
        nbytes = kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, torch.float32)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        kda.kda_chunk_prefill_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                    pool, t_in, t_out, o, ws)
        torch.cuda.synchronize()
    assert torch.equal(o, o_dense)
    if t_out is not None:
        assert torch.equal(pool[t_out.long()], S_dense)
    used = [t for t in (t_in, t_out) if t is not None]
    rest = untouched_rows(n_slots, *used)
    assert torch.equal(pool[rest], pool0[rest])


def test_prefill_paged_segments_against_oracle():
    """Longer than one split-plan segment (1,024 chunks): the state crosses
    segments through the output slots; checked against the fp64 oracle."""
    dev = need_gpu()
    B, T, H, d, n_slots = 1, 16 * 1024 + 40, 2, 32, 3
    pool, s_in, _ = pool_and_slots(B, H, d, n_slots, dev, seed=10)
    s_out = torch.tensor([2 if int(s_in[0]) != 2 else 0], dtype=torch.int32, device=dev)
    x = prefill_inputs(B, T, H, d, d, torch.float32, seed=14, device=dev)
    S0 = pool[s_in.long()].clone()
    o = torch.empty_like(x["v"])
    with plan("split"):
        nbytes = kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, torch.float32)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        kda.kda_chunk_prefill_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                    pool, s_in, s_out, o, ws)
        torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"], S0)
    eo, es = rel_err(o, o_ref), rel_err(pool[s_out.long()], S_ref)
    say(f"paged prefill over 2 segments: o {eo:.2e} S {es:.2e}")
    assert eo < TOL[torch.float32] and es < TOL[torch.float32]
    assert torch.equal(pool[s_in.long()], S0)


@pytest.mark.parametrize("p", ["split", "fused:32"])
def test_out_of_range_slot_is_skipped(p):
    dev = need_gpu()
    B, T, H, d, n_slots = 3, 40, 2, 32, 4
    pool, s_in, _ = pool_and_slots(B, H, d, n_slots, dev, seed=15)
    s_bad = s_in.clone()
    s_bad[1] = n_slots          # out of range
    pool0 = pool.clone()
    x = prefill_inputs(B, T, H, d, d, torch.float32, seed=16, device=dev)
    o = torch.full_like(x["v"], 7.0)
    with plan(p):
        nbytes = kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, torch.float32)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        kda.kda_chunk_prefill_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                    pool, s_bad, s_bad, o, ws)
        torch.cuda.synchronize()
    assert torch.all(o[1] == 7.0)                      # the skipped sequence's outputs
    assert torch.equal(pool[s_in[1:2].long()], pool0[s_in[1:2].long()]) or int(s_in[1]) >= n_slots
    assert not torch.all(o[0] == 7.0) and not torch.all(o[2] == 7.0)
    # decode with a negative slot: that sequence's row and output stay
    gen, A, _ = decode_state(B, H, d, d, seed=17, device=dev)
    xd = decode_step_inputs(gen, B, H, d, d, torch.float32, dev)
    s_neg = s_in.clone()
    s_neg[0] = -1
    pool1 = pool.clone()
    od = torch.full((B, H, d), 7.0, device=dev)
    kda.kda_decode_step_paged(xd["q"], xd["k"], xd["v"], xd["z"], xd["beta"], A, -5.0, pool, s_neg, od)
    torch.cuda.synchronize()
    assert torch.all(od[0] == 7.0) and not torch.all(od[1] == 7.0)
    assert torch.equal(pool[int(s_in[0])], pool1[int(s_in[0])])


def test_decode_paged_d128_pairs_with_skipped_units():
    """At d = 128 one workgroup takes two consecutive (b, h) units. With an
    odd head count the pairs straddle sequences, so a live unit shares its
    workgroup with a skipped one (negative or out-of-range slot) and the last
    workgroup holds a single unit; the live units still match the oracle and
    the skipped ones leave their outputs and pool rows as they were."""
    dev = need_gpu()
    B, H, d, n_slots = 5, 3, 128, 9
    pool, slots, _ = pool_and_slots(B, H, d, n_slots, dev, seed=31)
    gen, A, _ = decode_state(B, H, d, d, seed=32, device=dev)
    x = decode_step_inputs(gen, B, H, d, d, torch.bfloat16, dev)
    s = slots.clone()
    s[1] = -1
    s[3] = n_slots
    live = [0, 2, 4]
    pool0 = pool.clone()
    S_ref = pool[slots[live].long()].double().cpu().numpy().copy()
    o = torch.full((B, H, d), 7.0, dtype=torch.bfloat16, device=dev)
    kda.kda_decode_step_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], A, -5.0, pool, s, o)
    torch.cuda.synchronize()
    sub = {kk: x[kk][live] for kk in ("q", "k", "v", "z", "beta")}
    o_ref = oracle.decode(sub["q"], sub["k"], sub["v"], sub["z"], sub["beta"], A, -5.0, S_ref)
    eo, es = rel_err(o[live], o_ref), rel_err(pool[slots[live].long()], S_ref)
    say(f"paged decode, d=128, skipped units in shared workgroups: o {eo:.2e} S {es:.2e}")
    assert eo < TOL[torch.bfloat16] and es < 1e-4
    assert torch.all(o[1] == 7.0) and torch.all(o[3] == 7.0)
    untouched = untouched_rows(n_slots, slots[live])
    assert torch.equal(pool[untouched], pool0[untouched])


def test_verify_paged_d128_pairs_with_skipped_units():
    """The verify step at d = 128 also takes two (b, h) units per workgroup,
    each on its own waves.  With an odd head count a live unit shares its
    workgroup with a skipped one (a negative input slot, an out-of-range
    output slot), and the last workgroup holds a single unit; T = 6 spans two
    groups of staged tokens.  Live units match the oracle, skipped outputs
    and every row no live unit writes stay as they were."""
    dev = need_gpu()
    B, H, d, n_slots, T = 5, 3, 128, 11, 6
    pool, s_in, s_out = pool_and_slots(B, H, d, n_slots, dev, seed=41)
    s_in = s_in.clone()
    s_out = s_out.clone()
    s_in[1] = -1
    s_out[3] = n_slots
    live = [0, 2, 4]
    gen, A, _ = decode_state(B, H, d, d, seed=42, device=dev)
    x = prefill_inputs(B, T, H, d, d, torch.bfloat16, seed=43, device=dev)
    pool0 = pool.clone()
    S_in = pool[s_in[live].long()].clone()
    o = torch.full((B, T, H, d), 7.0, dtype=torch.bfloat16, device=dev)
    kda.kda_decode_tokens_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], A, -5.0, pool, s_in,
                                s_out, o)
    torch.cuda.synchronize()
    sub = {kk: x[kk][live].contiguous() for kk in ("q", "k", "v", "z", "beta")}
    o_ref, S_ref = oracle.prefill(sub["q"], sub["k"], sub["v"], sub["z"], sub["beta"], A, -5.0, S_in)
    eo, es = rel_err(o[live], o_ref), rel_err(pool[s_out[live].long()], S_ref)
    say(f"paged verify, d=128 T={T}, skipped units in shared workgroups: o {eo:.2e} S {es:.2e}")
    assert eo < TOL[torch.bfloat16] and es < 1e-4
    assert torch.all(o[1] == 7.0) and torch.all(o[3] == 7.0)
    kept = untouched_rows(n_slots, s_out[live])
    assert torch.equal(pool[kept], pool0[kept])


def test_decode_and_verify_paged_against_oracle():
    """Paged decode (two steps in place) and the paged 5-token verify step
    (snapshot kept) against the fp64 oracle directly, bf16 at d = 128."""
    dev = need_gpu()
    B, H, d, n_slots, T = 6, 4, 128, 13, 5
    pool, slots, s_out = pool_and_slots(B, H, d, n_slots, dev, seed=21)
    gen, A, _ = decode_state(B, H, d, d, seed=22, device=dev)
    S_ref = pool[slots.long()].double().cpu().numpy().copy()
    for step in range(2):
        x = decode_step_inputs(gen, B, H, d, d, torch.bfloat16, dev)
        o = torch.empty(B, H, d, dtype=torch.bfloat16, device=dev)
        kda.kda_decode_step_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], A, -5.0, pool, slots, o)
        torch.cuda.synchronize()
        o_ref = oracle.decode(x["q"], x["k"], x["v"], x["z"], x["beta"], A, -5.0, S_ref)
        eo, es = rel_err(o, o_ref), rel_err(pool[slots.long()], S_ref)
        say(f"paged decode step {step + 1}: o {eo:.2e} S {es:.2e}")
        assert eo < TOL[torch.bfloat16] and es < 1e-4
    xv = prefill_inputs(B, T, H, d, d, torch.bfloat16, seed=23, device=dev)
    S_in = pool[slots.long()].clone()
    ov = torch.empty(B, T, H, d, dtype=torch.bfloat16, device=dev)
    kda.kda_decode_tokens_paged(xv["q"], xv["k"], xv["v"], xv["z"], xv["beta"], A, -5.0, pool,
                                slots, s_out, ov)
    torch.cuda.synchronize()
    o_ref, S_T_ref = oracle.prefill(xv["q"], xv["k"], xv["v"], xv["z"], xv["beta"], A, -5.0, S_in)
    eo, es = rel_err(ov, o_ref), rel_err(pool[s_out.long()], S_T_ref)
    say(f"paged verify T={T}: o {eo:.2e} S {es:.2e}")
    assert eo < TOL[torch.bfloat16] and es < 1e-4
    assert torch.equal(pool[slots.long()], S_in)   # the snapshot rows stay


@pytest.mark.parametrize("p", ["auto", "fused:128", "fused:64"])
def test_prefill_paged_bf16_d128_against_oracle(p):
    """Paged prefill, bf16 at d = 128, from pool rows into other pool rows,
    against the oracle; 'auto' picks the fused plan at B * H = 128."""
    dev = need_gpu()
    B, T, H, d, n_slots = 32, 77, 4, 128, 70
    pool, s_in, s_out = pool_and_slots(B, H, d, n_slots, dev, seed=24)
    x = prefill_inputs(B, T, H, d, d, torch.bfloat16, seed=25, device=dev)
    S0 = pool[s_in.long()].clone()
    o = torch.empty_like(x["v"])
    with plan(p):
        nbytes = kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, torch.bfloat16)
        assert p != "auto" or nbytes == 0   # the fused plan needs no workspace
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        kda.kda_chunk_prefill_paged(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                    pool, s_in, s_out, o, ws)
        torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                  S0, nthreads=16)
    eo, es = rel_err(o, o_ref), rel_err(pool[s_out.long()], S_ref)
    say(f"paged prefill bf16 d128 plan {p}: o {eo:.2e} S {es:.2e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16]
    assert torch.equal(pool[s_in.long()], S0)
