"""kda_chunk_prefill_noalloc (the prefill without a workspace argument: its
scratch is a static per-GPU array) against kda_chunk_prefill with a caller
workspace, through the C ABI: equal results on consecutive calls of shrinking
size and of each plan that uses scratch (the segment scan, the ring plan, the
split plan), and sizes beyond the scratch rejected before any launch."""
from __future__ import annotations

import pytest
import torch

import linear_attention_recurrence_05_amd as kda
from linear_attention_recurrence_05_amd.inputs import prefill_inputs

from gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


def _both(x):
    o_ref, S_ref = kda.chunk_prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"],
                                     x["g_min"], x["S0"])
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    kda.kda_chunk_prefill_noalloc(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["g_min"],
                                  x["S0"], o, S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    dev = need_gpu()
    # (B, T, H, d, dtype, S0 std): the segment scan (67 MB of scratch), the
    # ring plan (14 MB; the split plan's 115 MB where no ring fits the
    # device), a smaller split-plan call (fp32), a fused-plan call (none)
    cases = [(1, 65536, 32, 128, torch.bfloat16, 0.1), (1, 4096, 32, 128, torch.bfloat16, None),
             (2, 100, 3, 32, torch.float32, 0.1), (8, 40, 32, 128, torch.bfloat16, 0.1)]
    sizes = []
    for i, (B, T, H, d, dt, s0) in enumerate(cases):
        need = kda.kda_chunk_prefill_workspace_bytes(B, T, H, d, d, dt)
        assert need <= (256 << 20)
        sizes.append(B * T * H)
        x = prefill_inputs(B, T, H, d, d, dt, seed=300 + i, s0_std=s0, device=dev)
        say(f"noalloc case {i}: B={B} T={T} H={H} d={d} {dt} scratch {need} bytes")
        o, S, o_ref, S_ref = _both(x)
        assert torch.equal(o, o_ref), f"case {i}: o differs"
        assert torch.equal(S, S_ref), f"case {i}: S_T differs"
    assert sizes[1] < sizes[0] and sizes[2] < sizes[1]   # later calls on smaller inputs


def test_noalloc_rejects_sizes_beyond_the_scratch():
    dev = need_gpu()
    # fp32 runs the split plan, whose pair blocks of 16,384 tokens x 32 heads
    # exceed the scratch
    B, T, H, d = 1, 16384, 32, 128
    need = kda.kda_chunk_prefill_workspace_bytes(B, T, H, d, d, torch.float32)
    assert need > (256 << 20)
    x = prefill_inputs(B, T, H, d, d, torch.float32, seed=310, device=dev)
    o = torch.zeros_like(x["v"])
    with pytest.raises(kda.KdaError, match="KDA_ERR_WORKSPACE_TOO_SMALL"):
        kda.kda_chunk_prefill_noalloc(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"],
                                      x["g_min"], None, o, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0   # nothing was launched
