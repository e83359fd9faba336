"""Seeded synthetic inputs for the KDA recurrence.

This module holds only the input recipe -- shapes, dtypes, value
distributions, seeds -- and none of the method's arithmetic.  Both the GPU
tests/benchmark and the oracle checks draw their inputs from here.

The pages measure nothing on a dataset and no trained weights are available,
so every workload is synthetic with the distributions below:

* q, k ~ N(0, 1) in fp32, L2-normalised per (token, head), then cast;
* v, z ~ N(0, 1), then cast;
* beta = Sigmoid(N(0, 1)), fp32;
* A_h ~ U(-1, 1) per head, fp32;
* S0 ~ N(0, 0.01) (variance 0.01, i.e. std 0.1) fp32 where a config carries a
  state, zeros otherwise;
* g_min = -5 (the value the dev.to page gives for the gate's lower bound).

Draw order from one ``torch.Generator`` seeded with the config index:
q, k, v, z, beta-logits, A, S0.  For decode: A, S0 first, then per step
q, k, v, z, beta-logits.  The generator lives on the device the tensors are
made on (CPU or GPU); the oracle always receives copies of the exact tensors
the GPU saw, so the two never need to agree on a random stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

G_MIN = -5.0
CHUNK = 16


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    s0_std: float | None
    seed: int
    note: str = ""


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    s0_std: float
    steps: int
    seed: int
    note: str = ""


# The five synthetic workloads (indices match their seeds).
PREFILL_CONFIGS = {
    0: PrefillConfig("tiny_fp32", 1, 64, 2, 32, 32, torch.float32, None, 0,
                     "B1 H2 T64 d32, fp32 throughout"),
    1: PrefillConfig("mid_bf16", 1, 4096, 32, 128, 128, torch.bfloat16, None, 1,
                     "B1 H32 T4096 d128, bf16 q/k/v/z"),
    2: PrefillConfig("batched_carry_bf16", 8, 32768, 32, 128, 128, torch.bfloat16, 0.1, 2,
                     "B8 H32 T32768 d128, bf16, S0 ~ N(0, 0.01)"),
    3: PrefillConfig("million_bf16", 1, 1048576, 32, 128, 128, torch.bfloat16, None, 3,
                     "B1 H32 T1048576 d128, bf16"),
}
DECODE_CONFIG = DecodeConfig("decode_b256", 256, 32, 128, 128, torch.bfloat16, 0.1, 1000, 4,
                             "B256 H32 d128, fp32 state 512 MiB in place, 1000 steps")


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(gen, shape, device):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Rows of the last axis scaled to unit L2 norm, in fp32 (no epsilon)."""
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def prefill_inputs(B, T, H, dk, dv, dtype=torch.bfloat16, seed=0, s0_std=None,
                   device="cpu"):
    """Dict with q, k, z [B,T,H,dk], v [B,T,H,dv] (``dtype``), beta [B,T,H],
    A [H], S0 [B,H,dk,dv] or None (fp32), g_min."""
    gen = _gen(seed, device)
    q = _unit_rows(_randn(gen, (B, T, H, dk), device)).to(dtype)
    k = _unit_rows(_randn(gen, (B, T, H, dk), device)).to(dtype)
    v = _randn(gen, (B, T, H, dv), device).to(dtype)
    z = _randn(gen, (B, T, H, dk), device).to(dtype)
    beta = torch.sigmoid(_randn(gen, (B, T, H), device))
    A = torch.rand(H, generator=gen, device=device, dtype=torch.float32) * 2.0 - 1.0
    S0 = None
    if s0_std:
        S0 = _randn(gen, (B, H, dk, dv), device) * float(s0_std)
    return dict(q=q, k=k, v=v, z=z, beta=beta, A=A, S0=S0, g_min=G_MIN)


def config_inputs(index: int, device="cpu", T: int | None = None):
    """Inputs of prefill config ``index``; ``T`` overrides the length (a prefix
    of the same recipe is NOT implied -- a new draw with the shorter shape)."""
    c = PREFILL_CONFIGS[index]
    return prefill_inputs(c.B, T or c.T, c.H, c.dk, c.dv, c.dtype, c.seed, c.s0_std, device)


def decode_state(B, H, dk, dv, seed=4, s0_std=0.1, device="cpu"):
    """(generator, A [H], S [B,H,dk,dv] fp32) for a decode run; keep drawing the
    per-step inputs from the returned generator with :func:`decode_step_inputs`."""
    gen = _gen(seed, device)
    A = torch.rand(H, generator=gen, device=device, dtype=torch.float32) * 2.0 - 1.0
    S = _randn(gen, (B, H, dk, dv), device) * float(s0_std)
    return gen, A, S


def decode_step_inputs(gen, B, H, dk, dv, dtype=torch.bfloat16, device="cpu", steps=None):
    """One decode step's q, k, z [B,H,dk], v [B,H,dv], beta [B,H]; with
    ``steps`` = n, a leading step axis of length n is added (drawn step by step
    in the same order as n single calls would draw them)."""
    if steps is None:
        q = _unit_rows(_randn(gen, (B, H, dk), device)).to(dtype)
        k = _unit_rows(_randn(gen, (B, H, dk), device)).to(dtype)
        v = _randn(gen, (B, H, dv), device).to(dtype)
        z = _randn(gen, (B, H, dk), device).to(dtype)
        beta = torch.sigmoid(_randn(gen, (B, H), device))
        return dict(q=q, k=k, v=v, z=z, beta=beta)
    parts = [decode_step_inputs(gen, B, H, dk, dv, dtype, device) for _ in range(steps)]
    return {key: torch.stack([p[key] for p in parts]) for key in parts[0]}


def backward_grads(B, T, H, dk, dv, dtype=torch.bfloat16, seed=0, with_dST=True,
                   device="cpu"):
    """Incoming gradients for a backward call: dO ~ N(0, 1) [B,T,H,dv] in the
    input dtype and, if asked, dS_T ~ N(0, 1) [B,H,dk,dv] fp32, drawn in that
    order from their own generator (seed + 1000)."""
    gen = _gen(seed + 1000, device)
    dO = _randn(gen, (B, T, H, dv), device).to(dtype)
    dST = _randn(gen, (B, H, dk, dv), device) if with_dST else None
    return dict(dO=dO, dST=dST)
