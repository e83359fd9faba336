"""Helpers shared by the GPU tests: device checks, error metrics, plan override."""
from __future__ import annotations

import contextlib
import os

import numpy as np
import pytest
import torch

# Tolerances: max |X_gpu - X_ref| / max |X_ref| per output tensor, for bf16
# inputs and for fp32 inputs respectively (normwise, because outputs cross zero).
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import linear_attention_recurrence_05_amd as kda
    kda.lib()   # raises KdaLibraryMissing if the HIP library was not built
    return torch.device("cuda:0")


def rel_err(x, ref) -> float:
    x = np.asarray(x.detach().float().cpu() if hasattr(x, "detach") else x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.abs(ref).max())
    return float(np.abs(x - ref).max() / max(denom, 1e-30))


@contextlib.contextmanager
def plan(name: str | None):
    """Run the body under KDA_PREFILL_PLAN=name (None or "auto": size-chosen)."""
    old = os.environ.get("KDA_PREFILL_PLAN")
    if name and name != "auto":
        os.environ["KDA_PREFILL_PLAN"] = name
    else:
        os.environ.pop("KDA_PREFILL_PLAN", None)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("KDA_PREFILL_PLAN", None)
        else:
            os.environ["KDA_PREFILL_PLAN"] = old


def say(*a):
    print(*a, flush=True)
