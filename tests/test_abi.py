"""The C ABI on the CPU: the library loads, exports every function kda.h
declares, and rejects bad arguments on the host before any HIP call (so these
run without a GPU; no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import linear_attention_recurrence_05_amd as kda
from linear_attention_recurrence_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

# Fake device addresses: aligned, distinct, far apart, never dereferenced
# because validation fails first in every call below.
BASE = 1 << 40
STEP = 1 << 36


def fake(i, misalign=0):
    return ctypes.c_void_p(BASE + i * STEP + misalign)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["kda_abi_version", "kda_status_string", "kda_last_error",
              "kda_chunk_prefill_workspace_bytes", "kda_chunk_prefill", "kda_decode_step",
              "kda_decode_tokens", "kda_chunk_prefill_paged", "kda_decode_step_paged",
              "kda_decode_tokens_paged", "kda_gate_chunk_cumsum", "kda_intra_chunk",
              "kda_chunk_backward_workspace_bytes", "kda_chunk_backward",
              "kda_chunk_prefill_segmented_workspace_bytes", "kda_chunk_prefill_segmented",
              "kda_chunk_prefill_paged_workspace_bytes", "kda_chunk_prefill_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = kda.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in kda.h but not exported"


def test_abi_version_and_status_strings():
    assert kda.abi_version() == 1
    assert kda.status_string(0) == "KDA_OK"
    for code, name in enumerate(_lib._STATUS):
        assert kda.status_string(code) == name
    assert kda.status_string(99) == "KDA_ERR_UNKNOWN"


def prefill(**over):
    """Call kda_chunk_prefill with fake pointers.  Every use below makes the
    call fail host-side validation, so nothing is ever launched."""
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5),
                g_min=-5.0, S0=None, o=fake(7), S_T=fake(8), B=1, T=64, H=2, d_k=32, d_v=32,
                dt=kda.KDA_F32, ws=fake(9), ws_bytes=1 << 33, stream=None)
    args.update(over)
    L = kda.lib()
    st = L.kda_chunk_prefill(args["q"], args["k"], args["v"], args["z"], args["beta"], args["A"],
                             args["g_min"], args["S0"], args["o"], args["S_T"], args["B"],
                             args["T"], args["H"], args["d_k"], args["d_v"], args["dt"],
                             args["ws"], args["ws_bytes"], args["stream"])
    return st, L.kda_last_error().decode()


def decode(**over):
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5),
                g_min=-5.0, S=fake(6), o=fake(7), B=4, H=2, d_k=128, d_v=128,
                dt=kda.KDA_BF16, stream=None)
    args.update(over)
    L = kda.lib()
    st = L.kda_decode_step(args["q"], args["k"], args["v"], args["z"], args["beta"], args["A"],
                           args["g_min"], args["S"], args["o"], args["B"], args["H"],
                           args["d_k"], args["d_v"], args["dt"], args["stream"])
    return st, L.kda_last_error().decode()


E = {n: i for i, n in enumerate(_lib._STATUS)}


@pytest.mark.parametrize("over,code", [
    (dict(q=None), "KDA_ERR_NULL_POINTER"),
    (dict(beta=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=None), "KDA_ERR_NULL_POINTER"),
    (dict(B=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(T=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(H=-1), "KDA_ERR_INVALID_SHAPE"),
    (dict(B=1, T=16, H=(1 << 19) + 1), "KDA_ERR_INVALID_SHAPE"),   # H * d_k above 2^24 (d_k 32)
    (dict(B=1, T=(1 << 30) + 1, H=1), "KDA_ERR_INVALID_SHAPE"),    # T above 2^30
    (dict(B=1, T=2**31 - 1, H=1), "KDA_ERR_INVALID_SHAPE"),
    (dict(g_min=-5.5), "KDA_ERR_INVALID_VALUE"),
    (dict(g_min=0.25), "KDA_ERR_INVALID_VALUE"),
    (dict(g_min=float("nan")), "KDA_ERR_INVALID_VALUE"),
    (dict(d_k=64, d_v=64), "KDA_ERR_UNSUPPORTED"),
    (dict(d_k=32, d_v=128), "KDA_ERR_UNSUPPORTED"),
    (dict(dt=7), "KDA_ERR_UNSUPPORTED"),
    (dict(k=fake(1, misalign=4)), "KDA_ERR_MISALIGNED"),
    (dict(beta=fake(4, misalign=2)), "KDA_ERR_MISALIGNED"),
    (dict(o=fake(0)), "KDA_ERR_ALIASING"),                       # o == q
    (dict(S0=fake(6), S_T=fake(6, misalign=16)), "KDA_ERR_ALIASING"),  # partial overlap
])
def test_prefill_rejects(over, code):
    st, detail = prefill(**over)
    assert st == E[code], (st, detail)
    assert detail


def test_prefill_state_alias_is_allowed_by_validation():
    # S_T == S0 exactly passes validation; with a workspace-requiring shape and
    # no workspace the call then stops at the workspace check, still on the host.
    os.environ["KDA_PREFILL_PLAN"] = "split"
    try:
        st, detail = prefill(S0=fake(6), S_T=fake(6), ws=None, ws_bytes=0)
        assert st == E["KDA_ERR_NULL_POINTER"] and "workspace" in detail
        need = kda.kda_chunk_prefill_workspace_bytes(1, 64, 2, 32, 32, kda.KDA_F32)
        assert need > 0
        st, detail = prefill(S0=fake(6), S_T=fake(6), ws=fake(9), ws_bytes=need - 1)
        assert st == E["KDA_ERR_WORKSPACE_TOO_SMALL"], detail
    finally:
        del os.environ["KDA_PREFILL_PLAN"]


def test_workspace_query():
    assert kda.kda_chunk_prefill_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_BF16) > 0
    assert kda.kda_chunk_prefill_workspace_bytes(0, 4096, 32, 128, 128, kda.KDA_BF16) == 0
    assert kda.kda_chunk_prefill_workspace_bytes(1, 4096, 32, 64, 64, kda.KDA_BF16) == 0
    os.environ["KDA_PREFILL_PLAN"] = "fused:64"
    try:
        assert kda.kda_chunk_prefill_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_BF16) == 0
    finally:
        del os.environ["KDA_PREFILL_PLAN"]


@pytest.mark.parametrize("over,code", [
    (dict(S=None), "KDA_ERR_NULL_POINTER"),
    (dict(B=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(g_min=1.0), "KDA_ERR_INVALID_VALUE"),
    (dict(d_k=16, d_v=16), "KDA_ERR_UNSUPPORTED"),
    (dict(S=fake(6, misalign=8)), "KDA_ERR_MISALIGNED"),
    (dict(beta=fake(4, misalign=1)), "KDA_ERR_MISALIGNED"),
    (dict(o=fake(6)), "KDA_ERR_ALIASING"),
])
def test_decode_rejects(over, code):
    st, detail = decode(**over)
    assert st == E[code], (st, detail)


def tokens(**over):
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5),
                g_min=-5.0, S=fake(6), S_out=fake(7), o=fake(8), B=4, T=4, H=2, d_k=128,
                d_v=128, dt=kda.KDA_BF16, stream=None)
    args.update(over)
    L = kda.lib()
    st = L.kda_decode_tokens(args["q"], args["k"], args["v"], args["z"], args["beta"], args["A"],
                             args["g_min"], args["S"], args["S_out"], args["o"], args["B"],
                             args["T"], args["H"], args["d_k"], args["d_v"], args["dt"],
                             args["stream"])
    return st, L.kda_last_error().decode()


@pytest.mark.parametrize("over,code", [
    (dict(T=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(T=17), "KDA_ERR_INVALID_SHAPE"),
    (dict(S=None), "KDA_ERR_NULL_POINTER"),
    (dict(S_out=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=None), "KDA_ERR_NULL_POINTER"),
    (dict(g_min=-6.0), "KDA_ERR_INVALID_VALUE"),
    (dict(d_k=64, d_v=64), "KDA_ERR_UNSUPPORTED"),
    (dict(S_out=fake(6, misalign=16)), "KDA_ERR_ALIASING"),   # partial overlap with S
    (dict(o=fake(6)), "KDA_ERR_ALIASING"),                     # o over S
    (dict(S_out=fake(1)), "KDA_ERR_ALIASING"),                 # S_out over k
    (dict(S=fake(6, misalign=8)), "KDA_ERR_MISALIGNED"),
])
def test_tokens_rejects(over, code):
    st, detail = tokens(**over)
    assert st == E[code], (st, detail)
    assert detail


def paged_decode(**over):
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5), g_min=-5.0,
                pool=fake(6), n_slots=8, slots=fake(7), o=fake(8), B=4, H=2, d_k=128, d_v=128,
                dt=kda.KDA_BF16, stream=None)
    args.update(over)
    L = kda.lib()
    st = L.kda_decode_step_paged(args["q"], args["k"], args["v"], args["z"], args["beta"], args["A"],
                                 args["g_min"], args["pool"], args["n_slots"], args["slots"],
                                 args["o"], args["B"], args["H"], args["d_k"], args["d_v"],
                                 args["dt"], args["stream"])
    return st, L.kda_last_error().decode()


@pytest.mark.parametrize("over,code", [
    (dict(n_slots=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(pool=None), "KDA_ERR_NULL_POINTER"),
    (dict(slots=None), "KDA_ERR_NULL_POINTER"),
    (dict(slots=fake(7, misalign=2)), "KDA_ERR_MISALIGNED"),
    (dict(o=fake(6)), "KDA_ERR_ALIASING"),          # o over the pool
    (dict(slots=fake(6)), "KDA_ERR_ALIASING"),      # slot table inside the pool
    (dict(d_k=32, d_v=128), "KDA_ERR_UNSUPPORTED"),
])
def test_paged_decode_rejects(over, code):
    st, detail = paged_decode(**over)
    assert st == E[code], (st, detail)
    assert detail


def test_paged_prefill_and_tokens_reject():
    L = kda.lib()
    # prefill: the split plan's workspace is checked like the dense call's
    os.environ["KDA_PREFILL_PLAN"] = "split"
    try:
        st = L.kda_chunk_prefill_paged(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), -5.0,
                                       fake(6), 4, fake(7), fake(7), fake(8), 1, 64, 2, 32, 32,
                                       kda.KDA_F32, None, 0, None)
        assert st == E["KDA_ERR_NULL_POINTER"]
        need = kda.kda_chunk_prefill_paged_workspace_bytes(1, 64, 2, 32, 32, kda.KDA_F32)
        st = L.kda_chunk_prefill_paged(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), -5.0,
                                       fake(6), 4, None, None, fake(8), 1, 64, 2, 32, 32,
                                       kda.KDA_F32, fake(9), need - 1, None)
        assert st == E["KDA_ERR_WORKSPACE_TOO_SMALL"]
    finally:
        del os.environ["KDA_PREFILL_PLAN"]
    # tokens: both tables required, T bounded
    st = L.kda_decode_tokens_paged(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), -5.0,
                                   fake(6), 4, fake(7), None, fake(8), 2, 3, 2, 32, 32,
                                   kda.KDA_F32, None)
    assert st == E["KDA_ERR_NULL_POINTER"]
    st = L.kda_decode_tokens_paged(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), -5.0,
                                   fake(6), 4, fake(7), fake(7), fake(8), 2, 17, 2, 32, 32,
                                   kda.KDA_F32, None)
    assert st == E["KDA_ERR_INVALID_SHAPE"]


def test_noalloc_prefill_rejects_on_the_host():
    """kda_chunk_prefill_noalloc checks its arguments like kda_chunk_prefill,
    and rejects sizes whose workspace exceeds its static scratch, before any
    HIP call."""
    L = kda.lib()

    def call(**over):
        a = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5), g_min=-5.0,
                 S0=None, o=fake(7), S_T=fake(8), B=1, T=64, H=2, d_k=32, d_v=32, dt=kda.KDA_F32)
        a.update(over)
        st = L.kda_chunk_prefill_noalloc(*(a[n] for n in ("q", "k", "v", "z", "beta", "A",
                                                          "g_min", "S0", "o", "S_T", "B", "T",
                                                          "H", "d_k", "d_v", "dt")), None)
        return st, L.kda_last_error().decode()

    assert call(q=None)[0] == E["KDA_ERR_NULL_POINTER"]
    assert call(g_min=1.0)[0] == E["KDA_ERR_INVALID_VALUE"]
    assert call(o=fake(0))[0] == E["KDA_ERR_ALIASING"]
    B, T, H, d = 1, 16384, 32, 128
    need = kda.kda_chunk_prefill_workspace_bytes(B, T, H, d, d, kda.KDA_BF16)
    assert need > 256 << 20
    st, detail = call(B=B, T=T, H=H, d_k=d, d_v=d, dt=kda.KDA_BF16)
    assert st == E["KDA_ERR_WORKSPACE_TOO_SMALL"], detail
    assert f"need {need} bytes" in detail and str(256 << 20) in detail


def test_paged_prefill_workspace_query_is_its_own():
    """At sizes where the dense prefill runs the segment scan (a smaller
    workspace), the paged prefill asks for exactly its own query's size."""
    L = kda.lib()
    B, T, H, d = 1, 65536, 32, 128
    assert kda.kda_chunk_prefill_segments(B, T, H, d, d, kda.KDA_BF16) > 1
    dense = kda.kda_chunk_prefill_workspace_bytes(B, T, H, d, d, kda.KDA_BF16)
    need = kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, kda.KDA_BF16)
    assert need > dense > 0
    st = L.kda_chunk_prefill_paged(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), -5.0,
                                   fake(6), 4, fake(7), fake(7), fake(8), B, T, H, d, d,
                                   kda.KDA_BF16, fake(9), need - 1, None)
    detail = L.kda_last_error().decode()
    assert st == E["KDA_ERR_WORKSPACE_TOO_SMALL"]
    assert f"{need} needed" in detail, detail
    assert kda.kda_chunk_prefill_paged_workspace_bytes(B, T, H, 64, 64, kda.KDA_BF16) == 0


def test_gate_and_intra_reject():
    L = kda.lib()
    st = L.kda_gate_chunk_cumsum(fake(0), fake(1), -5.0, None, 1, 16, 1, 32, kda.KDA_F32, None)
    assert st == E["KDA_ERR_NULL_POINTER"]
    st = L.kda_gate_chunk_cumsum(fake(0), fake(1), -5.0, fake(0), 1, 16, 1, 32, kda.KDA_F32, None)
    assert st == E["KDA_ERR_ALIASING"]
    st = L.kda_intra_chunk(fake(0), fake(1), fake(2), fake(3), fake(4), -6.0, fake(5), fake(6),
                           fake(7), 1, 16, 1, 32, kda.KDA_F32, None)
    assert st == E["KDA_ERR_INVALID_VALUE"]


def test_binding_raises_named_errors():
    # a status code from the library becomes a KdaError naming it, with the
    # thread's detail string
    L = kda.lib()
    st = L.kda_gate_chunk_cumsum(fake(0), fake(1), -5.0, fake(2), 1, 16, 1, 48, kda.KDA_F32, None)
    with pytest.raises(kda.KdaError, match="KDA_ERR_UNSUPPORTED"):
        _lib._check(st, "kda_gate_chunk_cumsum")


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 16, 2, 32)
    with pytest.raises(ValueError, match="CUDA device"):
        kda.kda_gate_chunk_cumsum(x, torch.zeros(2), -5.0, torch.zeros_like(x), stream=0)
    with pytest.raises(ValueError, match="CUDA device"):
        kda.kda_chunk_prefill(x, x, x, x, torch.zeros(1, 16, 2), torch.zeros(2), -5.0, None,
                              torch.zeros_like(x), None, None, stream=0)


def _prefill_args(B=1, T=16, H=2, d=32, dt=None):
    import torch
    dt = dt or torch.float32
    t = lambda *s, dtype=dt: torch.zeros(*s, dtype=dtype)
    return dict(q=t(B, T, H, d), k=t(B, T, H, d), v=t(B, T, H, d), z=t(B, T, H, d),
                beta=t(B, T, H, dtype=torch.float32), A=t(H, dtype=torch.float32), g_min=-5.0,
                S0=t(B, H, d, d, dtype=torch.float32), o=t(B, T, H, d),
                S_T=t(B, H, d, d, dtype=torch.float32))


@pytest.mark.parametrize("name,bad,match", [
    ("beta", lambda a: a["beta"].to(__import__("torch").bfloat16), "beta must be"),
    ("A", lambda a: a["A"].double(), "A must be"),
    ("k", lambda a: a["k"].to(__import__("torch").bfloat16), "k must be"),
    ("o", lambda a: a["o"].to(__import__("torch").bfloat16), "o must be"),
    ("S0", lambda a: a["S0"][:, :1].contiguous(), "S0 has shape"),       # undersized state
    ("S_T", lambda a: a["S_T"].reshape(-1)[:100], "S_T has shape"),
    ("v", lambda a: a["v"][:, :8].contiguous(), "v has shape"),
    ("z", lambda a: a["z"].transpose(1, 2), "z must be contiguous"),
    ("beta", lambda a: None, "beta is required"),
])
def test_binding_rejects_mistyped_and_undersized(monkeypatch, name, bad, match):
    monkeypatch.setattr(_lib, "_DEVICE_TYPE", "cpu")
    a = _prefill_args()
    a[name] = bad(a)
    with pytest.raises(ValueError, match=match):
        kda.kda_chunk_prefill(a["q"], a["k"], a["v"], a["z"], a["beta"], a["A"], a["g_min"],
                              a["S0"], a["o"], a["S_T"], None, stream=0)


def test_binding_rejects_mixed_devices(monkeypatch):
    import torch
    monkeypatch.setattr(_lib, "_DEVICE_TYPE", "cpu")
    a = _prefill_args()
    k = torch.zeros(1, 16, 2, 32, device="meta")
    with pytest.raises(ValueError, match="k is on meta"):
        kda.kda_chunk_prefill(a["q"], k, a["v"], a["z"], a["beta"], a["A"], -5.0, None,
                              a["o"], None, None, stream=0)


def test_binding_checks_decode_and_paged(monkeypatch):
    import torch
    monkeypatch.setattr(_lib, "_DEVICE_TYPE", "cpu")
    B, H, d = 3, 2, 32
    q = torch.zeros(B, H, d)
    beta, A = torch.zeros(B, H), torch.zeros(H)
    with pytest.raises(ValueError, match="S has shape"):   # a state too small for B
        kda.kda_decode_step(q, q, q, q, beta, A, -5.0, torch.zeros(B - 1, H, d, d),
                            torch.zeros(B, H, d), stream=0)
    with pytest.raises(ValueError, match="pool must be"):
        kda.kda_decode_step_paged(q, q, q, q, beta, A, -5.0, torch.zeros(4, H, d, d).double(),
                                  torch.zeros(B, dtype=torch.int32), torch.zeros(B, H, d),
                                  stream=0)
    with pytest.raises(ValueError, match="slots must be"):
        kda.kda_decode_step_paged(q, q, q, q, beta, A, -5.0, torch.zeros(4, H, d, d),
                                  torch.zeros(B, dtype=torch.int64), torch.zeros(B, H, d),
                                  stream=0)
    with pytest.raises(ValueError, match="slots has shape"):
        kda.kda_decode_step_paged(q, q, q, q, beta, A, -5.0, torch.zeros(4, H, d, d),
                                  torch.zeros(B + 1, dtype=torch.int32), torch.zeros(B, H, d),
                                  stream=0)
    x = torch.zeros(B, 4, H, d)
    with pytest.raises(ValueError, match="S_out has shape"):
        kda.kda_decode_tokens(x, x, x, x, torch.zeros(B, 4, H), A, -5.0,
                              torch.zeros(B, H, d, d), torch.zeros(B, H, d, d - 1), x.clone(),
                              stream=0)


def test_binding_checks_backward(monkeypatch):
    import torch
    monkeypatch.setattr(_lib, "_DEVICE_TYPE", "cpu")
    a = _prefill_args()
    g = {n: torch.zeros_like(a[n]) for n in ("q", "k", "v", "z")}
    with pytest.raises(ValueError, match="dbeta must be"):
        kda.kda_chunk_backward(a["q"], a["k"], a["v"], a["z"], a["beta"], a["A"], -5.0, None,
                               a["o"], None, g["q"], g["k"], g["v"], g["z"],
                               torch.zeros(1, 16, 2, dtype=torch.bfloat16), torch.zeros(2),
                               None, None, stream=0)
    with pytest.raises(ValueError, match="dA has shape"):
        kda.kda_chunk_backward(a["q"], a["k"], a["v"], a["z"], a["beta"], a["A"], -5.0, None,
                               a["o"], None, g["q"], g["k"], g["v"], g["z"],
                               torch.zeros(1, 16, 2), torch.zeros(3), None, None, stream=0)


def backward(**over):
    """Call kda_chunk_backward with fake pointers; every use below fails
    host-side validation, so nothing is launched."""
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5), g_min=-5.0,
                S0=fake(6), dO=fake(7), dST=fake(8), dq=fake(9), dk=fake(10), dv=fake(11),
                dz=fake(12), dbeta=fake(13), dA=fake(14), dS0=fake(15), B=1, T=64, H=2, d_k=32,
                d_v=32, dt=kda.KDA_F32, ws=fake(16), ws_bytes=0, stream=None)
    args.update(over)
    L = kda.lib()
    st = L.kda_chunk_backward(*(args[n] for n in ("q", "k", "v", "z", "beta", "A", "g_min", "S0",
                                                  "dO", "dST", "dq", "dk", "dv", "dz", "dbeta",
                                                  "dA", "dS0", "B", "T", "H", "d_k", "d_v", "dt",
                                                  "ws", "ws_bytes", "stream")))
    return st, L.kda_last_error().decode()


@pytest.mark.parametrize("over,code", [
    (dict(dO=None), "KDA_ERR_NULL_POINTER"),
    (dict(dz=None), "KDA_ERR_NULL_POINTER"),
    (dict(dA=None), "KDA_ERR_NULL_POINTER"),
    (dict(ws=None), "KDA_ERR_NULL_POINTER"),
    (dict(T=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(g_min=-6.0), "KDA_ERR_INVALID_VALUE"),
    (dict(d_k=64, d_v=64), "KDA_ERR_UNSUPPORTED"),
    (dict(dS0=fake(15, misalign=4)), "KDA_ERR_MISALIGNED"),
    (dict(dST=fake(8, misalign=8)), "KDA_ERR_MISALIGNED"),
    (dict(), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(ws_bytes=1 << 33, dq=fake(0)), "KDA_ERR_ALIASING"),          # dq == q
    (dict(ws_bytes=1 << 33, dS0=fake(14)), "KDA_ERR_ALIASING"),        # dS0 == dA
    (dict(ws_bytes=1 << 33, ws=fake(12, misalign=16)), "KDA_ERR_ALIASING"),   # inside dz
])
def test_backward_rejects(over, code):
    st, detail = backward(**over)
    assert st == E[code], (st, detail)
    assert detail


def test_backward_workspace_query():
    n = kda.kda_chunk_backward_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_BF16)
    # at least the chunk-start states: 32 heads x 256 chunks x 128 x 128 fp32
    assert n >= 32 * 256 * 128 * 128 * 4
    # the chunkwise plan (bf16, d = 128): per extra chunk of every head, a
    # start state, an end-state gradient, the chain's operand block, the fp32
    # triangular factors (P, Aqk, Ninv) and a dA term; the segment scan behind
    # the segment-parallel forward sweep runs state-only passes here (no zero
    # v, no scratch o)
    n2 = kda.kda_chunk_backward_workspace_bytes(1, 8192, 32, 128, 128, kda.KDA_BF16)
    extra = 32 * 256 * (2 * 128 * 128 * 4 + 13824 + 3 * 16 * 16 * 4 + 4)
    assert extra <= n2 - n <= extra + (1 << 20)
    # the token-level sweep (forced) holds the per-token corrections and
    # bounded partial sums instead
    os.environ["KDA_BACKWARD_PLAN"] = "sweep"
    try:
        ns = kda.kda_chunk_backward_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_BF16)
        ns2 = kda.kda_chunk_backward_workspace_bytes(1, 8192, 32, 128, 128, kda.KDA_BF16)
        nc = kda.kda_chunk_backward_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_F32)
    finally:
        del os.environ["KDA_BACKWARD_PLAN"]
    extra = 32 * 256 * 128 * 128 * 4 + 32 * 4096 * 128 * 4
    assert extra <= ns2 - ns <= extra + (1 << 20)
    # fp32 takes the token-level sweep without any setting
    assert kda.kda_chunk_backward_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_F32) == nc
    # the chain plan adds the cumulative log-decay, Tm, Aqk, gamma and the
    # end-state gradient of every chunk to the sweep's
    os.environ["KDA_BACKWARD_PLAN"] = "chain"
    try:
        nch = kda.kda_chunk_backward_workspace_bytes(1, 4096, 32, 128, 128, kda.KDA_BF16)
    finally:
        del os.environ["KDA_BACKWARD_PLAN"]
    chain = (32 * 4096 * 128 * 4 + 2 * 32 * 256 * 256 * 4 + 32 * 256 * 128 * 4
             + 32 * 256 * 128 * 128 * 4)
    assert chain <= nch - ns <= chain + (1 << 20)
    assert kda.kda_chunk_backward_workspace_bytes(0, 64, 2, 32, 32, kda.KDA_F32) == 0
    assert kda.kda_chunk_backward_workspace_bytes(1, 64, 2, 64, 64, kda.KDA_F32) == 0


def segmented(**over):
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), beta=fake(4), A=fake(5), g_min=-5.0,
                S0=None, o=fake(7), S_T=fake(8), B=1, T=64, H=2, d_k=32, d_v=32, n_seg=4,
                dt=kda.KDA_F32, ws=fake(9), ws_bytes=0, stream=None)
    args.update(over)
    L = kda.lib()
    st = L.kda_chunk_prefill_segmented(*(args[n] for n in ("q", "k", "v", "z", "beta", "A",
                                                           "g_min", "S0", "o", "S_T", "B", "T",
                                                           "H", "d_k", "d_v", "n_seg", "dt", "ws",
                                                           "ws_bytes", "stream")))
    return st, L.kda_last_error().decode()


@pytest.mark.parametrize("over,code", [
    (dict(n_seg=0), "KDA_ERR_INVALID_SHAPE"),
    (dict(n_seg=5), "KDA_ERR_INVALID_SHAPE"),              # does not divide T = 64
    (dict(ws=None), "KDA_ERR_NULL_POINTER"),
    (dict(), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(ws_bytes=1 << 33, o=fake(2)), "KDA_ERR_ALIASING"),
    (dict(g_min=-7.0), "KDA_ERR_INVALID_VALUE"),
])
def test_segmented_rejects(over, code):
    st, detail = segmented(**over)
    assert st == E[code], (st, detail)
    assert detail


def test_segmented_workspace_query():
    n1 = kda.kda_chunk_prefill_segmented_workspace_bytes(1, 4096, 32, 128, 128, 1, kda.KDA_BF16)
    n4 = kda.kda_chunk_prefill_segmented_workspace_bytes(1, 4096, 32, 128, 128, 4, kda.KDA_BF16)
    # one segment: 32 units run the split plan, whose passes need a zero value
    # tensor of v's size; four state tensors per segment
    assert n1 >= 4096 * 32 * 128 * 2 + 4 * 32 * 128 * 128 * 4
    # four segments: 128 units run the fused plan's state-only passes (no zero
    # v); the four state tensors per segment remain
    assert 4 * 4 * 32 * 128 * 128 * 4 <= n4 < 4096 * 32 * 128 * 2 + 4 * 4 * 32 * 128 * 128 * 4
    assert kda.kda_chunk_prefill_segmented_workspace_bytes(1, 4096, 32, 128, 128, 3,
                                                           kda.KDA_BF16) == 0


def test_prefill_plan_names():
    """kda_chunk_prefill_plan names the plan the dense entry point runs (host
    logic; without a GPU no device reports CUs, so the ring plan is never
    chosen here)."""
    f = kda.kda_chunk_prefill_plan
    bf, f32 = kda.KDA_BF16, kda.KDA_F32
    assert f(1, 1048576, 32, 128, 128, bf) == "segment scan"
    assert f(8, 32768, 32, 128, 128, bf) == "fused:128"    # 256 units
    assert f(1, 4096, 128, 128, 128, bf) == "fused:64"     # 128 units
    assert f(1, 4096, 32, 128, 128, bf) in ("split", "ring")
    assert f(1, 4096, 32, 32, 32, f32) == "split"          # the ring plan is bf16 at d = 128
    assert f(0, 4096, 32, 128, 128, bf) == ""              # rejected sizes
    assert f(1, 4096, 32, 64, 64, bf) == ""


def test_prefill_segment_choice():
    """Which sizes kda_chunk_prefill runs as a segment scan (host logic)."""
    f = kda.kda_chunk_prefill_segments
    bf, f32 = kda.KDA_BF16, kda.KDA_F32
    assert f(1, 4096, 32, 128, 128, bf) == 1          # short: direct
    assert f(1, 32768, 32, 128, 128, bf) == 1         # below 65,536 tokens
    assert f(1, 65536, 32, 128, 128, bf) == 8         # 32 heads -> 256 units
    assert f(1, 1048576, 32, 128, 128, bf) == 8
    assert f(1, 65536, 16, 128, 128, bf) == 16
    assert f(1, 65536, 24, 128, 128, bf) == 8         # 192 units
    assert f(2, 65536, 32, 128, 128, bf) == 1         # 64 heads fill the chip
    # 2 or 4 heads: at most 16 segments of >= 4,096 tokens, too few units
    # (32, 64 < 128) for the fused plan's state-only passes: direct
    assert f(1, 65536, 2, 128, 128, bf) == 1
    assert f(1, 65536, 4, 128, 128, bf) == 1
    assert f(1, 1048576, 2, 128, 128, bf) == 128      # 256 units of 8,192 tokens
    assert f(1, 1048576, 32, 128, 128, f32) == 1      # fp32: direct
    assert f(1, 1048576, 32, 32, 32, bf) == 1         # d = 32: direct
    assert f(1, 65536 + 16, 32, 128, 128, bf) == 1    # T not a multiple of 16 R: direct
    assert f(0, 65536, 32, 128, 128, bf) == 0         # rejected arguments
    # the workspace query follows the choice
    assert (kda.kda_chunk_prefill_workspace_bytes(1, 65536, 32, 128, 128, bf)
            == kda.kda_chunk_prefill_segmented_workspace_bytes(1, 65536, 32, 128, 128, 8, bf))
    os.environ["KDA_PREFILL_PLAN"] = "split"
    try:
        assert f(1, 1048576, 32, 128, 128, bf) == 1   # a forced plan runs as forced
    finally:
        del os.environ["KDA_PREFILL_PLAN"]
