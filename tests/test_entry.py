"""The build entry point reaches both builders (the GPU library and the C
oracle) and then imports the package.  The builders themselves are replaced by
recorders here, so this runs in a second; the real compile is the build step."""
import importlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_calls_both_builders(monkeypatch):
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    entry = importlib.import_module("__graft_entry__")
    import oracle
    from linear_attention_recurrence_05_amd import build as kbuild

    calls = []
    monkeypatch.setattr(kbuild, "build", lambda verbose=False: calls.append("libkda"))
    monkeypatch.setattr(oracle, "build", lambda verbose=False: calls.append("oracle"))
    entry.build()
    assert calls == ["libkda", "oracle"]
