"""Build ``oracle/liboracle.so`` from ``kda_oracle.c`` with gcc (fp64, OpenMP).

TEST INFRASTRUCTURE ONLY.  No fast-math: the oracle keeps IEEE double
semantics."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str | None = None, out: str | None = None) -> str:
    """Compile ``src`` (default: the committed oracle source) into ``out``."""
    src = src or os.path.join(HERE, "kda_oracle.c")
    out = out or library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
