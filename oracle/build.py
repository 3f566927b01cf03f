"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, OpenMP for row-level parallelism only, no fast-math: every
floating-point operation keeps IEEE binary64 semantics.
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False, src: str | None = None, out: str | None = None) -> str:
    """Compile ``src`` (default: the committed oracle.c) into ``out``."""
    src = src or os.path.join(_HERE, "oracle.c")
    out = out or os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
