"""Build the HIP library libosm.so (gfx950 only) in-tree.

hipcc compiles every source in csrc/ for --offload-arch=gfx950 into one
shared object next to this file.  Packed fp32 VALU instructions are switched
off for the device code (``-packed-fp32-ops``); the host pass warns that it
does not know that feature, which is harmless.  ``-fno-honor-nans``: the C ABI
requires finite inputs, so max operations need not quiet NaN operands.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libosm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Inputs are finite by contract; without NaN semantics fmaxf maps straight
    # to v_max/v_max3 instead of first quieting each operand.
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(_HERE, "csrc", "*.hip")))


def build(verbose: bool = False, out: str | None = None, extra: list[str] | None = None) -> str:
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(_HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # Drop the host pass's notice about the device-only feature; keep the rest.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stderr or "").splitlines() if noise not in ln]
    if msgs:
        print("\n".join(msgs), file=sys.stderr, flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
