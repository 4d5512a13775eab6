"""Build libvspmm.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m sparse_dense_matmul_amd.build`` or through
``__graft_entry__.build()``. The library lands next to this file, where the
binding loads it from.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvspmm.so")
SOURCES = [os.path.join(CSRC, "vspmm.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # only explicit fma contracts, so every instance rounds the same way
        "-ffp-contract=off",
        # float atomics lower to the hardware add, not a compare-and-swap loop
        "-munsafe-fp-atomics",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = True) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc()] + flags() + (extra or []) + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(extra=sys.argv[1:])
