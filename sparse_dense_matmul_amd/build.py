"""Build libvspmm.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m sparse_dense_matmul_amd.build`` or through
``__graft_entry__.build()``. The library lands next to this file, where the
binding loads it from. Each translation unit (the host code with the layout
builders, and one per kernel family; the VCS walks once per vector width and
k_short once per element type) is
compiled to an object in parallel under ``_build/``, then the objects are
linked into the library.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvspmm.so")
# the benchmark's ceiling probes (not part of the product library)
PROBE_LIB = os.path.join(HERE, "libvspmm_probe.so")
PROBE_SRC = "probe.hip"
OBJDIR = os.path.join(HERE, "_build")
# (source, extra defines, object name)
UNITS = [
    ("vspmm.hip", [], "vspmm"),
    ("walk_short.hip", ["-DVSPMM_ELT=float"], "walk_short_f32"),
    ("walk_short.hip", ["-DVSPMM_ELT=double"], "walk_short_f64"),
    ("walk_long.hip", [], "walk_long"),
    ("walk_plain.hip", [], "walk_plain"),
    ("walk_scatter.hip", [], "walk_scatter"),
] + [(f"walk_vcs_{kind}.hip", [f"-DVSPMM_VEC={v}"], f"walk_vcs_{kind}_v{v}")
     for kind in ("rows", "long") for v in (1, 2, 4)]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # only explicit fma contracts, so every instance rounds the same way
        "-ffp-contract=off",
        # float atomics lower to the hardware add, not a compare-and-swap loop
        "-munsafe-fp-atomics",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
    ]


def _up_to_date(obj: str, dep: str, cmd: list[str]) -> bool:
    """True when obj was built by the same command and is newer than every
    file its dependency list names."""
    try:
        t = os.path.getmtime(obj)
        text = open(dep).read()
        if open(obj + ".cmd").read() != " ".join(cmd):
            return False
    except OSError:
        return False
    files = text.replace("\\\n", " ").split(":", 1)[1].split()
    return all(os.path.exists(f) and os.path.getmtime(f) <= t for f in files)


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = True,
          jobs: int | None = None, incremental: bool = False) -> str:
    """Compile every unit and link. With incremental, a unit whose object is
    newer than the sources and headers it was built from is not compiled
    again (a development shortcut; the default always compiles)."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    base = flags() + (extra or [])

    def compile_unit(unit):
        src, defs, name = unit
        obj = os.path.join(OBJDIR, name + ".o")
        dep = os.path.join(OBJDIR, name + ".d")
        cmd = [cc] + base + defs + ["-c", "-o", obj, os.path.join(CSRC, src)]
        if incremental and _up_to_date(obj, dep, cmd):
            return obj
        with open(obj + ".cmd", "w") as fh:
            fh.write(" ".join(cmd))
        cmd = cmd + ["-MD", "-MF", dep]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = jobs or min(len(UNITS), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        probe = pool.submit(compile_unit, (PROBE_SRC, [], "probe"))
        objs = list(pool.map(compile_unit, UNITS))
        probe_obj = probe.result()
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    tmp = PROBE_LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, probe_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    inc = "--incremental" in args
    build(extra=[a for a in args if a != "--incremental"], incremental=inc)
