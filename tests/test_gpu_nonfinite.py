"""Non-finite inputs spread only through stored entries: an output element is
NaN, +Inf or -Inf exactly where the float64 oracle's is (IEEE arithmetic over
the entries of its own slice), and the finite elements meet the float
tolerance. A walk that pads a step with lanes of another slice, or past a
round's end, must keep those lanes' B rows and group values out of its sums
(a zero value times an infinite B element is NaN).

Inputs: B with +Inf, -Inf and NaN elements and one all-Inf row, or the
matrix's values with a few non-finite ones. Matrices chosen so that every walk
family runs: a 20,000 x 2,000 count matrix (the short run-planned walk, its
wider-lane form, the tiled copy, the scatter walk), a 200 x 3,000 one with
slices of ~1,500 entries (the long-slice walk), and the regridding-shaped CSR
operator in float32 and float64 (the CSR walks, the transpose walk)."""

import dataclasses

import numpy as np
import pytest

import workloads as W
from helpers import dims, need_gpu, to_dev, handle

pytestmark = pytest.mark.gpu

TOL = {np.float32: 1e-5, np.float64: 1e-12}


@pytest.fixture(scope="module")
def mats():
    rng = W.rng_for(85)
    t = W.count_matrix(20000, 2000, 100.0, 64, rng)
    tl = W.count_matrix(200, 3000, 1500.0, 64, rng)
    _, c32 = W.config4(np.float32)
    _, c64 = W.config4(np.float64)
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc"),
            "vcsr_long": W.build_vcs(tl, "vcsr"), "vcsc_long": W.build_vcs(tl, "vcsc"),
            "csr32": c32, "csr64": c64}


def _vals(L):
    return L.values if hasattr(L, "major_ptr") else L.val


def _with_vals(L, v):
    return dataclasses.replace(L, **({"values": v} if hasattr(L, "major_ptr") else {"val": v}))


def check_ieee(orc, L, direction, B, got, tol, where):
    ref = orc.spmm(L, direction, B)
    g = got.detach().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, where
    for cls in (np.isnan, np.isposinf, np.isneginf):
        bad = cls(g) != cls(ref)
        assert not bad.any(), (f"{where}: {cls.__name__} differs at {len(np.argwhere(bad))} elements, "
                               f"e.g. {np.argwhere(bad)[:4].tolist()}")
    fin = np.isfinite(ref)
    v = _vals(L)
    Lz = _with_vals(L, np.where(np.isfinite(v), v, 0).astype(v.dtype))
    scale = orc.abs_scale(Lz, direction, np.where(np.isfinite(B), B, 0).astype(B.dtype))
    err = np.abs(np.where(fin, g, 0) - np.where(fin, ref, 0))
    zero = fin & (scale == 0)
    assert not (err[zero] > 0).any(), f"{where}: an output with |A||B| = 0 is not exactly zero"
    pos = fin & (scale > 0)
    rel = float((err[pos] / scale[pos]).max()) if pos.any() else 0.0
    assert rel <= tol, f"{where}: max relative error {rel:.3e} > {tol:g}"
    assert (~fin).sum() > 0, f"{where}: the case spreads no non-finite value"


def poisoned_b(rng, rows, width, dtype):
    B = W.dense_normal(rng, rows, width, dtype)
    r = rng.choice(rows, size=13, replace=False)
    c = rng.integers(0, width, size=13)
    B[r[:4], c[:4]] = np.inf
    B[r[4:8], c[4:8]] = -np.inf
    B[r[8:12], c[8:12]] = np.nan
    B[r[12], :] = np.inf
    return B


def poisoned_vals(rng, L):
    v = _vals(L).copy()
    k = rng.choice(v.size, size=6, replace=False)
    v[k[:2]] = np.inf
    v[k[2:4]] = -np.inf
    v[k[4:]] = np.nan
    return _with_vals(L, v)


@pytest.mark.parametrize("width", [1, 16, 64])
@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("which", ["B", "values"])
@pytest.mark.parametrize("name", ["vcsr", "vcsc", "vcsr_long", "vcsc_long", "csr32", "csr64"])
def test_nonfinite_spreads_through_stored_entries(orc, mats, name, which, direction, mode, width):
    dev = need_gpu()
    L = mats[name]
    dtype = np.float64 if name == "csr64" else np.float32
    rng = np.random.default_rng([width, len(name), ord(which[0]), ord(direction[0]), ord(mode[0])])
    rows, _ = dims(L, direction)
    if which == "values":
        L = poisoned_vals(rng, L)
        B = W.dense_normal(rng, rows, width, dtype)
    else:
        B = poisoned_b(rng, rows, width, dtype)
    A = handle(L, dev)
    kernel = A.plan_info(width, direction, mode)["kernel_name"]
    where = f"{name} {which} {direction} {mode} w={width} ({kernel})"
    Bd = to_dev(B, dev)
    if mode == "deterministic":
        out = A.spmm(Bd, direction, mode=mode, workspace=A.workspace(direction, mode, width))
    else:
        out = A.spmm(Bd, direction)
    check_ieee(orc, L, direction, B, out, TOL[dtype], where)
