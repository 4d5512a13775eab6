"""Parity at full size and on shapes that stress the walks' bookkeeping:
the 60,000 x 2,000 count matrix (~6M entries) in both layouts at every width
the benchmark and the pages use, compared output by output with the float64
oracle, plus matrices with many tiny slices, slices larger than a register
round, and slices with hundreds of value groups."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, dims, need_gpu, to_dev, vcs_handle, with_empty_groups

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def count60k():
    t = W.count_60k()
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


CASES = [("vcsr", "AB", w) for w in (1, 8, 16, 64)] + [("vcsr", "BA", w) for w in (1, 16)] + \
        [("vcsc", "AB", w) for w in (8, 16)] + [("vcsc", "BA", w) for w in (8, 16, 64)]


@pytest.mark.parametrize("layout,direction,width", CASES)
def test_60k_parity(orc, count60k, layout, direction, width):
    dev = need_gpu()
    L = count60k[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    B = W.dense_normal(np.random.default_rng(width), rows, width)
    Bd = to_dev(B, dev)
    aligned = (layout == "vcsr") == (direction == "AB")
    modes = ["atomic"] if aligned else ["atomic", "deterministic"]
    for mode in modes:
        ws = A.workspace(direction, mode)
        out = A.spmm(Bd, direction, mode=mode, workspace=ws)
        check_close(orc, L, direction, B, out, where=f"60k {layout} {direction} w={width} {mode}")
        if aligned or mode == "deterministic":
            again = A.spmm(Bd, direction, mode=mode, workspace=ws)
            assert torch.equal(again.view(torch.int32), out.view(torch.int32))


def stress_matrices():
    rng = W.rng_for(31)
    yield "tiny_rows", W.count_matrix(120_000, 300, 3.0, 64, rng)        # many slices per wave, empty rows
    yield "long_rows", W.count_matrix(400, 30_000, 3000.0, 255, rng)     # rows beyond one round, ~250 groups
    yield "many_groups", W.count_matrix(6_000, 4_000, 700.0, 255, rng)   # ~200 groups per row
    yield "mixed_rows", mixed_rows(rng)


def mixed_rows(rng):
    """Short rows with a few planted long ones: rows of 1,500-2,900 entries
    (several register rounds each), rows whose entries take ~600 distinct
    values (more groups than one round holds), among Poisson(30) rows."""
    t = W.count_matrix(20_000, 3_000, 30.0, 64, rng)
    planted = rng.choice(20_000, size=12, replace=False)
    keep = ~np.isin(t.rows, planted)
    rows, cols, vals = [t.rows[keep]], [t.cols[keep]], [t.vals[keep]]
    for k, r in enumerate(planted):
        n = int(rng.integers(1_500, 2_900))
        c = rng.choice(3_000, size=n, replace=False)
        v = (rng.integers(1, 600, size=n) if k % 2 else W.count_values(rng, n, 64))
        rows.append(np.full(n, r, dtype=t.rows.dtype))
        cols.append(c.astype(t.cols.dtype))
        vals.append(np.asarray(v, dtype=np.float32))
    return W.Triplets(t.shape, np.concatenate(rows), np.concatenate(cols), np.concatenate(vals))


@pytest.fixture(scope="module")
def stress():
    out = {}
    for name, t in stress_matrices():
        out[name] = {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}
    rng = W.rng_for(32)
    out["empty_groups"] = {lay: with_empty_groups(out["mixed_rows"][lay], rng)
                           for lay in ("vcsr", "vcsc")}
    return out


STRESS = ["tiny_rows", "long_rows", "many_groups", "mixed_rows", "empty_groups"]


@pytest.mark.parametrize("width", [1, 5, 16])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
@pytest.mark.parametrize("name", STRESS)
def test_stress_parity(orc, stress, name, layout, direction, width):
    dev = need_gpu()
    L = stress[name][layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    B = W.dense_normal(np.random.default_rng(width), rows, width)
    aligned = (layout == "vcsr") == (direction == "AB")
    mode = "atomic" if aligned else "deterministic"
    out = A.spmm(to_dev(B, dev), direction, mode=mode, workspace=A.workspace(direction, mode))
    check_close(orc, L, direction, B, out, where=f"{name} {layout} {direction} w={width}")


@pytest.mark.parametrize("name", STRESS)
def test_stress_integer_exact(orc, stress, name):
    dev = need_gpu()
    for layout in ("vcsr", "vcsc"):
        L = stress[name][layout]
        A = vcs_handle(L, dev)
        for direction in ("AB", "BA"):
            rows, _ = dims(L, direction)
            B = W.dense_int(np.random.default_rng(3), rows, 16)
            want = orc.spmm(L, direction, B)
            out = A.spmm(to_dev(B, dev), direction)
            assert np.array_equal(out.cpu().numpy().astype(np.float64), want), (name, layout,
                                                                                direction)
