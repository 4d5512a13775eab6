"""The scatter walk (a misaligned direction in atomic mode) on shapes that
stress its bookkeeping: runs of hundreds of empty slices and of empty value
groups (more than the 64 a window holds), one slice holding every entry, a
matrix with fewer entries than the grid has waves, and widths that leave lanes
idle or need several column passes. Both ways of adding run: into a private
LDS copy of a small, narrow output, and straight into the output with L2
atomics. Float results are judged against the float64 oracle; integer data
must match it exactly, whatever order the atomics land in."""

import numpy as np
import pytest

import workloads as W
from helpers import check_close, csr_handle, dims, need_gpu, to_dev, vcs_handle, with_empty_groups

pytestmark = pytest.mark.gpu

WIDTHS = [1, 3, 8, 16, 17, 64, 100]


def gapped_rows(rng):
    """100,000 x 300, rows active only in alternate blocks of 500 (so runs of
    500 empty rows), Poisson(1.2) entries per active row."""
    m, n = 100_000, 300
    active = (np.arange(m) // 500) % 2 == 0
    counts = np.where(active, rng.poisson(1.2, size=m), 0)
    rows, cols = W.sample_columns(rng, counts, n)
    return W.Triplets((m, n), rows, cols, W.count_values(rng, rows.size, 64))


def one_slice(rng):
    """A single row of 5,000 entries over 40,000 columns."""
    return W.count_matrix(1, 40_000, 5_000.0, 255, rng)


@pytest.fixture(scope="module")
def mats():
    rng = W.rng_for(41)
    g, o = gapped_rows(rng), one_slice(rng)
    t = W.tiny_count(3, 5, 0.3, 9, rng)
    out = {}
    for name, trip in (("gapped", g), ("one_slice", o), ("tiny", t)):
        out[name] = {"vcsr": W.build_vcs(trip, "vcsr"), "vcsc": W.build_vcs(trip, "vcsc"),
                     "csr32": W.build_csr(trip)}
        c = out[name]["csr32"]
        out[name]["csr64"] = W.Csr(c.shape, c.row_ptr, c.col, c.val.astype(np.float64))
    out["empty_groups"] = {lay: with_empty_groups(out["gapped"][lay], W.rng_for(42), n_rows=8,
                                                  per_row=150)
                           for lay in ("vcsr", "vcsc")}
    return out


def scatter_direction(layout):
    # the direction whose output rows are the layout's minor indices
    return "AB" if layout == "vcsc" else "BA"


def make(L, dev):
    return vcs_handle(L, dev) if hasattr(L, "major_ptr") else csr_handle(L, dev)


CASES = [(name, lay) for name in ("gapped", "one_slice", "tiny")
         for lay in ("vcsr", "vcsc", "csr32", "csr64")] + \
        [("empty_groups", "vcsr"), ("empty_groups", "vcsc")]


@pytest.mark.parametrize("width", WIDTHS)
@pytest.mark.parametrize("name,layout", CASES)
def test_scatter_parity(orc, mats, name, layout, width):
    dev = need_gpu()
    L = mats[name][layout]
    A = make(L, dev)
    direction = scatter_direction(layout)
    assert A.plan_info(width, direction)["kernel_name"] == "k_scatter"
    rows, _ = dims(L, direction)
    dtype = np.float64 if layout == "csr64" else np.float32
    B = W.dense_normal(np.random.default_rng(width), rows, width, dtype=dtype)
    out = A.spmm(to_dev(B, dev), direction)
    tol = 1e-12 if layout == "csr64" else 1e-5
    check_close(orc, L, direction, B, out, tol=tol, where=f"{name} {layout} w={width}")


@pytest.mark.parametrize("name,layout", CASES)
def test_scatter_integer_exact(orc, mats, name, layout):
    dev = need_gpu()
    L = mats[name][layout]
    A = make(L, dev)
    direction = scatter_direction(layout)
    rows, _ = dims(L, direction)
    dtype = np.float64 if layout == "csr64" else np.float32
    for width in (1, 8, 16):
        B = W.dense_int(np.random.default_rng(7), rows, width, dtype=dtype)
        out = A.spmm(to_dev(B, dev), direction)
        want = orc.spmm(L, direction, B)
        assert np.array_equal(out.cpu().numpy().astype(np.float64), want), (name, layout, width)


def test_both_add_paths_run(mats):
    """The cases above include outputs added through the LDS copy and
    outputs added with L2 atomics alone."""
    dev = need_gpu()
    seen = set()
    for name, layout in CASES:
        A = make(mats[name][layout], dev)
        for width in WIDTHS:
            seen.add(A.plan_info(width, scatter_direction(layout))["lds_staged"])
    assert seen == {0, 1}
