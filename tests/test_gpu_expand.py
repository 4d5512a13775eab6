"""VCS expansion to one value per entry on the device (vspmm_expand_vcs), bit
for bit against the oracle's expand_vcs_format: the CSR or CSC of A from
either layout, index-sorted or in stored order, on the 60,000 x 2,000 count
matrix, on a ragged matrix with runs of empty groups and empty slices, on a
hand-worked matrix with repeated indices, and on an empty matrix."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import need_gpu, to_dev, vcs_handle, with_empty_groups

pytestmark = pytest.mark.gpu

CASES = [(fmt, sort) for fmt in ("csr", "csc") for sort in (True, False)]


@pytest.fixture(scope="module")
def count60k():
    t = W.count_60k()
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


def check(orc, L, A, fmt, sort, ws=None):
    ptr, idx, val = A.expand(fmt, sort, workspace=ws)
    want = orc.expand_vcs_format(L.layout, L.shape, L.major_ptr, L.values, L.value_ptr,
                                 L.indices, fmt, sort)
    assert np.array_equal(ptr.cpu().numpy(), want[0]), (L.layout, fmt, sort, "ptr")
    assert np.array_equal(idx.cpu().numpy(), want[1]), (L.layout, fmt, sort, "idx")
    got_v = val.cpu().numpy()
    assert np.array_equal(got_v.view(np.uint32), want[2].view(np.uint32)), (L.layout, fmt, sort)


@pytest.mark.parametrize("fmt,sort", CASES)
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_expand_60k(orc, count60k, layout, fmt, sort):
    dev = need_gpu()
    L = count60k[layout]
    check(orc, L, vcs_handle(L, dev), fmt, sort)


@pytest.mark.parametrize("fmt,sort", CASES)
def test_expand_ragged_empty_groups(orc, fmt, sort):
    """5,003 x 700, Poisson(8) rows (some empty), runs of 40 empty groups
    inserted into 12 slices of the VCSC."""
    dev = need_gpu()
    t = W.count_matrix(5_003, 700, 8.0, 30, W.rng_for(91))
    for L in (W.build_vcs(t, "vcsr"),
              with_empty_groups(W.build_vcs(t, "vcsc"), W.rng_for(92), n_rows=12, per_row=40)):
        check(orc, L, vcs_handle(L, dev), fmt, sort)


@pytest.mark.parametrize("fmt,sort", CASES)
def test_expand_repeated_indices(orc, fmt, sort):
    """Row 0 holds index 1 in two groups (values 2 and 3): sorted, the two keep
    their stored order."""
    dev = need_gpu()
    L = W.Vcs("vcsr", (2, 6), np.array([0, 2, 3], np.int32), np.array([2, 3, 7], np.float32),
              np.array([0, 2, 3, 5], np.int32), np.array([5, 1, 1, 4, 0], np.int32))
    check(orc, L, vcs_handle(L, dev), fmt, sort)


def test_expand_empty_and_errors(orc):
    dev = need_gpu()
    L = W.Vcs("vcsc", (4, 3), np.zeros(4, np.int32), np.zeros(0, np.float32),
              np.zeros(1, np.int32), np.zeros(0, np.int32))
    A = vcs_handle(L, dev)
    for fmt, sort in CASES:
        ptr, idx, val = A.expand(fmt, sort)
        assert ptr.cpu().tolist() == [0] * ((4 if fmt == "csr" else 3) + 1)
        assert idx.numel() == 0 and val.numel() == 0
    with pytest.raises(ValueError):
        A.expand("coo")


def test_expand_overwrites_a_built_schedule(orc, count60k):
    """A workspace that holds B @ VCSR's built schedule serves an expansion;
    the next deterministic product on it rebuilds and is still right."""
    dev = need_gpu()
    L = count60k["vcsr"]
    A = vcs_handle(L, dev)
    ws = A.workspace("BA")
    B = to_dev(W.dense_normal(np.random.default_rng(4), L.shape[0], 16), dev)
    first = A.spmm(B, "BA", mode="deterministic", workspace=ws).clone()
    check(orc, L, A, "csr", True, ws=ws)
    again = A.spmm(B, "BA", mode="deterministic", workspace=ws)
    assert torch.equal(again, first)


def _vcs_from_lengths(lengths, n, layout, seed):
    rng = np.random.default_rng(seed)
    rows, cols = W.sample_columns(rng, np.asarray(lengths), n)
    vals = rng.integers(1, 10, size=rows.size).astype(np.float32)
    return W.build_vcs(W.Triplets((len(lengths), n), rows, cols, vals), layout)


@pytest.mark.parametrize("case", ["long_mean", "short_mean_with_long"])
def test_expand_sorted_every_slice_path(orc, case):
    """The sorted expansion sorts a slice in LDS when it fits (up to 512 entries
    with 64-thread blocks, chosen when the mean slice holds at most 128, else
    up to 2,048 with 256 threads) and by a block radix sort otherwise: rows of
    0 to 3,000 entries (mean ~1,500), and Poisson(40) rows with 20 rows of 600
    to 2,000 entries, cover all four."""
    dev = need_gpu()
    rng = np.random.default_rng(5)
    if case == "long_mean":
        lengths = rng.integers(0, 3_001, size=300)
    else:
        lengths = rng.poisson(40, size=3_000)
        lengths[rng.choice(3_000, 20, replace=False)] = rng.integers(600, 2_001, size=20)
    L = _vcs_from_lengths(lengths, 4_000, "vcsr", seed=len(lengths))
    check(orc, L, vcs_handle(L, dev), "csr", True)
