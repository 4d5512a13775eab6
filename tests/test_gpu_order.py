"""Stored order. A value-grouped layout fixes which entries share a value, not
the order of the groups in a slice or of the indices in a group; every other
VCS test uses the generator's canonical order (ascending value, then
ascending index), where a builder that sorted by index instead of keeping
stored order would pass unnoticed. Here the 60,000 x 2,000 count matrix is
stored with its groups permuted within each slice and its indices permuted
within each group, and 300 entries repeated under a second value of their
slice (stored entries add). On integer data every sum is an exact integer,
so each product is compared with the float64 oracle exactly: all four
directions, atomic and deterministic (two-pass and tiled, through spmm_ex
and through a schedule); the regrouping and the expansions are compared with
the oracle bit for bit."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def shuffled():
    t = W.count_60k()
    return {lay: W.shuffled_vcs(W.build_vcs(t, lay), W.rng_for(71, i), n_dup=300)
            for i, lay in enumerate(("vcsr", "vcsc"))}


def _exact(orc, L, direction, B, got, where):
    ref = orc.spmm(L, direction, B)
    got = got.cpu().numpy().astype(np.float64)
    bad = np.flatnonzero((got != ref).any(axis=1))
    assert bad.size == 0, f"{where}: {bad.size} rows differ, first {bad[:5]}"


@pytest.mark.parametrize("width", [1, 16])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_shuffled_products_exact(orc, shuffled, layout, direction, width):
    dev = need_gpu()
    L = shuffled[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    B = W.dense_int(np.random.default_rng(width), rows, width)
    Bd = to_dev(B, dev)
    where = f"shuffled {layout} {direction} w={width}"
    _exact(orc, L, direction, B, A.spmm(Bd, direction), where + " atomic")
    ws = A.workspace(direction, "deterministic", width)
    det = A.spmm(Bd, direction, mode="deterministic", workspace=ws)
    tiles = A.plan_info(width, direction, "deterministic")["tiles"]
    _exact(orc, L, direction, B, det, where + f" deterministic ({tiles} tiles)")
    small = A.workspace(direction, "deterministic")  # no room for the tiled copy
    _exact(orc, L, direction, B,
           A.spmm(Bd, direction, mode="deterministic", workspace=small), where + " untiled")
    sc = A.schedule(direction, width)
    assert torch.equal(sc.spmm(Bd), det), where + " schedule"


@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_shuffled_regroup_bitwise(orc, shuffled, layout):
    dev = need_gpu()
    L = shuffled[layout]
    R = vcs_handle(L, dev).regroup()
    mp, v, vp, ix = orc.regroup_vcs(L.n_minor, L.major_ptr, L.values, L.value_ptr, L.indices)
    assert np.array_equal(R.major_ptr.cpu().numpy(), mp)
    assert np.array_equal(R.values.cpu().numpy().view(np.uint32), v.view(np.uint32))
    assert np.array_equal(R.value_ptr.cpu().numpy(), vp)
    assert np.array_equal(R.indices.cpu().numpy(), ix)


@pytest.mark.parametrize("fmt,sort", [("csr", True), ("csr", False), ("csc", True),
                                      ("csc", False)])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_shuffled_expand_bitwise(orc, shuffled, layout, fmt, sort):
    dev = need_gpu()
    L = shuffled[layout]
    ptr, idx, val = vcs_handle(L, dev).expand(fmt, sort)
    want = orc.expand_vcs_format(L.layout, L.shape, L.major_ptr, L.values, L.value_ptr,
                                 L.indices, fmt, sort)
    assert np.array_equal(ptr.cpu().numpy(), want[0])
    assert np.array_equal(idx.cpu().numpy(), want[1])
    assert np.array_equal(val.cpu().numpy().view(np.uint32), want[2].view(np.uint32))
