"""A dense operand with 2^24 rows or more. The short VCS walk addresses B with
32-bit byte offsets built from 24-bit multiplies, so the plan gives such a B
to the plain walk (k_aligned) instead; the same holds for the deterministic
pass over the opposite layout when its B is that tall. A 3,000 x (2^24 + 7)
count matrix, Poisson(60) entries per row: every direction of both layouts,
atomic and deterministic, against the float64 oracle, at widths 1 and 3."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu

N_WIDE = 2**24 + 7


@pytest.fixture(scope="module")
def wide():
    t = W.count_matrix(3000, N_WIDE, 60.0, 64, W.rng_for(81))
    return {lay: W.build_vcs(t, lay) for lay in ("vcsr", "vcsc")}


@pytest.mark.parametrize("width", [1, 3])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_tall_b(orc, wide, layout, direction, width):
    dev = need_gpu()
    L = wide[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    aligned = (layout == "vcsr") == (direction == "AB")
    if aligned and rows >= 2**24:
        assert A.plan_info(width, direction)["kernel_name"] == "k_aligned"
    B = W.dense_normal(np.random.default_rng(width), rows, width)
    Bd = to_dev(B, dev)
    where = f"tall B {layout} {direction} w={width}"
    out = A.spmm(Bd, direction)
    check_close(orc, L, direction, B, out, where=where + " atomic")
    ws = A.workspace(direction, "deterministic", width)
    det = A.spmm(Bd, direction, mode="deterministic", workspace=ws)
    check_close(orc, L, direction, B, det, where=where + " deterministic")
    assert torch.equal(det.view(torch.int32),
                       A.spmm(Bd, direction, mode="deterministic", workspace=ws).view(torch.int32))
