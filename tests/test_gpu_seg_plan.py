"""The short VCS walk (k_vcs_seg) gives a slice the same bits whichever wave
walks it and wherever that wave's run, rounds and windows start: every slot
adds its residue class of the slice's positions in stored order, and the slot
tree pairs the same residue classes whatever slot the slice starts at. So the
run plan (shares weighted by a wave's place on its SIMD, cut at slice starts)
changes the speed, never the result.

The check stacks 37 short slices, a matrix X and X again along the major axis.
The plan cuts the stacked matrix's runs elsewhere than X's, yet both copies'
output rows must equal X's product bit for bit; X's product is also checked
against the float64 oracle. VCSR@B over a 20,000 x 2,000 count matrix (B staged
in LDS) and B@VCSC over a 6,000 x 2,000 one (B gathered from L2), at widths 1,
8 and 16."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu


def stack_major(parts, layout):
    """The VCS whose major slices are those of `parts`, in order (one minor
    dimension shared by all)."""
    mp, vp = [np.zeros(1, np.int32)], [np.zeros(1, np.int32)]
    vals, idx = [], []
    g0 = e0 = n_major = 0
    for P in parts:
        mp.append(P.major_ptr[1:] + g0)
        vp.append(P.value_ptr[1:] + e0)
        vals.append(P.values)
        idx.append(P.indices)
        g0 += P.n_groups
        e0 += P.nnz
        n_major += P.major_ptr.size - 1
    n_minor = parts[0].shape[1] if layout == "vcsr" else parts[0].shape[0]
    shape = (n_major, n_minor) if layout == "vcsr" else (n_minor, n_major)
    return W.Vcs(layout, shape, np.concatenate(mp).astype(np.int32),
                 np.concatenate(vals).astype(np.float32), np.concatenate(vp).astype(np.int32),
                 np.concatenate(idx).astype(np.int32))


@pytest.fixture(scope="module")
def mats():
    rng = W.rng_for(83)
    out = {}
    xr = W.count_matrix(20000, 2000, 100.0, 64, rng)
    sr = W.count_matrix(37, 2000, 3.0, 64, rng)
    X, S = W.build_vcs(xr, "vcsr"), W.build_vcs(sr, "vcsr")
    out["vcsr"] = (X, S, stack_major([S, X, X], "vcsr"))
    xc = W.count_matrix(6000, 2000, 100.0, 64, rng)
    sc = W.count_matrix(6000, 37, 3.0, 64, rng)
    X, S = W.build_vcs(xc, "vcsc"), W.build_vcs(sc, "vcsc")
    out["vcsc"] = (X, S, stack_major([S, X, X], "vcsc"))
    return out


@pytest.mark.parametrize("width", [1, 8, 16])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_slice_bits_do_not_depend_on_the_plan(orc, mats, layout, width):
    dev = need_gpu()
    X, S, Y = mats[layout]
    direction = "AB" if layout == "vcsr" else "BA"
    hx, hy = vcs_handle(X, dev), vcs_handle(Y, dev)
    for h in (hx, hy):
        assert h.plan_info(width, direction)["kernel_name"] == "k_vcs_seg"
    rows, n_out = dims(X, direction)
    B = W.dense_normal(np.random.default_rng(width), rows, width)
    Bd = to_dev(B, dev)
    ox = hx.spmm(Bd, direction)
    oy = hy.spmm(Bd, direction)
    check_close(orc, X, direction, B, ox, where=f"{layout} {direction} w={width}")
    n0 = S.major_ptr.size - 1
    bits = ox.view(torch.int32)
    assert torch.equal(oy[n0:n0 + n_out].view(torch.int32), bits)
    assert torch.equal(oy[n0 + n_out:].view(torch.int32), bits)
