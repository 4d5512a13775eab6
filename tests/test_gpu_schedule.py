"""Schedules (vspmm_schedule_*): the deterministic product's layout built once
and kept in memory the schedule owns (regridding page, section "API": the
exact transpose is kept once built; section "How it is built": a two-pass
counting sort). Checked here:

- a schedule's products equal vspmm_spmm_ex's deterministic products (which
  build their layout on every call) bit for bit, and the float64 oracle to the
  float tolerance: VCSR and VCSC in both directions (the opposite layout, and
  the tiled copy where it applies), CSR in float32, float64 and float32 values
  summed in float64, and an int64 CSR cut into several row blocks;
- the schedule does not depend on its build scratch: scratch overwritten or
  freed after the build changes nothing;
- its resident bytes: at most 1.2 times the compressed opposite layout (VCS
  regrouped by the other axis; CSR transposed), with no float per entry for a
  VCS;
- errors: a product at another width, scratch below the required size.
"""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, csr_handle, dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small():
    t = W.count_matrix(3000, 700, 40.0, 64, W.rng_for(11))
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


@pytest.fixture(scope="module")
def count60k():
    t = W.count_60k()
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


def _bits(t):
    return t.view(torch.int64 if t.dtype == torch.float64 else torch.int32)


def _compare(orc, L, A, direction, width, seed, where, np_t=np.float32, scratch=None):
    """Schedule product vs spmm_ex (deterministic) vs the oracle; returns the
    schedule."""
    dev = A.device
    rows, _ = dims(L, direction)
    B = W.dense_normal(np.random.default_rng(seed), rows, width, dtype=np_t)
    Bd = to_dev(B, dev)
    sc = A.schedule(direction, width, workspace=scratch)
    got = sc.spmm(Bd)
    ws = A.workspace(direction, "deterministic", width)
    ref = A.spmm(Bd, direction, mode="deterministic", workspace=ws)
    torch.cuda.synchronize()
    check_close(orc, L, direction, B, got, where=where)
    assert torch.equal(_bits(got), _bits(ref)), f"{where}: schedule != spmm_ex"
    again = sc.spmm(Bd)
    assert torch.equal(_bits(again), _bits(got)), f"{where}: repeat"
    return sc


@pytest.mark.parametrize("width", [1, 16, 37])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_vcs_schedule_equals_spmm_ex(orc, small, layout, direction, width):
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev)
    sc = _compare(orc, L, A, direction, width, width, f"{layout} {direction} w={width}")
    aligned = (layout == "vcsr") == (direction == "AB")
    info = A.plan_info(width, direction, "deterministic")
    if aligned and not info["tiles"]:
        assert sc.nbytes == 0  # the plain walk over the handle's own layout
    else:
        assert sc.nbytes > 0


@pytest.mark.parametrize("width", [4, 16, 32])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_tiled_schedule_equals_spmm_ex(orc, count60k, layout, width):
    """B @ A over the 60,000 x 2,000 count matrix: LDS tiles at widths 4 and
    16, L2 tiles at 32."""
    dev = need_gpu()
    L = count60k[layout]
    A = vcs_handle(L, dev)
    assert A.plan_info(width, "BA", "deterministic")["tiles"] > 1
    _compare(orc, L, A, "BA", width, 100 + width, f"tiled {layout} w={width}")


def test_resident_bytes(orc, count60k):
    """The misaligned VCSC direction at a width whose B fits LDS whole (no
    tiles): the schedule holds the regrouped VCSR (pointers, the realized
    groups, indices) plus the walk's per-slice starts and per-wave plan,
    within 1.2x the regrouped layout's own bytes."""
    dev = need_gpu()
    L = count60k["vcsc"]
    A = vcs_handle(L, dev)
    assert A.plan_info(8, "AB", "deterministic")["tiles"] == 0
    sc = _compare(orc, L, A, "AB", 8, 5, "vcsc AB w=8")
    opp = A.regroup()
    assert 0 < sc.nbytes <= 1.2 * opp.footprint()[0], (sc.nbytes, opp.footprint())


@pytest.mark.parametrize("dt", ["f32", "f64", "f32_f64"])
def test_csr_schedule(orc, dt):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    np_val = np.float64 if dt == "f64" else np.float32
    C = W.config4(np_val)[1]
    A = csr_handle(C, dev, dtype=torch.float64 if dt != "f32" else None)
    np_t = np.float32 if dt == "f32" else np.float64
    for width in (1, 8):
        sc = _compare(orc, C, A, "BA", width, width, f"csr {dt} BA w={width}", np_t=np_t)
        nnz = C.col.size
        e = 8 if dt == "f64" else 4
        assert sc.nbytes <= 1.2 * (4 * (C.shape[1] + 1) + (4 + e) * nnz) + 4096
    assert isinstance(sc, sdm.Schedule)


def test_int64_csr_schedule(orc):
    """Row blocks of at most 5,000 entries: one transpose per block in the
    schedule, block products added in block order."""
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    C = W.config4(np.float32)[1]
    A = sdm.CsrMatrix.from_arrays(C.shape, to_dev(C.row_ptr.astype(np.int64), dev),
                                  to_dev(C.col, dev), to_dev(C.val, dev), ptr64=True,
                                  block_nnz=5000)
    for width in (1, 16):
        _compare(orc, C, A, "BA", width, 7 + width, f"csr64 BA w={width}")
        _compare(orc, C, A, "AB", width, 9 + width, f"csr64 AB w={width}")


def test_scratch_is_not_kept(orc, small):
    """The schedule copies what it built out of the scratch: scratch written
    over and freed after the build leaves the products unchanged."""
    dev = need_gpu()
    L = small["vcsr"]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, "BA")
    B = W.dense_normal(np.random.default_rng(4), rows, 16)
    Bd = to_dev(B, dev)
    scratch = A.workspace("BA", "deterministic", 16)
    sc = A.schedule("BA", 16, workspace=scratch)
    first = sc.spmm(Bd).clone()
    scratch.fill_(0x5A)
    torch.cuda.synchronize()
    del scratch
    junk = torch.full((1 << 22,), -1, dtype=torch.int32, device=dev)  # takes the freed memory
    out = sc.spmm(Bd)
    torch.cuda.synchronize()
    check_close(orc, L, "BA", B, out, where="after scratch reuse")
    assert torch.equal(_bits(out), _bits(first))
    del junk


def test_schedule_errors(small):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    L = small["vcsr"]
    A = vcs_handle(L, dev)
    sc = A.schedule("BA", 16)
    rows, _ = dims(L, "BA")
    with pytest.raises(sdm.VspmmError):  # another width
        sc.spmm(torch.zeros((rows, 8), dtype=torch.float32, device=dev))
    need = A.workspace_size("BA", "deterministic", 16)
    tiny = torch.empty(need // 2, dtype=torch.uint8, device=dev)
    with pytest.raises(sdm.VspmmError):
        A.schedule("BA", 16, workspace=tiny)
    # an empty matrix: nothing to hold, products are zeros
    Z = W.build_vcs(W.Triplets((5, 4), np.zeros(0, np.int64), np.zeros(0, np.int64),
                               np.zeros(0, np.float32)), "vcsr")
    AZ = vcs_handle(Z, dev)
    sz = AZ.schedule("BA", 3)
    assert sz.nbytes == 0
    out = sz.spmm(torch.ones((5, 3), dtype=torch.float32, device=dev))
    assert torch.count_nonzero(out).item() == 0
