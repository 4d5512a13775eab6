"""Normalized views on the GPU (vspmm_set_view): the "scale" view, whose
stored entries (r, c, v) act as v * row_stat[r] * col_stat[c], against the
oracle's per-entry product, in every direction of VCSR, VCSC, CSR (float32,
float64, float32 values summed in float64) and an int64 CSR of several row
blocks; atomic and deterministic (spmm_ex, schedules, the no-alloc entry).
The identity view and unit statistics give the plain product bit for bit;
the transposed view is the view of the transpose; an unknown view, a missing
statistic and a product wider than the view's buffer are refused."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from helpers import TOL, csr_handle, dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small():
    t = W.count_matrix(3000, 700, 40.0, 64, W.rng_for(11))
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


def stats(shape, seed, dtype=np.float32):
    rng = np.random.default_rng(seed)
    m, n = shape
    return (rng.uniform(0.5, 2.0, m).astype(dtype), rng.uniform(0.5, 2.0, n).astype(dtype))


def check_view(orc, L, direction, B, got, r, c, tol=TOL, where=""):
    got = got.detach().cpu().numpy() if isinstance(got, torch.Tensor) else got
    ref = orc.spmm_view(L, direction, B, r, c)
    scale = orc.abs_scale_view(L, direction, B, r, c)
    rel, zeros_ok = orc.max_rel_error(got, ref, scale)
    assert zeros_ok, f"{where}: outputs with |G||B| = 0 are not exactly zero"
    assert rel <= tol, f"{where}: max relative error {rel:.3e} > {tol:g}"


def _bits(t):
    return t.view(torch.int64 if t.dtype == torch.float64 else torch.int32)


def _noalloc(A, B, out, direction, mode):
    import sparse_dense_matmul_amd as sdm
    return sdm.lib.vspmm_spmm_noalloc(A.handle, ctypes.c_void_p(B.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()), B.shape[1],
                                      sdm.DIRECTIONS[direction], sdm.MODES[mode],
                                      sdm._stream(A.device))


def _all_paths(orc, L, V, direction, width, r, c, seed, np_t=np.float32, tol=TOL, where=""):
    dev = V.device
    rows, n_out = dims(L, direction)
    B = W.dense_normal(np.random.default_rng(seed), rows, width, dtype=np_t)
    Bd = to_dev(B, dev)
    at = V.spmm(Bd, direction)
    check_view(orc, L, direction, B, at, r, c, tol, where + " atomic")
    ws = V.workspace(direction, "deterministic", width)
    det = V.spmm(Bd, direction, mode="deterministic", workspace=ws)
    check_view(orc, L, direction, B, det, r, c, tol, where + " deterministic")
    sc = V.schedule(direction, width)
    assert torch.equal(_bits(sc.spmm(Bd)), _bits(det)), where + " schedule"
    out = torch.empty_like(det)
    if V.workspace_size(direction, "deterministic") <= (64 << 20):
        assert _noalloc(V, Bd, out, direction, "deterministic") == 0
        torch.cuda.synchronize()
        if V.workspace_size(direction, "deterministic", width) <= (64 << 20):
            assert torch.equal(_bits(out), _bits(det)), where + " no-alloc"
        else:  # (the tiled copy does not fit the no-alloc array: the untiled walk)
            check_view(orc, L, direction, B, out, r, c, tol, where + " no-alloc")


@pytest.mark.parametrize("width", [1, 16, 37])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_vcs_scale_view(orc, small, layout, direction, width):
    dev = need_gpu()
    L = small[layout]
    r, c = stats(L.shape, width)
    V = vcs_handle(L, dev).normalized("scale", to_dev(r, dev), to_dev(c, dev))
    _all_paths(orc, L, V, direction, width, r, c, 100 + width,
               where=f"scale view {layout} {direction} w={width}")


@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_60k_scale_view(orc, layout, direction):
    """The 60,000 x 2,000 count matrix at width 16, the tiled copy included."""
    dev = need_gpu()
    L = W.build_vcs(W.count_60k(), layout)
    r, c = stats(L.shape, 5)
    V = vcs_handle(L, dev).normalized("scale", to_dev(r, dev), to_dev(c, dev), max_width=16)
    _all_paths(orc, L, V, direction, 16, r, c, 7, where=f"60k scale view {layout} {direction}")


@pytest.mark.parametrize("dt", ["f32", "f64", "f32_f64"])
def test_csr_scale_view(orc, dt):
    dev = need_gpu()
    np_val = np.float64 if dt == "f64" else np.float32
    np_t = np.float32 if dt == "f32" else np.float64
    C = W.config4(np_val)[1]
    A = csr_handle(C, dev, dtype=torch.float64 if dt != "f32" else None)
    r, c = stats(C.shape, 9, np_t)
    V = A.normalized("scale", to_dev(r, dev), to_dev(c, dev), max_width=8)
    tol = TOL if dt == "f32" else 1e-12
    for direction in ("AB", "BA"):
        for width in (1, 8):
            _all_paths(orc, C, V, direction, width, r, c, width, np_t=np_t, tol=tol,
                       where=f"csr {dt} {direction} w={width}")


def test_int64_csr_scale_view(orc):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    C = W.config4(np.float32)[1]
    A = sdm.CsrMatrix.from_arrays(C.shape, to_dev(C.row_ptr.astype(np.int64), dev),
                                  to_dev(C.col, dev), to_dev(C.val, dev), ptr64=True,
                                  block_nnz=5000)
    r, c = stats(C.shape, 13)
    V = A.normalized("scale", to_dev(r, dev), to_dev(c, dev), max_width=4)
    for direction in ("AB", "BA"):
        _all_paths(orc, C, V, direction, 4, r, c, 3, where=f"csr64 {direction}")


def test_identity_and_unit_statistics(small):
    """The identity view and the scale view with statistics of 1 give the
    plain product bit for bit (multiplying by 1 is exact)."""
    dev = need_gpu()
    for layout in ("vcsr", "vcsc"):
        L = small[layout]
        A = vcs_handle(L, dev)
        m, n = L.shape
        I = A.normalized("identity")
        U = A.normalized("scale", torch.ones(m, device=dev), torch.ones(n, device=dev))
        for direction in ("AB", "BA"):
            rows, _ = dims(L, direction)
            Bd = to_dev(W.dense_normal(np.random.default_rng(1), rows, 16), dev)
            want = A.spmm(Bd, direction, mode="deterministic",
                          workspace=A.workspace(direction, "deterministic", 16))
            for V in (I, U):
                got = V.spmm(Bd, direction, mode="deterministic",
                             workspace=V.workspace(direction, "deterministic", 16))
                assert torch.equal(_bits(got), _bits(want)), (layout, direction)


def test_transposed_view(small):
    """(V.T) @ x equals x @ V for a scale view V (the statistics change axes)."""
    dev = need_gpu()
    L = small["vcsr"]
    r, c = stats(L.shape, 21)
    V = vcs_handle(L, dev).normalized("scale", to_dev(r, dev), to_dev(c, dev))
    x = to_dev(W.dense_normal(np.random.default_rng(2), L.shape[0], 5), dev)
    want = V.spmm(x, "BA", mode="deterministic", workspace=V.workspace("BA", "deterministic", 5))
    T = V.T
    got = T.spmm(x, "AB", mode="deterministic", workspace=T.workspace("AB", "deterministic", 5))
    assert torch.equal(_bits(got), _bits(want))


def test_view_errors(small):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    L = small["vcsr"]
    A = vcs_handle(L, dev)
    m, n = L.shape
    with pytest.raises(ValueError):
        A.normalized("parafac2")
    assert sdm.lib.vspmm_set_view(A.handle, 7, None, None, 4) == 3  # VSPMM_ERR_ENUM
    assert sdm.lib.vspmm_set_view(A.handle, 1, None, None, 4) == 1  # VSPMM_ERR_NULL
    V = A.normalized("scale", torch.ones(m, device=dev), torch.ones(n, device=dev), max_width=4)
    with pytest.raises(sdm.VspmmError):  # wider than the view's buffer
        V.spmm(torch.ones((n, 5), device=dev), "AB")
