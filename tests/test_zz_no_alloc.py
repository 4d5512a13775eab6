"""vspmm_spmm_noalloc: vspmm_spmm_ex with the library's own per-device
workspace array instead of a workspace argument, for callers that cannot
allocate. Called through the C ABI (ctypes) and compared with vspmm_spmm_ex
given a fresh workspace, bit for bit: deterministic products over a VCS
(the tiled copy and the opposite layout), a float64 CSR and an int64 CSR of
several row blocks, and atomic products on integer data (exact in any order);
each case is two calls in a row, the second with a smaller input, so the
second call runs over what the first left in the array. A product whose
workspace exceeds the array is refused with VSPMM_ERR_WORKSPACE."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, csr_handle, dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu

ERR_WORKSPACE = 5
LIMIT = 64 << 20  # VSPMM_NOALLOC_WS_BYTES


def _noalloc(A, B, out, direction, mode):
    import sparse_dense_matmul_amd as sdm
    st = sdm.lib.vspmm_spmm_noalloc(A.handle, ctypes.c_void_p(B.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), B.shape[1],
                                    sdm.DIRECTIONS[direction], sdm.MODES[mode],
                                    sdm._stream(A.device))
    return st


def _ex(A, B, out, direction, mode):
    import sparse_dense_matmul_amd as sdm
    size = A.workspace_size(direction, mode, B.shape[1])
    ws = torch.empty(max(size, 1), dtype=torch.uint8, device=A.device)
    ws.fill_(0x77)
    st = sdm.lib.vspmm_spmm_ex(A.handle, ctypes.c_void_p(B.data_ptr()),
                               ctypes.c_void_p(out.data_ptr()), B.shape[1],
                               sdm.DIRECTIONS[direction], sdm.MODES[mode],
                               ctypes.c_void_p(ws.data_ptr()), size, sdm._stream(A.device))
    torch.cuda.synchronize()
    return st


def _bits(t):
    return t.view(torch.int64 if t.dtype == torch.float64 else torch.int32)


def _pair(orc, L, A, direction, mode, width, seed, integer=False, np_t=np.float32):
    dev = A.device
    rows, n_out = dims(L, direction)
    B = (W.dense_int(np.random.default_rng(seed), rows, width) if integer else
         W.dense_normal(np.random.default_rng(seed), rows, width, dtype=np_t))
    Bd = to_dev(B.astype(np_t), dev)
    got = torch.full((n_out, width), 3.0, dtype=Bd.dtype, device=dev)
    want = torch.empty_like(got)
    assert A.workspace_size(direction, mode) <= LIMIT
    assert _noalloc(A, Bd, got, direction, mode) == 0
    torch.cuda.synchronize()
    assert _ex(A, Bd, want, direction, mode) == 0
    where = f"{L.shape} {direction} {mode} w={width}"
    assert torch.equal(_bits(got), _bits(want)), where
    check_close(orc, L, direction, B.astype(np_t), got, where=where)


@pytest.mark.parametrize("layout,direction", [("vcsr", "BA"), ("vcsc", "AB"), ("vcsc", "BA"),
                                              ("vcsr", "AB")])
def test_vcs_deterministic_twice(orc, layout, direction):
    dev = need_gpu()
    big = W.build_vcs(W.count_matrix(3000, 700, 40.0, 64, W.rng_for(11)), layout)
    small = W.build_vcs(W.count_matrix(500, 300, 9.0, 16, W.rng_for(12)), layout)
    _pair(orc, big, vcs_handle(big, dev), direction, "deterministic", 16, 1)
    _pair(orc, small, vcs_handle(small, dev), direction, "deterministic", 5, 2)


def test_csr_f64_deterministic_twice(orc):
    dev = need_gpu()
    C = W.config4(np.float64)[1]
    A = csr_handle(C, dev)
    _pair(orc, C, A, "BA", "deterministic", 8, 3, np_t=np.float64)
    _, S = W.config1()
    S64 = W.Csr(S.shape, S.row_ptr, S.col, S.val.astype(np.float64))
    _pair(orc, S64, csr_handle(S64, dev), "BA", "deterministic", 3, 4, np_t=np.float64)


def test_int64_csr_deterministic_twice(orc):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    C = W.config4(np.float32)[1]

    def h64(C, block):
        return sdm.CsrMatrix.from_arrays(C.shape, to_dev(C.row_ptr.astype(np.int64), dev),
                                         to_dev(C.col, dev), to_dev(C.val, dev), ptr64=True,
                                         block_nnz=block)
    _pair(orc, C, h64(C, 50_000), "BA", "deterministic", 4, 5)
    _, S = W.config1()
    _pair(orc, S, h64(S, 4_000), "BA", "deterministic", 2, 6)


@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_atomic_integer_twice(orc, layout):
    dev = need_gpu()
    big = W.build_vcs(W.count_matrix(3000, 700, 40.0, 64, W.rng_for(11)), layout)
    small = W.build_vcs(W.count_matrix(500, 300, 9.0, 16, W.rng_for(12)), layout)
    misaligned = "BA" if layout == "vcsr" else "AB"
    _pair(orc, big, vcs_handle(big, dev), misaligned, "atomic", 16, 7, integer=True)
    _pair(orc, small, vcs_handle(small, dev), misaligned, "atomic", 3, 8, integer=True)


def test_over_the_limit_is_refused():
    """The 60,000 x 2,000 count matrix (~6M entries): its deterministic B @ VCSR
    needs a workspace well past 64 MiB. The call returns VSPMM_ERR_WORKSPACE and
    leaves out as it was; the atomic product of the same matrix needs no
    workspace and runs."""
    dev = need_gpu()
    L = W.build_vcs(W.count_60k(), "vcsr")
    A = vcs_handle(L, dev)
    assert A.workspace_size("BA", "deterministic") > LIMIT
    m, n = L.shape
    B = torch.ones((m, 16), dtype=torch.float32, device=dev)
    out = torch.full((n, 16), 5.0, dtype=torch.float32, device=dev)
    assert _noalloc(A, B, out, "BA", "deterministic") == ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
    assert _noalloc(A, B, out, "BA", "atomic") == 0
    torch.cuda.synchronize()
    want = A.spmm(B, "BA")
    assert torch.allclose(out, want, rtol=1e-5, atol=1e-3)
