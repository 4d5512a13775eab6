"""A regridder's operator on the GPU: its elements' weights assembled into
one CSR by the device counting sort (vspmm_assemble_csr) for every role of
the orthogonal axis, bit for bit against the oracle's two-pass counting
sort; products over it against the oracle, with each column of a batch
equal to the same column alone; and the per-entry scaled transpose
(vspmm_transpose_csr_scaled) bit for bit, sharing the exact transpose's
indices.

Elements: 80 (as many as the regridding page's tutorial resample has), each
a sparse matrix from 400 input cells to 500 output cells with a log-normal
number of weights (mean ~1,000, some elements empty), coordinates uniform
and repeated coordinates allowed, weights U(0, 1), in random order within
an element."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, need_gpu, to_dev

pytestmark = pytest.mark.gpu

ROLES = ["own", "shared", "summed", "sum_of"]
N_ELEM, N_OUT, N_IN = 80, 500, 400


def elements(seed, dtype):
    rng = np.random.default_rng(seed)
    sizes = np.rint(rng.lognormal(np.log(800.0), 0.8, N_ELEM)).astype(np.int64)
    sizes[rng.choice(N_ELEM, 4, replace=False)] = 0
    elem_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    nnz = int(elem_ptr[-1])
    out_idx = rng.integers(0, N_OUT, nnz).astype(np.int32)
    in_idx = rng.integers(0, N_IN, nnz).astype(np.int32)
    weight = rng.random(nnz).astype(dtype)
    return elem_ptr, out_idx, in_idx, weight


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)


def assembled(orc, role, dtype, seed=1):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    ep, oi, ii, wt = elements(seed, dtype)
    A = sdm.assemble_csr(role, N_OUT, N_IN, to_dev(ep, dev), to_dev(oi, dev), to_dev(ii, dev),
                         to_dev(wt, dev))
    want = orc.assemble_csr(role, N_ELEM, N_OUT, N_IN, ep, oi, ii, wt)
    C = W.Csr(orc.assembled_shape(role, N_ELEM, N_OUT, N_IN), *want)
    return A, C


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("role", ROLES)
def test_assembly_bitwise(orc, role, dtype):
    A, C = assembled(orc, role, dtype)
    assert A.shape == C.shape
    assert np.array_equal(A.row_ptr.cpu().numpy(), C.row_ptr)
    assert np.array_equal(A.col.cpu().numpy(), C.col)
    assert np.array_equal(_bits(A.val.cpu().numpy()), _bits(C.val))


@pytest.mark.parametrize("role", ROLES)
def test_products_and_batch_equals_solo(orc, role):
    """A @ x and x @ A (atomic and deterministic) against the oracle over the
    oracle's own assembly; a batch of 8 columns gives each column exactly
    what it gives alone (aligned walk, and deterministic x @ A)."""
    A, C = assembled(orc, role, np.float32, seed=2)
    dev = A.device
    m, n = C.shape
    for direction, rows in (("AB", n), ("BA", m)):
        B = W.dense_normal(np.random.default_rng(3), rows, 8)
        Bd = to_dev(B, dev)
        modes = ["atomic"] if direction == "AB" else ["atomic", "deterministic"]
        for mode in modes:
            sc = A.schedule(direction, 8) if mode == "deterministic" else None
            out = sc.spmm(Bd) if sc else A.spmm(Bd, direction)
            check_close(orc, C, direction, B, out, where=f"{role} {direction} {mode}")
            if direction == "AB" or mode == "deterministic":
                for k in (0, 5):
                    col = Bd[:, k:k + 1].contiguous()
                    solo = (A.schedule(direction, 1).spmm(col) if sc else
                            A.spmm(col, direction))
                    assert torch.equal(solo[:, 0], out[:, k]), (role, direction, mode, k)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_scaled_transpose_bitwise(orc, dtype):
    """Per-entry factors U(0.5, 2) (one per assembled entry): the scaled
    transpose equals the oracle's bit for bit, shares the exact transpose's
    row pointers and indices, and its products match the oracle."""
    A, C = assembled(orc, "shared", dtype, seed=4)
    dev = A.device
    f = np.random.default_rng(5).uniform(0.5, 2.0, C.nnz).astype(dtype)
    T = A.transpose_scaled(to_dev(f, dev))
    want = orc.transpose_csr_scaled(C.shape[1], C.row_ptr, C.col, C.val, f)
    assert np.array_equal(T.row_ptr.cpu().numpy(), want[0])
    assert np.array_equal(T.col.cpu().numpy(), want[1])
    assert np.array_equal(_bits(T.val.cpu().numpy()), _bits(want[2]))
    P = A.transpose()
    assert torch.equal(P.row_ptr, T.row_ptr) and torch.equal(P.col, T.col)
    Ct = W.Csr((C.shape[1], C.shape[0]), *want)
    x = W.dense_normal(np.random.default_rng(6), C.shape[0], 4, dtype=dtype)
    tol = 1e-5 if dtype == np.float32 else 1e-12
    check_close(orc, Ct, "AB", x, T.spmm(to_dev(x, dev), "AB"), tol=tol, where="scaled T @ x")


def test_empty_and_errors(orc):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    z = torch.zeros(0, dtype=torch.int32, device=dev)
    A = sdm.assemble_csr("own", 3, 2, torch.zeros(5, dtype=torch.int32, device=dev), z, z,
                         torch.zeros(0, dtype=torch.float32, device=dev))
    assert A.shape == (12, 8) and A.row_ptr.cpu().tolist() == [0] * 13
    with pytest.raises(ValueError):
        sdm.assemble_csr("diagonal", 3, 2, torch.zeros(2, dtype=torch.int32, device=dev), z, z,
                         torch.zeros(0, dtype=torch.float32, device=dev))
    assert sdm.lib.vspmm_assemble_csr(9, 1, 1, 1, 0, None, None, None, None, 0, None, None,
                                      None, None, 0, None) == 3  # VSPMM_ERR_ENUM
