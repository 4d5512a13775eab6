"""CSR with int64 row pointers and int32 column indices (regridding page,
section "Why not cuSPARSE": past 2^31 entries the row pointers must be int64,
while the column indices can stay int32). The library cuts the rows into
blocks of whole rows and walks each as an int32 CSR. Small block sizes drive
the blocked products against the float64 oracle at sizes it finishes in
seconds; one matrix of more than 2^31 entries, built on the device, is checked
on sampled rows against the oracle and by the dot-product identity."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, csr_handle, dims, need_gpu, to_dev

pytestmark = pytest.mark.gpu


def h64(C, dev, **kw):
    import sparse_dense_matmul_amd as sdm
    return sdm.CsrMatrix.from_arrays(C.shape, to_dev(C.row_ptr.astype(np.int64), dev),
                                     to_dev(C.col, dev), to_dev(C.val, dev), ptr64=True, **kw)


@pytest.fixture(scope="module")
def regrid32():
    return W.config4(np.float32)[1]


@pytest.fixture(scope="module")
def regrid64():
    return W.config4(np.float64)[1]


def _all_products(orc, C, A, dev, tol, np_t, widths=(1, 8, 33), where=""):
    for direction in ("AB", "BA"):
        rows, _ = dims(C, direction)
        for width in widths:
            B = W.dense_normal(np.random.default_rng(width), rows, width, dtype=np_t)
            Bd = to_dev(B, dev)
            for mode in (["atomic"] if direction == "AB" else ["atomic", "deterministic"]):
                ws = A.workspace(direction, mode, width) if mode == "deterministic" else None
                out = A.spmm(Bd, direction, mode=mode, workspace=ws)
                check_close(orc, C, direction, B, out, tol=tol,
                            where=f"{where} {direction} {mode} w={width}")
                if direction == "AB" or mode == "deterministic":
                    again = A.spmm(Bd, direction, mode=mode, workspace=ws)
                    assert torch.equal(out, again), (where, direction, mode, width)


@pytest.mark.parametrize("block_nnz", [0, 5000, 100_000])
@pytest.mark.parametrize("dtype", ["f32", "f64", "mixed"])
def test_blocked_products(orc, regrid32, regrid64, dtype, block_nnz):
    """The regridding-shaped operator (20,000 rows, ~1.1M entries, heavy-tailed
    rows) in 1, ~11 or ~220 row blocks: every direction and mode against the
    oracle; aligned and deterministic products repeat bit for bit."""
    dev = need_gpu()
    C = regrid64 if dtype == "f64" else regrid32
    kw = {"dtype": torch.float64} if dtype == "mixed" else {}
    A = h64(C, dev, block_nnz=block_nnz, **kw)
    np_t = np.float32 if dtype == "f32" else np.float64
    _all_products(orc, C, A, dev, 1e-5 if dtype == "f32" else 1e-12, np_t,
                  where=f"{dtype} block_nnz={block_nnz}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_one_block_equals_int32_handle(regrid32, regrid64, dtype):
    """With one block the walk is the int32 handle's: equal bit for bit."""
    dev = need_gpu()
    C = regrid32 if dtype == "f32" else regrid64
    A64, A32 = h64(C, dev), csr_handle(C, dev)
    np_t = np.float32 if dtype == "f32" else np.float64
    for direction in ("AB", "BA"):
        rows, _ = dims(C, direction)
        Bd = to_dev(W.dense_normal(np.random.default_rng(3), rows, 16, dtype=np_t), dev)
        for mode in ("atomic", "deterministic"):
            if direction == "AB" and mode == "deterministic":
                continue
            w64 = A64.workspace(direction, mode, 16) if mode == "deterministic" else None
            w32 = A32.workspace(direction, mode, 16) if mode == "deterministic" else None
            got = A64.spmm(Bd, direction, mode=mode, workspace=w64)
            want = A32.spmm(Bd, direction, mode=mode, workspace=w32)
            if direction == "AB" or mode == "deterministic":
                assert torch.equal(got, want), (direction, mode)


def test_blocks_with_empty_and_long_rows(orc):
    """Block size 4 over rows of 0 .. 40 entries: empty blocks, blocks of
    several empty rows, and rows longer than the block size, which form blocks
    of their own; also a matrix with no entries at all."""
    dev = need_gpu()
    rng = np.random.default_rng(64)
    lengths = np.array([0, 5, 0, 0, 40, 1, 0, 3, 4, 4, 0, 2, 2, 0, 0, 9], dtype=np.int64)
    n_cols = 16
    rows = np.repeat(np.arange(lengths.size), lengths)
    cols = np.concatenate([rng.choice(n_cols, size=k, replace=True) for k in lengths if k])
    vals = rng.uniform(0, 1, size=rows.size)
    C = W.Csr((lengths.size, n_cols), np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32),
              cols.astype(np.int32), vals)
    for bn in (1, 4, 7):
        A = h64(C, dev, block_nnz=bn)
        _all_products(orc, C, A, dev, 1e-12, np.float64, widths=(1, 5), where=f"bn={bn}")
    Z = W.Csr((5, 3), np.zeros(6, np.int32), np.zeros(0, np.int32), np.zeros(0))
    A = h64(Z, dev, block_nnz=2)
    _all_products(orc, Z, A, dev, 0.0, np.float64, widths=(1, 2), where="empty")


def test_structure_and_workspace_errors(regrid32):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    C = regrid32
    col, val = to_dev(C.col, dev), to_dev(C.val, dev)
    rp = C.row_ptr.astype(np.int64)
    for bad in (rp + 1, np.concatenate([rp[:-1], [rp[-1] - 1]]),
                np.concatenate([rp[:5], rp[4:5] - 1, rp[6:]])):
        with pytest.raises(sdm.VspmmError):
            sdm.CsrMatrix.from_arrays(C.shape, to_dev(bad, dev), col, val, ptr64=True)
    A = h64(C, dev, block_nnz=5000)
    m, n = C.shape
    y = to_dev(W.dense_normal(np.random.default_rng(1), m, 4), dev)
    small = A.workspace("BA", "deterministic")  # without the block-sum buffer
    with pytest.raises(sdm.VspmmError):
        A.spmm(y, "BA", mode="deterministic", workspace=small)
    with pytest.raises(sdm.VspmmError):
        A.transpose()
    info = A.plan_info(16, "AB")
    assert info["entry_lanes"] >= 1


def test_more_than_2_31_entries(orc):
    """2^21 rows of 1,025 entries: 2,149,580,800 entries, past int32. Column
    indices uniform on 4,096 columns and values U(0,1) drawn on the device
    (seeded), float32 values summed in float64. A @ x on sampled rows (the
    first and last rows of each block, the row holding entry 2^31, and random
    rows) against the oracle row by row; B @ A (atomic and deterministic)
    through <A x, y> = <x, A^T y> and against each other; the deterministic
    product repeats bit for bit."""
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    n_rows, L, n_cols = 2**21, 1025, 4096
    nnz = n_rows * L
    assert nnz > 2**31 - 1
    g = torch.Generator(device=dev)
    g.manual_seed(20261202)
    col = torch.empty(nnz, dtype=torch.int32, device=dev)
    val = torch.empty(nnz, dtype=torch.float32, device=dev)
    chunk = 2**28
    for s in range(0, nnz, chunk):
        e = min(nnz, s + chunk)
        col[s:e] = torch.randint(0, n_cols, (e - s,), generator=g, device=dev, dtype=torch.int32)
        val[s:e] = torch.rand(e - s, generator=g, device=dev)
    row_ptr = torch.arange(n_rows + 1, dtype=torch.int64, device=dev) * L
    A = sdm.CsrMatrix.from_arrays((n_rows, n_cols), row_ptr, col, val, dtype=torch.float64)
    x = torch.rand(n_cols, 1, generator=g, device=dev, dtype=torch.float64)
    y = torch.rand(n_rows, 1, generator=g, device=dev, dtype=torch.float64)
    Ax = A.spmm(x, "AB")
    yA_atomic = A.spmm(y, "BA")
    ws = A.workspace("BA", "deterministic", 1)
    yA = A.spmm(y, "BA", mode="deterministic", workspace=ws)
    assert torch.equal(yA, A.spmm(y, "BA", mode="deterministic", workspace=ws))
    # rows per block of 2^30 entries: 1,047,552
    per = (2**30) // L
    sample = [0, 1, per - 1, per, per + 1, 2 * per - 1, 2 * per, (2**31) // L, n_rows - 1]
    sample += np.random.default_rng(7).integers(0, n_rows, 24).tolist()
    xh = x.cpu().numpy()
    got = Ax.cpu().numpy()
    for r in sample:
        C1 = W.Csr((1, n_cols), np.array([0, L], dtype=np.int32),
                   col[r * L:(r + 1) * L].cpu().numpy(), val[r * L:(r + 1) * L].cpu().numpy())
        check_close(orc, C1, "AB", xh, got[r:r + 1], tol=1e-12, where=f"row {r}")
    lhs = float((Ax * y).sum())
    for name, v in (("deterministic", yA), ("atomic", yA_atomic)):
        rhs = float((x * v).sum())
        assert abs(lhs - rhs) <= 1e-10 * abs(lhs), (name, lhs, rhs)
    assert torch.allclose(yA, yA_atomic, rtol=1e-12, atol=0)
