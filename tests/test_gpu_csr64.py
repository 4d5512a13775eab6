"""CSR with int64 row pointers and int32 column indices (regridding page,
section "Why not cuSPARSE": past 2^31 entries the row pointers must be int64,
while the column indices can stay int32). The library cuts the rows into
blocks of whole rows and walks each as an int32 CSR. Small block sizes drive
the blocked products against the float64 oracle at sizes it finishes in
seconds; one matrix of more than 2^31 entries, built on the device, is checked
against the oracle on sampled rows of A @ x and on every output of B @ A, in
float32 and with float32 values summed in float64."""

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


@pytest.mark.timeout(900)
def test_more_than_2_31_entries(orc):
    """2^21 rows of 1,025 entries: 2,149,580,800 entries, past int32. Column
    indices uniform on 4,096 columns and values U(0,1) drawn on the device
    (seeded); x and y U(0,1) in float32. Two instances over the same arrays:
    float32 values summed in float64, and float32 throughout. For each: A @ x
    on sampled rows (the first and last rows of each block, the row holding
    entry 2^31, and random rows) against the oracle row by row; B @ A (atomic,
    deterministic through vspmm_spmm_ex, and through a schedule) on every one
    of the 4,096 outputs against the oracle run over the host copy of the
    matrix in row chunks (each under 2^31 entries; their float64 sums added);
    the deterministic products repeat bit for bit and the schedule's equal
    spmm_ex's. Values and operands are nonnegative, so |A||B| = AB is the
    error scale."""
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
    x32 = torch.rand(n_cols, 1, generator=g, device=dev)
    y32 = torch.rand(n_rows, 1, generator=g, device=dev)
    got = {}
    for name, dt in (("f32 values, f64 sums", torch.float64), ("f32", torch.float32)):
        A = sdm.CsrMatrix.from_arrays((n_rows, n_cols), row_ptr, col, val, dtype=dt)
        x, y = x32.to(dt), y32.to(dt)
        Ax = A.spmm(x, "AB")
        yA_atomic = A.spmm(y, "BA")
        ws = A.workspace("BA", "deterministic", 1)
        yA = A.spmm(y, "BA", mode="deterministic", workspace=ws)
        assert torch.equal(yA, A.spmm(y, "BA", mode="deterministic", workspace=ws)), name
        del ws
        sc = A.schedule("BA", 1)
        assert torch.equal(sc.spmm(y), yA), name
        del sc
        got[name] = (Ax.cpu().numpy(), yA.cpu().numpy(), yA_atomic.cpu().numpy())
        del A, Ax, yA, yA_atomic
        torch.cuda.empty_cache()
    col_h, val_h = col.cpu().numpy(), val.cpu().numpy()
    xh, yh = x32.cpu().numpy(), y32.cpu().numpy()
    # rows per block of 2^30 entries: 1,047,552
    per = (2**30) // L
    sample = [0, 1, per - 1, per, per + 1, 2 * per - 1, 2 * per, (2**31) // L, n_rows - 1]
    sample += np.random.default_rng(7).integers(0, n_rows, 24).tolist()
    tols = {"f32 values, f64 sums": 1e-12, "f32": 1e-5}
    for r in sample:
        C1 = W.Csr((1, n_cols), np.array([0, L], dtype=np.int32), col_h[r * L:(r + 1) * L],
                   val_h[r * L:(r + 1) * L])
        for name, (Ax, _, _) in got.items():
            check_close(orc, C1, "AB", xh, Ax[r:r + 1], tol=tols[name], where=f"{name} row {r}")
    ref = np.zeros((n_cols, 1))
    rows_per = 2**18  # 268,697,600 entries per chunk
    for r0 in range(0, n_rows, rows_per):
        r1 = min(n_rows, r0 + rows_per)
        Cc = W.Csr((r1 - r0, n_cols), (np.arange(r1 - r0 + 1, dtype=np.int64) * L).astype(np.int32),
                   col_h[r0 * L:r1 * L], val_h[r0 * L:r1 * L])
        ref += orc.spmm(Cc, "BA", yh[r0:r1])
    for name, (_, yA, yA_atomic) in got.items():
        for mode, v in (("deterministic", yA), ("atomic", yA_atomic)):
            rel, zeros_ok = orc.max_rel_error(v, ref, ref)
            assert zeros_ok and rel <= tols[name], (name, mode, rel)
