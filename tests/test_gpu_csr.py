"""CSR products on the GPU against the float64 oracle: the 2,000 x 500
workload, the regridding-shaped operator in float32 and float64, its exact
transpose (bit for bit), batch-vs-solo bit identity for every entry split, and
the deterministic misaligned direction."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, csr_handle, dims, need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfg1():
    return W.config1()[1]


@pytest.fixture(scope="module")
def regrid32():
    return W.config4(np.float32)[1]


@pytest.fixture(scope="module")
def regrid64():
    return W.config4(np.float64)[1]


@pytest.mark.parametrize("width", [1, 2, 3, 8, 16, 33])
@pytest.mark.parametrize("direction", ["AB", "BA"])
def test_config1(orc, cfg1, direction, width):
    dev = need_gpu()
    A = csr_handle(cfg1, dev)
    rows, _ = dims(cfg1, direction)
    B = W.dense_normal(np.random.default_rng(width), rows, width)
    check_close(orc, cfg1, direction, B, A.spmm(to_dev(B, dev), direction),
                where=f"csr {direction} w={width}")


def test_config1_operators(orc, cfg1):
    """A @ B with B 500 x 8 and B @ A with B 8 x 2,000, plus SpMV both ways."""
    dev = need_gpu()
    A = csr_handle(cfg1, dev)
    rng = np.random.default_rng(1)
    B = W.dense_normal(rng, 500, 8)
    check_close(orc, cfg1, "AB", B, A @ to_dev(B, dev), where="A@B")
    Bl = W.dense_normal(rng, 8, 2000)  # the 8 x 2,000 left operand
    got = (to_dev(Bl, dev) @ A).t()
    check_close(orc, cfg1, "BA", np.ascontiguousarray(Bl.T), got, where="B@A")
    x = W.dense_normal(rng, 500, 1)[:, 0]
    check_close(orc, cfg1, "AB", x[:, None], (A @ to_dev(x, dev))[:, None], where="A@x")
    y = W.dense_normal(rng, 2000, 1)[:, 0]
    check_close(orc, cfg1, "BA", y[:, None], (to_dev(y, dev) @ A)[:, None], where="y@A")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("direction", ["AB", "BA"])
def test_regridding_operator(orc, regrid32, regrid64, dtype, direction):
    dev = need_gpu()
    C = regrid32 if dtype == "f32" else regrid64
    A = csr_handle(C, dev)
    rows, _ = dims(C, direction)
    np_t = np.float32 if dtype == "f32" else np.float64
    for width in (1, 32):
        B = W.dense_normal(np.random.default_rng(width), rows, width, dtype=np_t)
        out = A.spmm(to_dev(B, dev), direction)
        tol = 1e-5 if dtype == "f32" else 1e-13
        check_close(orc, C, direction, B, out, tol=tol, where=f"{dtype} {direction} w={width}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_transpose_equals_oracle_bitwise(orc, regrid32, regrid64, dtype):
    dev = need_gpu()
    C = regrid32 if dtype == "f32" else regrid64
    T = csr_handle(C, dev).transpose()
    tp, ti, tv = orc.transpose_csr(C.shape[1], C.row_ptr, C.col, C.val)
    assert np.array_equal(T.row_ptr.cpu().numpy(), tp)
    assert np.array_equal(T.col.cpu().numpy(), ti)
    assert np.array_equal(T.val.cpu().numpy().view(np.uint8), tv.view(np.uint8))
    # and back again
    TT = T.transpose()
    assert np.array_equal(TT.row_ptr.cpu().numpy(), C.row_ptr)
    assert np.array_equal(TT.col.cpu().numpy(), C.col)
    assert np.array_equal(TT.val.cpu().numpy().view(np.uint8), C.val.view(np.uint8))


@pytest.mark.parametrize("group", [0, 1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("which", ["forward", "transpose"])
def test_batch_equals_solo_bitwise(orc, regrid32, regrid64, which, dtype, group):
    """With the entry split taken from the matrix, each column of a batch of
    32 gets exactly the bits it gets alone (regridding page, section "How it is
    built"), for the forward operator and its exact transpose."""
    dev = need_gpu()
    C = regrid32 if dtype == "f32" else regrid64
    A = csr_handle(C, dev, force_group=group)
    if which == "transpose":
        A = A.transpose()
    np_t = np.float32 if dtype == "f32" else np.float64
    rows = A.shape[1]
    Bb = to_dev(W.dense_normal(np.random.default_rng(5), rows, 32, dtype=np_t), dev)
    batch = A.spmm(Bb, "AB")
    for c in (0, 1, 7, 16, 31):
        solo = A.spmm(Bb[:, c:c + 1].contiguous(), "AB")
        assert torch.equal(batch[:, c], solo[:, 0]), (which, dtype, group, c)
    if group == 0:
        info1, info32 = A.plan_info(1), A.plan_info(32)
        assert info1["entry_lanes"] == info32["entry_lanes"]


def test_group_size_follows_matrix(regrid32):
    """The entry split is the power of two at or below the mean entries per
    row, at most 64: ~55 -> 32 for the forward operator, ~3 -> 2 for its
    transpose (regridding page, section "How it is built")."""
    dev = need_gpu()
    A = csr_handle(regrid32, dev)
    assert A.plan_info(1)["entry_lanes"] == 32
    assert A.transpose().plan_info(1)["entry_lanes"] == 2


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_deterministic_misaligned(orc, regrid32, regrid64, dtype):
    dev = need_gpu()
    C = regrid32 if dtype == "f32" else regrid64
    A = csr_handle(C, dev)
    np_t = np.float32 if dtype == "f32" else np.float64
    B = W.dense_normal(np.random.default_rng(9), C.shape[0], 32, dtype=np_t)
    ws = A.workspace("BA")
    first = A.spmm(to_dev(B, dev), "BA", mode="deterministic", workspace=ws)
    tol = 1e-5 if dtype == "f32" else 1e-13
    check_close(orc, C, "BA", B, first, tol=tol, where=f"det BA {dtype}")
    first = first.clone()
    for _ in range(5):
        again = A.spmm(to_dev(B, dev), "BA", mode="deterministic", workspace=ws)
        assert torch.equal(again, first)


def test_integer_exact_atomics(orc, cfg1):
    dev = need_gpu()
    C = W.Csr(cfg1.shape, cfg1.row_ptr, cfg1.col, np.rint(cfg1.val * 8).astype(np.float32))
    A = csr_handle(C, dev)
    B = W.dense_int(np.random.default_rng(2), 2000, 9)
    out = A.spmm(to_dev(B, dev), "BA")
    assert np.array_equal(out.cpu().numpy().astype(np.float64), orc.spmm(C, "BA", B))


def test_csr_edge_cases():
    dev = need_gpu()
    C = W.Csr((3, 4), np.array([0, 0, 0, 0], np.int32), np.zeros(0, np.int32),
              np.zeros(0, np.float64))
    A = csr_handle(C, dev)
    out = torch.full((3, 2), 5.0, dtype=torch.float64, device=dev)
    A.spmm(torch.ones((4, 2), dtype=torch.float64, device=dev), out=out)
    assert not out.any()
    T = A.transpose()
    assert T.row_ptr.cpu().tolist() == [0, 0, 0, 0, 0]


def heavy_tail(dtype, rng):
    """4,541 x 50,000: Poisson(20) rows, 60 rows of 2,000-6,000 entries, and
    one row of every length from 60 to 1,600 in random places. The long-row
    bound (one wave's share of the entries, at least 64, at most one round of
    the short walk) lies in that range on any device, so rows at it and one
    past it are walked, long rows sit between short ones in a wave's range,
    and rows past one round (1,536 float32 / 768 float64 entries) are there
    too."""
    m, n = 4_541, 50_000
    lengths = rng.poisson(20, size=m)
    picked = rng.permutation(m)
    lengths[picked[:60]] = rng.integers(2_000, 6_000, size=60)
    lengths[picked[60:60 + 1_541]] = np.arange(60, 1_601)
    rows, cols = W.sample_columns(rng, lengths, n)
    vals = rng.random(rows.size).astype(dtype)
    return W.build_csr(W.Triplets((m, n), rows, cols, vals))


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_long_rows_split(orc, dtype):
    """Rows longer than the long-row bound go to the long walk over the
    handle's list of long rows, the others to the short walk over
    entry-balanced row ranges: parity at widths 1, 8, 32, batch columns equal
    to solo products bit for bit, and repeats bit for bit."""
    dev = need_gpu()
    np_t = np.float32 if dtype == "f32" else np.float64
    C = heavy_tail(np_t, np.random.default_rng(61))
    A = csr_handle(C, dev)
    for width in (1, 8, 32):
        B = W.dense_normal(np.random.default_rng(width), C.shape[1], width, dtype=np_t)
        out = A.spmm(to_dev(B, dev), "AB")
        tol = 1e-12 if dtype == "f64" else 1e-5
        check_close(orc, C, "AB", B, out, tol=tol, where=f"long rows {dtype} w={width}")
        again = A.spmm(to_dev(B, dev), "AB")
        assert torch.equal(again, out)
    Bb = to_dev(W.dense_normal(np.random.default_rng(5), C.shape[1], 32, dtype=np_t), dev)
    batch = A.spmm(Bb, "AB")
    for c in (0, 5, 31):
        solo = A.spmm(Bb[:, c:c + 1].contiguous(), "AB")
        assert torch.equal(batch[:, c], solo[:, 0]), (dtype, c)


def test_long_rows_on_two_streams(regrid32):
    """Products over a handle with long rows (two launches per product: the
    short walk, then the long-row walk) on two streams at once, each followed
    on its own stream by a copy of the output, equal the same products run one
    at a time, bit for bit."""
    dev = need_gpu()
    A = csr_handle(regrid32, dev)
    n = regrid32.shape[1]
    Bs = [to_dev(W.dense_normal(np.random.default_rng(70 + k), n, w), dev)
          for k, w in enumerate((1, 32, 8, 32))]
    want = [A.spmm(B, "AB").clone() for B in Bs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    got = []
    for k, B in enumerate(Bs):
        st = streams[k % 2]
        st.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(st):
            out = torch.empty((regrid32.shape[0], B.shape[1]), device=dev)
            A.spmm(B, "AB", out=out)
            got.append(out.clone())  # runs on st after the join
    torch.cuda.synchronize()
    for k in range(len(Bs)):
        assert torch.equal(got[k], want[k]), k


def _csr_from_lengths(lengths, n, dtype, seed):
    rng = np.random.default_rng(seed)
    rows, cols = W.sample_columns(rng, np.asarray(lengths), n)
    vals = rng.random(rows.size).astype(dtype)
    return W.build_csr(W.Triplets((len(lengths), n), rows, cols, vals))


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("case", ["few_rows", "all_long", "one_row", "empty_runs"])
def test_row_ranges_and_long_rows(orc, dtype, case):
    """Entry-balanced row ranges and the long-row bound on shapes far from the
    workloads: fewer rows than waves (most ranges empty), every row long, a
    single non-empty row, and runs of empty rows around long ones; widths 1, 8
    and 32, repeats bit for bit, and batch columns equal to solo products."""
    dev = need_gpu()
    np_t = np.float32 if dtype == "f32" else np.float64
    n = 5_000
    if case == "few_rows":
        lengths = [3, 700, 0, 90, 2_500]
    elif case == "all_long":
        lengths = [900 + 37 * k for k in range(40)]
    elif case == "one_row":
        lengths = [0] * 300 + [1_800] + [0] * 300
    else:
        lengths = ([0] * 50 + [1_200] + [0] * 50 + [5] * 200) * 4
    C = _csr_from_lengths(lengths, n, np_t, seed=len(lengths))
    A = csr_handle(C, dev)
    tol = 1e-5 if dtype == "f32" else 1e-12
    for width in (1, 8, 32):
        B = W.dense_normal(np.random.default_rng(width), n, width, dtype=np_t)
        out = A.spmm(to_dev(B, dev), "AB")
        check_close(orc, C, "AB", B, out, tol=tol, where=f"{case} {dtype} w={width}")
        assert torch.equal(A.spmm(to_dev(B, dev), "AB"), out)
    Bb = to_dev(W.dense_normal(np.random.default_rng(3), n, 32, dtype=np_t), dev)
    batch = A.spmm(Bb, "AB")
    for c in (0, 13, 31):
        assert torch.equal(batch[:, c], A.spmm(Bb[:, c:c + 1].contiguous(), "AB")[:, 0]), (case, c)


@pytest.mark.parametrize("width", [1, 8, 32])
def test_float32_values_summed_in_float64(orc, regrid32, width):
    """float32 values with float64 operands and sums (regridding page, section
    "Why not cuSPARSE"): every value widens exactly, so each product equals,
    bit for bit, the float64 handle over the widened values (the same walks),
    and both match the oracle to float64 rounding. A@x, x@A atomic and
    deterministic; batch columns equal solo products; the transpose keeps
    float32 values."""
    dev = need_gpu()
    C = regrid32
    m, n = C.shape
    A = csr_handle(C, dev, dtype=torch.float64)
    assert A.dtype == torch.float64 and A.val.dtype == torch.float32
    C64 = W.Csr(C.shape, C.row_ptr, C.col, C.val.astype(np.float64))
    A64 = csr_handle(C64, dev)
    for direction in ("AB", "BA"):
        rows = n if direction == "AB" else m
        B = W.dense_normal(np.random.default_rng(width), rows, width, dtype=np.float64)
        Bd = to_dev(B, dev)
        modes = ["atomic"] if direction == "AB" else ["atomic", "deterministic"]
        for mode in modes:
            ws = A.workspace(direction, mode) if mode == "deterministic" else None
            ws64 = A64.workspace(direction, mode) if mode == "deterministic" else None
            out = A.spmm(Bd, direction, mode=mode, workspace=ws)
            assert out.dtype == torch.float64
            check_close(orc, C, direction, B, out, tol=1e-12, where=f"mixed {direction} {mode}")
            if direction == "AB" or mode == "deterministic":
                ref = A64.spmm(Bd, direction, mode=mode, workspace=ws64)
                assert torch.equal(out, ref), (direction, mode, width)
    if width == 32:
        Bb = to_dev(W.dense_normal(np.random.default_rng(5), n, 32, dtype=np.float64), dev)
        batch = A.spmm(Bb, "AB")
        for c in (0, 9, 31):
            assert torch.equal(batch[:, c], A.spmm(Bb[:, c:c + 1].contiguous(), "AB")[:, 0])
        T = A.transpose()
        assert T.val.dtype == torch.float32 and T.dtype == torch.float64
        want = orc.transpose_csr(n, C.row_ptr, C.col, C.val)
        assert np.array_equal(T.row_ptr.cpu().numpy(), want[0])
        assert np.array_equal(T.val.cpu().numpy().view(np.uint32), want[2].view(np.uint32))


@pytest.mark.parametrize("mean", [800, 1700, 3300, 7000, 13000])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_long_walk_waves_follow_mean_row(orc, mean, dtype):
    """Matrices whose mean row fills a round of the short walk go to the long
    walk with 1, 2, 4 or 8 waves per row (as many as the mean row fills passes
    of 1,536 / 768 entries): against the oracle at widths 1, 8 and 33 in both
    directions, with rows from a tenth to twice the mean and a few empty rows,
    and each batch column equal, bit for bit, to its solo product."""
    dev = need_gpu()
    rng = np.random.default_rng(mean)
    m, n = 96, 5000
    np_t = np.float32 if dtype == "f32" else np.float64
    lengths = rng.integers(mean // 10, 2 * mean, m)
    lengths[rng.choice(m, 5, replace=False)] = 0
    rows = np.repeat(np.arange(m), lengths)
    cols = rng.integers(0, n, rows.size).astype(np.int32)
    vals = rng.uniform(-1, 1, rows.size).astype(np_t)
    C = W.Csr((m, n), np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), cols, vals)
    A = csr_handle(C, dev)
    tol = 1e-5 if dtype == "f32" else 1e-13
    for direction in ("AB", "BA"):
        rows_in, _ = dims(C, direction)
        for width in (1, 8, 33):
            B = W.dense_normal(np.random.default_rng(width), rows_in, width, dtype=np_t)
            check_close(orc, C, direction, B, A.spmm(to_dev(B, dev), direction), tol=tol,
                        where=f"mean {mean} {dtype} {direction} w={width}")
    Bb = to_dev(W.dense_normal(np.random.default_rng(2), n, 8, dtype=np_t), dev)
    batch = A.spmm(Bb, "AB")
    for c in (0, 5):
        assert torch.equal(batch[:, c], A.spmm(Bb[:, c:c + 1].contiguous(), "AB")[:, 0])


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_deep_ring_rows_of_a_thousand(orc, dtype):
    """Rows of 500 to 1,500 entries over 1,000 columns: 64 entry lanes, a
    window per step, and B small enough to sit in LDS beside the eight-window
    ring at widths 1 to 16 (float32; float64 up to width 4, beyond which the
    two-window ring keeps B in LDS). Against the oracle in both directions and
    modes, repeats, and batch columns equal to solo products bit for bit."""
    dev = need_gpu()
    rng = np.random.default_rng(1000)
    m, n = 700, 1000
    np_t = np.float32 if dtype == "f32" else np.float64
    lengths = rng.integers(500, 1500, m)
    lengths[[3, 350]] = 0
    rows = np.repeat(np.arange(m), lengths)
    cols = rng.integers(0, n, rows.size).astype(np.int32)
    vals = rng.uniform(-1, 1, rows.size).astype(np_t)
    C = W.Csr((m, n), np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), cols, vals)
    A = csr_handle(C, dev)
    assert A.plan_info(1, "AB")["entry_lanes"] == 64
    tol = 1e-5 if dtype == "f32" else 1e-13
    for width in (1, 4, 8, 16):
        for direction in ("AB", "BA"):
            rows_in, _ = dims(C, direction)
            B = W.dense_normal(np.random.default_rng(width), rows_in, width, dtype=np_t)
            Bd = to_dev(B, dev)
            for mode in (["atomic"] if direction == "AB" else ["atomic", "deterministic"]):
                ws = A.workspace(direction, mode) if mode == "deterministic" else None
                out = A.spmm(Bd, direction, mode=mode, workspace=ws)
                check_close(orc, C, direction, B, out, tol=tol,
                            where=f"{dtype} {direction} {mode} w={width}")
                if direction == "AB" or mode == "deterministic":
                    assert torch.equal(out, A.spmm(Bd, direction, mode=mode, workspace=ws))
    Bb = to_dev(W.dense_normal(np.random.default_rng(9), n, 16, dtype=np_t), dev)
    batch = A.spmm(Bb, "AB")
    for c in (0, 7, 15):
        assert torch.equal(batch[:, c], A.spmm(Bb[:, c:c + 1].contiguous(), "AB")[:, 0])
