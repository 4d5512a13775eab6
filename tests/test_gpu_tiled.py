"""The tiled schedule of deterministic mode: B's rows cut into tiles, each
output row's entries split by tile and grouped by value per (tile, output
row), partial rows added in a fixed order. Tiles fit a CU's LDS for rows of up
to 64 bytes (staged there), and one XCD's L2 for wider rows (gathered from
global memory, the blocks of a tile on one XCD). Checked on the 60,000 x 2,000
count matrix in both directions whose dense input (60,000 rows) is too large
for LDS, at widths where LDS tiles apply (4, 8, 16), where L2 tiles apply (32,
64), and at width 1, where the fewest tiles would leave virtual slices too long
for the short walk and the tile count rises; on a matrix whose last tile is
short and holds runs of empty groups; across workspaces and widths sharing one workspace; and against
the float64 oracle, exactly on integer data."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, dims, need_gpu, to_dev, vcs_handle, with_empty_groups

pytestmark = pytest.mark.gpu

# (layout, direction) pairs whose input rows are the 60,000 matrix rows
LONG = [("vcsr", "BA"), ("vcsc", "BA")]


@pytest.fixture(scope="module")
def count60k():
    t = W.count_60k()
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


@pytest.fixture(scope="module")
def ragged():
    """50,003 x 1,500, Poisson(60) per row: the last of the tiles is short;
    runs of 70 empty groups inserted in some slices."""
    t = W.count_matrix(50_003, 1_500, 60.0, 255, W.rng_for(43))
    out = {lay: W.build_vcs(t, lay) for lay in ("vcsr", "vcsc")}
    out["vcsc_empty"] = with_empty_groups(out["vcsc"], W.rng_for(44), n_rows=10, per_row=70)
    return out


def run_det(A, L, direction, width, seed=0, ws=None, integer=False):
    dev = A.device
    rows, _ = dims(L, direction)
    B = (W.dense_int(np.random.default_rng(seed), rows, width) if integer else
         W.dense_normal(np.random.default_rng(seed), rows, width))
    if ws is None:
        ws = A.workspace(direction, "deterministic", width)
    out = A.spmm(to_dev(B, dev), direction, mode="deterministic", workspace=ws)
    return B, out, ws


@pytest.mark.parametrize("width", [4, 8, 16])
@pytest.mark.parametrize("layout,direction", LONG)
def test_tiled_parity(orc, count60k, layout, direction, width):
    dev = need_gpu()
    L = count60k[layout]
    A = vcs_handle(L, dev)
    info = A.plan_info(width, direction, "deterministic")
    assert info["tiles"] > 1 and info["kernel_name"] == "k_vcs_seg" and info["lds_staged"] == 1
    B, out, ws = run_det(A, L, direction, width)
    check_close(orc, L, direction, B, out, where=f"tiled {layout} {direction} w={width}")
    again = A.spmm(to_dev(B, dev), direction, mode="deterministic", workspace=ws)
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))
    # a second workspace builds the same schedule: the same bits
    _, other, _ = run_det(A, L, direction, width)
    assert torch.equal(other.view(torch.int32), out.view(torch.int32))


@pytest.mark.parametrize("width", [32, 64])
@pytest.mark.parametrize("layout,direction", LONG)
def test_l2_tiled_parity(orc, count60k, layout, direction, width):
    """Rows of 128 and 256 bytes: B (7.7 / 15.4 MB) cut into 8 tiles of about
    2 MB, one per XCD, gathered from L2 (no LDS staging); parity, repeats bit
    for bit, and a second workspace gives the same bits."""
    dev = need_gpu()
    L = count60k[layout]
    A = vcs_handle(L, dev)
    info = A.plan_info(width, direction, "deterministic")
    assert info["tiles"] == 8 and info["kernel_name"] == "k_vcs_rows" and info["lds_staged"] == 0
    B, out, ws = run_det(A, L, direction, width)
    check_close(orc, L, direction, B, out, where=f"L2 tiled {layout} {direction} w={width}")
    again = A.spmm(to_dev(B, dev), direction, mode="deterministic", workspace=ws)
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))
    _, other, _ = run_det(A, L, direction, width)
    assert torch.equal(other.view(torch.int32), out.view(torch.int32))


@pytest.mark.parametrize("width", [1])
@pytest.mark.parametrize("layout,direction", LONG)
def test_width1_tiles_follow_slice_length(orc, count60k, layout, direction, width):
    """Width 1: B (240 KB) would fit two tiles, leaving virtual slices of
    ~1,500 entries, beyond the short walk; the tile count rises to a multiple
    of 8 until the mean is at most 512 (8 tiles, ~375 entries). Parity and a
    bit-for-bit repeat."""
    dev = need_gpu()
    L = count60k[layout]
    A = vcs_handle(L, dev)
    info = A.plan_info(width, direction, "deterministic")
    assert info["tiles"] == 8 and info["kernel_name"] == "k_vcs_seg" and info["lds_staged"] == 1
    B, out, ws = run_det(A, L, direction, width)
    check_close(orc, L, direction, B, out, where=f"width 1 {layout} {direction}")
    again = A.spmm(to_dev(B, dev), direction, mode="deterministic", workspace=ws)
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))


@pytest.mark.parametrize("name,direction,width", [("vcsr", "BA", 16), ("vcsc", "BA", 8),
                                                  ("vcsc_empty", "BA", 8)])
def test_tiled_ragged(orc, ragged, name, direction, width):
    """(The VCSC, with fewer groups than the VCSR, takes tiles at width 8; at
    width 16 its tiles' partial rows would outweigh half the matrix.)"""
    dev = need_gpu()
    L = ragged[name]
    A = vcs_handle(L, dev)
    assert A.plan_info(width, direction, "deterministic")["tiles"] > 1
    for integer in (False, True):
        B, out, _ = run_det(A, L, direction, width, seed=5, integer=integer)
        if integer:
            want = orc.spmm(L, direction, B)
            assert np.array_equal(out.cpu().numpy().astype(np.float64), want), name
        else:
            check_close(orc, L, direction, B, out, where=f"ragged {name}")


@pytest.fixture(scope="module")
def tall():
    """50,000 x 20,000, Poisson(200) per row (~10M entries): at width 8 its
    B (640 KB) needs 5 LDS tiles, and 8 (a multiple of 8) would write more
    partial rows than half the matrix's bytes."""
    t = W.count_matrix(50_000, 20_000, 200.0, 64, W.rng_for(47))
    return {lay: W.build_vcs(t, lay) for lay in ("vcsr", "vcsc")}


@pytest.mark.parametrize("layout,direction", [("vcsr", "AB"), ("vcsc", "AB")])
def test_unrounded_tile_count(orc, tall, layout, direction):
    """The fewest LDS tiles as they are (5) when a multiple of 8 does not pay:
    VCSR@B (aligned) and VCSC@B (misaligned) at width 8, deterministic mode,
    against the float64 oracle, bit for bit on repeat and through a schedule,
    and exactly on integer data."""
    dev = need_gpu()
    L = tall[layout]
    A = vcs_handle(L, dev)
    info = A.plan_info(8, direction, "deterministic")
    assert info["tiles"] == 5 and info["kernel_name"] == "k_vcs_seg" and info["lds_staged"] == 1
    B, out, ws = run_det(A, L, direction, 8, seed=3)
    check_close(orc, L, direction, B, out, where=f"5 tiles {layout} {direction}")
    Bd = to_dev(B, dev)
    again = A.spmm(Bd, direction, mode="deterministic", workspace=ws)
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))
    assert torch.equal(A.schedule(direction, 8).spmm(Bd).view(torch.int32), out.view(torch.int32))
    Bi, outi, _ = run_det(A, L, direction, 8, seed=4, ws=ws, integer=True)
    assert np.array_equal(outi.cpu().numpy().astype(np.float64), orc.spmm(L, direction, Bi))


def test_workspace_shared_across_widths(orc, count60k):
    """One workspace large enough for every width, shared by products of
    widths 16, 8, 32 and 64 in turn (each call builds its tiled copy again in
    it): every width's result repeats bit for bit when it comes round again."""
    dev = need_gpu()
    L = count60k["vcsr"]
    A = vcs_handle(L, dev)
    n = max(A.workspace_size("BA", "deterministic", w) for w in (8, 16, 32, 64))
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    first = {}
    for width in (16, 8, 32, 64, 16, 8, 64, 32):
        B, out, _ = run_det(A, L, "BA", width, seed=width, ws=ws)
        if width in first:
            assert torch.equal(out.view(torch.int32), first[width].view(torch.int32))
        else:
            check_close(orc, L, "BA", B, out, where=f"shared ws w={width}")
            first[width] = out.clone()


def test_small_workspace_falls_back(orc, count60k):
    """A workspace sized without the width holds only the opposite layout: the
    misaligned product takes the untiled two-pass path, the aligned one the
    plain walk; both stay correct."""
    dev = need_gpu()
    for layout in ("vcsr", "vcsc"):
        L = count60k[layout]
        A = vcs_handle(L, dev)
        small = A.workspace("BA", "deterministic")
        assert small.numel() < A.workspace_size("BA", "deterministic", 16)
        B, out, _ = run_det(A, L, "BA", 16, ws=small)
        check_close(orc, L, "BA", B, out, where=f"fallback {layout}")
