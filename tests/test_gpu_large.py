"""The large count matrix: 1,000,000 x 20,000, ~200M entries, values
min(1 + Geometric(0.3), 255), at widths 8 and 32, all four directions.

The VCSR comes from the generator (built in parallel row chunks). The VCSC is
the same matrix regrouped on the device by the library itself. The expected
values come from the float64 oracle run on the generator's VCSR (the same
matrix, so one oracle call serves A@B from either layout, and another serves
B@A), output by output on sampled rows. The device footprint is checked against
the expanded CSR of the same matrix.
"""

import os
import sys
import time

import numpy as np
import pytest
import torch

import workloads as W
from helpers import check_close, need_gpu, to_dev, vcs_handle

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_SAMPLE = 300


def log(msg):
    print(f"[large] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def large():
    dev = need_gpu()
    t0 = time.time()
    workers = max(1, min(16, os.cpu_count() or 1))
    L = W.config5_vcsr(workers=workers)
    log(f"VCSR built on the host: {L.nnz} entries, {L.n_groups} groups, {time.time() - t0:.1f} s")
    A = vcs_handle(L, dev)
    C = A.regroup()  # the VCSC of the same matrix, built on the device
    torch.cuda.synchronize()
    log(f"VCSC regrouped on the device: {C.values.numel()} groups, {time.time() - t0:.1f} s")
    rng = np.random.default_rng(55)
    m, n = L.shape
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, N_SAMPLE, replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, N_SAMPLE, replace=False)]))
    return {"L": L, "vcsr": A, "vcsc": C, "dev": dev, "want": {"AB": rows, "BA": cols}}


def test_large_footprint(large):
    L = large["L"]
    for lay in ("vcsr", "vcsc"):
        h = large[lay]
        dev_bytes, expanded = h.footprint()
        ratio = dev_bytes / expanded
        log(f"{lay}: {dev_bytes / 1e9:.3f} GB on the device vs {expanded / 1e9:.3f} GB expanded "
            f"({ratio:.3f})")
        assert h.indices.numel() == L.nnz
        # value groups shrink the structure well below one float per entry
        assert 0.45 < ratio < 0.65, (lay, ratio)


@pytest.mark.parametrize("width", [8, 32])
@pytest.mark.parametrize("layout,direction", [("vcsr", "AB"), ("vcsr", "BA"), ("vcsc", "AB"),
                                              ("vcsc", "BA")])
def test_large_parity(orc, large, layout, direction, width):
    L, dev = large["L"], large["dev"]
    A = large[layout]
    want = large["want"][direction]
    rows_in = L.shape[1] if direction == "AB" else L.shape[0]
    B = W.dense_normal(np.random.default_rng(width), rows_in, width)
    Bd = to_dev(B, dev)
    aligned = (layout == "vcsr") == (direction == "AB")
    modes = ["atomic"] if aligned else ["deterministic"] + (["atomic"] if width == 8 else [])
    for mode in modes:
        t0 = time.time()
        ws = A.workspace(direction, mode) if mode == "deterministic" else None
        out = A.spmm(Bd, direction, mode=mode, workspace=ws)
        torch.cuda.synchronize()
        got = out[torch.from_numpy(want).to(dev)].cpu().numpy()
        rel = check_close(orc, L, direction, B, got, want=want,
                          where=f"large {layout} {direction} w={width} {mode}")
        log(f"{layout} {direction} w={width} {mode}: max rel error {rel:.2e} "
            f"({time.time() - t0:.1f} s)")
        if aligned or mode == "deterministic":
            again = A.spmm(Bd, direction, mode=mode, workspace=ws)
            assert torch.equal(again.view(torch.int32), out.view(torch.int32))
        del out, ws


def test_large_integer_exact(orc, large):
    """Integer data: every partial sum is an integer below 2^24, so every
    direction, atomics included, must equal the oracle exactly."""
    L, dev = large["L"], large["dev"]
    for layout, direction, mode in [("vcsr", "AB", "atomic"), ("vcsr", "BA", "atomic"),
                                    ("vcsc", "AB", "atomic"), ("vcsc", "BA", "atomic"),
                                    ("vcsr", "BA", "deterministic")]:
        A = large[layout]
        want = large["want"][direction]
        rows_in = L.shape[1] if direction == "AB" else L.shape[0]
        B = W.dense_int(np.random.default_rng(3), rows_in, 8)
        ws = A.workspace(direction, mode) if mode == "deterministic" else None
        out = A.spmm(to_dev(B, dev), direction, mode=mode, workspace=ws)
        got = out[torch.from_numpy(want).to(dev)].cpu().numpy().astype(np.float64)
        ref = orc.spmm(L, direction, B, want=want)[want]
        assert np.array_equal(got, ref), (layout, direction, mode)
        del out, ws


@pytest.mark.parametrize("width", [8, 16, 32])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_large_tiled(orc, large, layout, width):
    """B @ A on the tiled schedule: B (1,000,000 rows, 32 / 64 / 128 MB) is cut
    into tiles: at width 8 into 248 LDS tiles (~5M virtual slices of ~40
    entries, their partial rows within half the matrix's bytes); at widths 16
    and 32, where LDS tiles' partial rows would outweigh that, into L2 tiles of
    ~2 MB (32 and 64), one XCD's worth of blocks per tile."""
    L, dev = large["L"], large["dev"]
    A = large[layout]
    want = large["want"]["BA"]
    info = A.plan_info(width, "BA", "deterministic")
    assert info["tiles"] > 8 and info["kernel_name"] == ("k_vcs_seg" if width <= 16 else "k_vcs_rows")
    B = W.dense_normal(np.random.default_rng(81), L.shape[0], width)
    Bd = to_dev(B, dev)
    t0 = time.time()
    ws = A.workspace("BA", "deterministic", width)
    out = A.spmm(Bd, "BA", mode="deterministic", workspace=ws)
    torch.cuda.synchronize()
    got = out[torch.from_numpy(want).to(dev)].cpu().numpy()
    rel = check_close(orc, L, "BA", B, got, want=want, where=f"large tiled {layout}")
    log(f"tiled {layout} B@A w={width} ({info['tiles']} tiles): max rel error {rel:.2e} "
        f"({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    t1 = time.time()
    again = A.spmm(Bd, "BA", mode="deterministic", workspace=ws)
    torch.cuda.synchronize()
    log(f"tiled {layout} B@A w={width}: {1e3 * (time.time() - t1):.2f} ms for a product on the built schedule")
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))
    del out, again, ws
