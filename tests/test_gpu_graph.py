"""Products captured in a HIP graph (torch.cuda.CUDAGraph over the library's
launches): a launch-bound caller can replay the hot path without per-call
launch overhead. The product path enqueues kernels only (outputs are cleared
by a fill kernel, never hipMemsetAsync; no host waits), so it captures. Each
graph is replayed several times with eager work and synchronizations between
the replays, and every replay is checked against an eager product of the same
inputs, bit for bit (atomic mode on integer data, where every sum is exact)."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import csr_handle, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def count60k():
    t = W.count_60k()
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


def replay_matches_eager(run, B, fresh, n_replays=3):
    """Capture run() (which reads B and writes its fixed output), then for each
    replay load new data into B, replay, and compare with an eager run."""
    dev = B.device
    run()  # warm-up outside the capture: builds schedules, sets kernel attributes
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out = run()
    torch.cuda.synchronize()
    for k in range(n_replays):
        B.copy_(fresh(k))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = run().clone()         # the same product, eager
        torch.cuda.synchronize()
        assert torch.equal(got, want), k


@pytest.mark.parametrize("layout,direction,mode", [("vcsr", "AB", "atomic"),
                                                   ("vcsc", "BA", "deterministic"),
                                                   ("vcsr", "BA", "deterministic"),
                                                   ("vcsr", "BA", "atomic")])
def test_vcs_graph(count60k, layout, direction, mode):
    """VCSR@B (aligned), the tiled B@VCSC and B@VCSR (deterministic, through a
    schedule built before the capture) and B@VCSR with float atomics (fill kernel, then
    the scatter), all at width 16."""
    dev = need_gpu()
    L = count60k[layout]
    A = vcs_handle(L, dev)
    m, n = L.shape
    rows, n_out = (n, m) if direction == "AB" else (m, n)
    integer = mode == "atomic" and direction == "BA"
    gen = (lambda k: W.dense_int(np.random.default_rng(k), rows, 16)) if integer else \
        (lambda k: W.dense_normal(np.random.default_rng(k), rows, 16))
    B = to_dev(gen(100), dev)
    out = torch.empty((n_out, 16), device=dev)
    if mode == "deterministic":
        sc = A.schedule(direction, 16)
        run = lambda: sc.spmm(B, out=out)
    else:
        run = lambda: A.spmm(B, direction, mode=mode, out=out)
    replay_matches_eager(run, B, lambda k: to_dev(gen(k), dev))


@pytest.mark.parametrize("width", [1, 32])
def test_csr_graph(width):
    """The regridding-shaped CSR operator, A @ x: the short walk with its long-row
    blocks in one launch."""
    dev = need_gpu()
    _, C = W.config4(np.float32)
    A = csr_handle(C, dev)
    m, n = C.shape
    gen = lambda k: W.dense_normal(np.random.default_rng(k), n, width)
    B = to_dev(gen(100), dev)
    out = torch.empty((m, width), device=dev)
    replay_matches_eager(lambda: A.spmm(B, "AB", out=out), B, lambda k: to_dev(gen(k), dev))
