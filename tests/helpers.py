"""Shared test helpers: upload generator output to the device, build handles,
and judge float results against the oracle."""

import numpy as np
import pytest
import torch

import workloads as W
from conftest import gpu_required

TOL = 1e-5  # max |gpu - oracle| / (|A| |B|) on float32 results


def need_gpu():
    if torch.cuda.is_available():
        return torch.device("cuda:0")
    if gpu_required():
        pytest.fail("VSPMM_REQUIRE_GPU=1 but no GPU is visible")
    pytest.skip("no GPU")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def vcs_handle(L, dev, **kw):
    import sparse_dense_matmul_amd as sdm
    return sdm.VcsMatrix.from_arrays(L.layout, L.shape, to_dev(L.major_ptr, dev),
                                     to_dev(L.values, dev), to_dev(L.value_ptr, dev),
                                     to_dev(L.indices, dev), **kw)


def csr_handle(C, dev, **kw):
    import sparse_dense_matmul_amd as sdm
    return sdm.CsrMatrix.from_arrays(C.shape, to_dev(C.row_ptr, dev), to_dev(C.col, dev),
                                     to_dev(C.val, dev), **kw)


def handle(L, dev, **kw):
    return vcs_handle(L, dev, **kw) if hasattr(L, "major_ptr") else csr_handle(L, dev, **kw)


def dims(L, direction):
    m, n = L.shape
    return (n, m) if direction == "AB" else (m, n)  # (rows of the dense input, rows of out)


def check_close(orc, L, direction, B, got, want=None, tol=TOL, where=""):
    """got (torch or numpy, rows listed in `want` or all) against the oracle."""
    got = got.detach().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = orc.spmm(L, direction, B, want=want)
    scale = orc.abs_scale(L, direction, B, want=want)
    if want is not None:
        ref, scale = ref[want], scale[want]
        got = got[want] if got.shape[0] != len(want) else got
    assert got.shape == ref.shape, (got.shape, ref.shape, where)
    rel, zeros_ok = orc.max_rel_error(got, ref, scale)
    assert zeros_ok, f"{where}: outputs with |A||B| = 0 are not exactly zero"
    assert rel <= tol, f"{where}: max relative error {rel:.3e} > {tol:g}"
    return rel


def with_empty_groups(L, rng, n_rows=6, per_row=300):
    """The same matrix with runs of empty groups (value_ptr[k] == value_ptr[k+1])
    inserted at the start, middle and end of some slices: the product must not
    change."""
    mp, vals, vp = L.major_ptr.astype(np.int64), L.values.copy(), L.value_ptr.astype(np.int64)
    for r in sorted(rng.choice(L.n_major, size=n_rows, replace=False), reverse=True):
        g0, g1 = int(mp[r]), int(mp[r + 1])
        at = [g0, (g0 + g1) // 2, g1][r % 3]
        vals = np.insert(vals, at, np.float32(7.0) * np.ones(per_row, np.float32))
        vp = np.insert(vp, at, np.full(per_row, vp[at]))
        mp[r + 1:] += per_row
    return W.Vcs(L.layout, L.shape, mp.astype(np.int32), vals.astype(np.float32),
                 vp.astype(np.int32), L.indices)
