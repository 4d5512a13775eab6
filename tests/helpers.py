"""Shared test helpers: upload generator output to the device, build handles,
and judge float results against the oracle."""

import numpy as np
import pytest
import torch

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
