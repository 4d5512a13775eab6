"""The C-ABI library loads on the CPU, exports every symbol include/vspmm.h
declares, and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "vspmm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vspmm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    import sparse_dense_matmul_amd as sdm
    declared = declared_symbols()
    assert len(declared) >= 13
    raw = ctypes.CDLL(sdm.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), f"{name} declared in vspmm.h but not exported"
    assert sorted(sdm.EXPORTS) == declared


def test_status_strings():
    import sparse_dense_matmul_amd as sdm
    for st in range(9):
        s = sdm.lib.vspmm_status_string(st).decode()
        assert s and s != "unknown status"
    assert sdm.lib.vspmm_status_string(99).decode() == "unknown status"


def test_host_argument_checks_without_device():
    """These checks run before any HIP call, so they hold on a CPU host."""
    import sparse_dense_matmul_amd as sdm
    L = sdm.lib
    h = ctypes.c_void_p()
    dummy = ctypes.c_void_p(0x1000)
    # null handle slot
    assert L.vspmm_create_vcs(None, 1, 2, 2, 1, 1, dummy, dummy, dummy, dummy, 0, 0, None) == 1
    # unknown layout / flag / dtype
    assert L.vspmm_create_vcs(ctypes.byref(h), 7, 2, 2, 1, 1, dummy, dummy, dummy, dummy, 0, 0,
                              None) == 3
    assert L.vspmm_create_vcs(ctypes.byref(h), 1, 2, 2, 1, 1, dummy, dummy, dummy, dummy, 64, 0,
                              None) == 3
    assert L.vspmm_create_csr(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 5, 0, 0, None) == 3
    # both split policies at once
    assert L.vspmm_create_csr(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 3, 0, None) == 3
    # negative or too large extents, bad forced group
    assert L.vspmm_create_vcs(ctypes.byref(h), 1, -1, 2, 1, 1, dummy, dummy, dummy, dummy, 0, 0,
                              None) == 2
    assert L.vspmm_create_csr(ctypes.byref(h), 2, 2**31, 1, dummy, dummy, dummy, 0, 0, 0,
                              None) == 2
    assert L.vspmm_create_csr(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 0, 3, None) == 2
    assert L.vspmm_create_csr(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 0, 128, None) == 2
    # int64 row pointers: nnz may pass int32 (here it reaches the null checks),
    # the extents may not; the block size is 0 or 1 .. 2^30
    C64 = L.vspmm_create_csr64
    assert C64(None, 2, 2, 1, dummy, dummy, dummy, 0, 0, 0, 0, None) == 1
    assert C64(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 5, 0, 0, 0, None) == 3
    assert C64(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 3, 0, 0, None) == 3
    assert C64(ctypes.byref(h), 2**31, 2, 1, dummy, dummy, dummy, 0, 0, 0, 0, None) == 2
    assert C64(ctypes.byref(h), 2, 2, -1, dummy, dummy, dummy, 0, 0, 0, 0, None) == 2
    assert C64(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 0, 0, -1, None) == 2
    assert C64(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 0, 0, 2**30 + 1, None) == 2
    assert C64(ctypes.byref(h), 2, 2, 1, dummy, dummy, dummy, 0, 0, 3, 0, None) == 2
    assert C64(ctypes.byref(h), 2, 2, 2**33, None, dummy, dummy, 0, 0, 0, 0, None) == 1
    assert C64(ctypes.byref(h), 2, 2, 2**33, dummy, None, dummy, 0, 0, 0, 0, None) == 1
    # missing arrays
    assert L.vspmm_create_vcs(ctypes.byref(h), 1, 2, 2, 1, 1, None, dummy, dummy, dummy, 0, 0,
                              None) == 1
    assert L.vspmm_create_csr(ctypes.byref(h), 2, 2, 1, dummy, None, dummy, 0, 0, 0, None) == 1
    # calls on a null handle
    assert L.vspmm_spmm(None, dummy, dummy, 4, 0, None) == 1
    assert L.vspmm_destroy(None) == 1
    n = ctypes.c_size_t()
    assert L.vspmm_workspace_size(None, 0, 0, ctypes.byref(n)) == 1
    assert h.value is None  # no handle was ever produced
