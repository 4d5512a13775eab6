"""Float64 CPU oracle (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``liboracle.so``, built from
``oracle.c`` with gcc, through ctypes. It shares no code with the HIP library
and never imports it; inputs come from the ``workloads`` generators or from
literals in the tests.

Every product here follows the plain definition: each stored entry (r, c, v)
adds ``v * B[c]`` to row ``r`` of ``A @ B`` and ``v * Bt[r]`` to row ``c`` of
``(B @ A)`` transposed (vsparse page, sections "The layout stays compressed"
and "The kernels"; regridding page, section "How it is built"). Float32 inputs
are widened to float64, which is exact.

Parity pins: the tests under ``tests/test_oracle_*.py`` tie each function to
something other than itself (brute-force dense products, scipy.sparse, closed
forms with all-ones operands, the dot-product identity, scipy's CSR->CSC
conversion and index sort, hand-worked examples, the generator's own
canonical layouts, the footprint ratios the vsparse page prints). No function
here is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

STATUS = {0: "ok", 1: "pointer array does not start at 0", 2: "pointer array decreases",
          3: "last pointer differs from the array length",
          4: "minor index out of range", 5: "negative extent"}


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (plain C11, -O2, no fast-math; OpenMP for
    the threaded timing mode)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-ffp-contract=off", "-fopenmp", "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load the oracle library (``ORACLE_LIB`` in the environment names another
    build of ``oracle.c``; the tests use it to plant mistakes in a copy)."""
    global _lib
    if path is None:
        path = os.environ.get("ORACLE_LIB", _LIB_PATH)
    if _lib is not None and path == _LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    i64, i32p, dp, vp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.orc_validate_csr.argtypes = [i64, i64, i64, i32p, i32p]
    lib.orc_validate_csr.restype = ctypes.c_int
    lib.orc_validate_vcs.argtypes = [i64, i64, i64, i64, i32p, i32p, i32p]
    lib.orc_validate_vcs.restype = ctypes.c_int
    lib.orc_spmm_vcs.argtypes = [ctypes.c_int, ctypes.c_int, i64, i32p, dp, i32p, i32p, dp,
                                 i64, dp, vp]
    lib.orc_spmm_vcs.restype = None
    lib.orc_spmm_csr.argtypes = [ctypes.c_int, i64, i32p, i32p, dp, dp, i64, dp, vp]
    lib.orc_spmm_csr.restype = None
    lib.orc_spmm_vcs_threaded.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i32p, dp, i32p,
                                          i32p, dp, i64, dp, ctypes.c_int]
    lib.orc_spmm_vcs_threaded.restype = ctypes.c_int
    lib.orc_spmm_csr_threaded.argtypes = [ctypes.c_int, i64, i64, i32p, i32p, dp, dp, i64, dp,
                                          ctypes.c_int]
    lib.orc_spmm_csr_threaded.restype = ctypes.c_int
    lib.orc_spmm_vcs_scaled.argtypes = [ctypes.c_int, ctypes.c_int, i64, i32p, dp, i32p, i32p,
                                        dp, dp, dp, i64, dp]
    lib.orc_spmm_vcs_scaled.restype = None
    lib.orc_spmm_csr_scaled.argtypes = [ctypes.c_int, i64, i32p, i32p, dp, dp, dp, dp, i64, dp]
    lib.orc_spmm_csr_scaled.restype = None
    lib.orc_expand_vcs.argtypes = [i64, i32p, vp, i32p, i32p, i32p, i32p, vp]
    lib.orc_expand_vcs.restype = None
    lib.orc_transpose_csr.argtypes = [i64, i64, i32p, i32p, vp, ctypes.c_int, i32p, i32p, vp]
    lib.orc_transpose_csr.restype = None
    lib.orc_assemble_csr.argtypes = [ctypes.c_int, i64, i64, i64, i32p, i32p, i32p, dp, i64,
                                     i32p, i32p, dp]
    lib.orc_assemble_csr.restype = None
    lib.orc_regroup_vcs.argtypes = [i64, i64, i32p, vp, i32p, i32p, i32p, vp, i32p, i32p]
    lib.orc_regroup_vcs.restype = ctypes.c_int64
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        raise TypeError(f"index arrays are int32, got {a.dtype}")
    return a


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _want(want, n_out):
    if want is None:
        return None
    mask = np.zeros(n_out, dtype=np.uint8)
    mask[np.asarray(want, dtype=np.int64)] = 1
    return mask


DIRS = {"AB": 0, "BA": 1}
LAYOUTS = {"vcsr": 1, "vcsc": 2}


def validate_csr(n_major, n_minor, ptr, idx, lib=None) -> int:
    lib = lib or load()
    ptr, idx = _i32(ptr), _i32(idx)
    if ptr.size != n_major + 1:
        return 3
    return lib.orc_validate_csr(n_major, n_minor, idx.size, _p(ptr), _p(idx))


def validate_vcs(n_major, n_minor, major_ptr, value_ptr, indices, n_groups=None, lib=None) -> int:
    lib = lib or load()
    major_ptr, value_ptr, indices = _i32(major_ptr), _i32(value_ptr), _i32(indices)
    n_groups = value_ptr.size - 1 if n_groups is None else n_groups
    if major_ptr.size != n_major + 1 or value_ptr.size != n_groups + 1:
        return 3
    return lib.orc_validate_vcs(n_major, n_minor, n_groups, indices.size, _p(major_ptr),
                                _p(value_ptr), _p(indices))


def spmm_vcs(layout, direction, shape, major_ptr, values, value_ptr, indices, B, want=None,
             lib=None) -> np.ndarray:
    """``A @ B`` (``direction="AB"``, B is n x w, result m x w) or ``(B @ A)``
    transposed (``direction="BA"``, B given transposed as m x w, result n x w),
    for A in VCSR or VCSC. ``want`` optionally lists the output rows to compute;
    the others are returned as zero."""
    lib = lib or load()
    m, n = shape
    n_major = m if layout == "vcsr" else n
    B = _f64(B)
    w = B.shape[1] if B.ndim == 2 else 1
    n_in, n_out = (n, m) if direction == "AB" else (m, n)
    if B.shape[0] != n_in:
        raise ValueError(f"dense operand has {B.shape[0]} rows, expected {n_in}")
    out = np.zeros((n_out, w), dtype=np.float64)
    mask = _want(want, n_out)
    major_ptr, value_ptr, indices = _i32(major_ptr), _i32(value_ptr), _i32(indices)
    vals = _f64(values)
    lib.orc_spmm_vcs(LAYOUTS[layout], DIRS[direction], n_major, _p(major_ptr), _p(vals),
                     _p(value_ptr), _p(indices), _p(B), w, _p(out),
                     None if mask is None else _p(mask))
    return out


def spmm_csr(direction, shape, row_ptr, col, val, B, want=None, lib=None) -> np.ndarray:
    """CSR counterpart of :func:`spmm_vcs` (rows are the major axis)."""
    lib = lib or load()
    m, n = shape
    B = _f64(B)
    w = B.shape[1] if B.ndim == 2 else 1
    n_in, n_out = (n, m) if direction == "AB" else (m, n)
    if B.shape[0] != n_in:
        raise ValueError(f"dense operand has {B.shape[0]} rows, expected {n_in}")
    out = np.zeros((n_out, w), dtype=np.float64)
    mask = _want(want, n_out)
    row_ptr, col, v = _i32(row_ptr), _i32(col), _f64(val)
    lib.orc_spmm_csr(DIRS[direction], m, _p(row_ptr), _p(col), _p(v), _p(B), w, _p(out),
                     None if mask is None else _p(mask))
    return out


def spmm(A, direction, B, want=None, lib=None) -> np.ndarray:
    """Dispatch on a ``workloads.Vcs`` or ``workloads.Csr`` container."""
    if hasattr(A, "major_ptr"):
        return spmm_vcs(A.layout, direction, A.shape, A.major_ptr, A.values, A.value_ptr,
                        A.indices, B, want=want, lib=lib)
    return spmm_csr(direction, A.shape, A.row_ptr, A.col, A.val, B, want=want, lib=lib)


def spmm_threaded(A, direction, B, threads, lib=None) -> np.ndarray:
    """The same product as :func:`spmm` on ``threads`` host threads (the timed
    CPU baseline): slices split over the threads, private float64 outputs
    summed in thread order where the output rows are not the slices. Equal
    to :func:`spmm` bit for bit where the output rows are the slices; else
    up to the regrouped additions' rounding."""
    lib = lib or load()
    m, n = A.shape
    B = _f64(B)
    w = B.shape[1] if B.ndim == 2 else 1
    n_in, n_out = (n, m) if direction == "AB" else (m, n)
    if B.shape[0] != n_in:
        raise ValueError(f"dense operand has {B.shape[0]} rows, expected {n_in}")
    out = np.zeros((n_out, w), dtype=np.float64)
    if hasattr(A, "major_ptr"):
        major_ptr, value_ptr, indices = _i32(A.major_ptr), _i32(A.value_ptr), _i32(A.indices)
        vals = _f64(A.values)
        n_major = m if A.layout == "vcsr" else n
        st = lib.orc_spmm_vcs_threaded(LAYOUTS[A.layout], DIRS[direction], n_major, n_out,
                                       _p(major_ptr), _p(vals), _p(value_ptr), _p(indices),
                                       _p(B), w, _p(out), int(threads))
    else:
        row_ptr, col, v = _i32(A.row_ptr), _i32(A.col), _f64(A.val)
        st = lib.orc_spmm_csr_threaded(DIRS[direction], m, n_out, _p(row_ptr), _p(col), _p(v),
                                       _p(B), w, _p(out), int(threads))
    if st != 0:
        raise MemoryError("the threaded oracle could not allocate its private outputs")
    return out


def spmm_view(A, direction, B, row_stat, col_stat, lib=None) -> np.ndarray:
    """The product of the normalized view whose stored entries (r, c, v) act
    as v * row_stat[r] * col_stat[c] (the library's "scale" view); otherwise
    as :func:`spmm`."""
    lib = lib or load()
    m, n = A.shape
    B = _f64(B)
    w = B.shape[1] if B.ndim == 2 else 1
    n_in, n_out = (n, m) if direction == "AB" else (m, n)
    if B.shape[0] != n_in:
        raise ValueError(f"dense operand has {B.shape[0]} rows, expected {n_in}")
    rs, cs = _f64(row_stat).reshape(-1), _f64(col_stat).reshape(-1)
    if rs.size != m or cs.size != n:
        raise ValueError("row_stat and col_stat must have n_rows and n_cols entries")
    out = np.zeros((n_out, w), dtype=np.float64)
    if hasattr(A, "major_ptr"):
        major_ptr, value_ptr, indices = _i32(A.major_ptr), _i32(A.value_ptr), _i32(A.indices)
        n_major = m if A.layout == "vcsr" else n
        lib.orc_spmm_vcs_scaled(LAYOUTS[A.layout], DIRS[direction], n_major, _p(major_ptr),
                                _p(_f64(A.values)), _p(value_ptr), _p(indices), _p(rs), _p(cs),
                                _p(B), w, _p(out))
    else:
        row_ptr, col = _i32(A.row_ptr), _i32(A.col)
        lib.orc_spmm_csr_scaled(DIRS[direction], m, _p(row_ptr), _p(col), _p(_f64(A.val)),
                                _p(rs), _p(cs), _p(B), w, _p(out))
    return out


def abs_scale_view(A, direction, B, row_stat, col_stat, lib=None) -> np.ndarray:
    """``|G| |B|`` for the "scale" view's transformed entries G: the scale of
    each output's rounding error."""
    absA = _abs_values(A)
    return spmm_view(absA, direction, np.abs(_f64(B)), np.abs(_f64(row_stat)),
                     np.abs(_f64(col_stat)), lib=lib)


def _abs_values(A):
    """The same container with every stored value replaced by its magnitude."""
    import dataclasses
    if hasattr(A, "major_ptr"):
        return dataclasses.replace(A, values=np.abs(np.asarray(A.values)))
    return dataclasses.replace(A, val=np.abs(np.asarray(A.val)))


def abs_scale(A, direction, B, want=None, lib=None) -> np.ndarray:
    """``|A| |B|`` in the same output layout: the scale of each output's
    rounding error, used to judge float32 results."""
    if hasattr(A, "major_ptr"):
        return spmm_vcs(A.layout, direction, A.shape, A.major_ptr, np.abs(_f64(A.values)),
                        A.value_ptr, A.indices, np.abs(_f64(B)), want=want, lib=lib)
    return spmm_csr(direction, A.shape, A.row_ptr, A.col, np.abs(_f64(A.val)),
                    np.abs(_f64(B)), want=want, lib=lib)


def expand_vcs(major_ptr, values, value_ptr, indices, lib=None):
    """VCS -> (ptr, idx, val float32) with one value per entry, stored order."""
    lib = lib or load()
    major_ptr, value_ptr, indices = _i32(major_ptr), _i32(value_ptr), _i32(indices)
    values = np.ascontiguousarray(values, dtype=np.float32)
    n_major = major_ptr.size - 1
    ptr = np.empty(n_major + 1, dtype=np.int32)
    idx = np.empty(indices.size, dtype=np.int32)
    val = np.empty(indices.size, dtype=np.float32)
    lib.orc_expand_vcs(n_major, _p(major_ptr), _p(values), _p(value_ptr), _p(indices),
                       _p(ptr), _p(idx), _p(val))
    return ptr, idx, val


def expand_vcs_format(layout, shape, major_ptr, values, value_ptr, indices, fmt="csr",
                      sort_indices=True, lib=None):
    """A VCSR or VCSC expanded to one value per entry as the CSR ("csr") or the
    CSC ("csc") of A (vsparse page, section "Benchmarks": the expansion the
    baseline runs on is index-sorted by default, with an opt-out, and takes a
    format so that a VCSC-backed matrix can be expanded to CSR). In the
    layout's own format (CSR from a VCSR, CSC from a VCSC) the stored-order
    expansion is returned, or with sort_indices each slice's entries ordered
    by index, a stable sort (repeated indices keep their stored order). In
    the other format the result is the exact transpose of the stored-order
    expansion, whose slices list their entries by ascending index already.
    Returns (ptr, idx, val float32)."""
    ptr, idx, val = expand_vcs(major_ptr, values, value_ptr, indices, lib=lib)
    own = "csr" if layout == "vcsr" else "csc"
    if fmt not in ("csr", "csc"):
        raise ValueError(fmt)
    if fmt == own:
        if sort_indices:
            slice_of = np.repeat(np.arange(ptr.size - 1), np.diff(ptr))
            order = np.lexsort((idx, slice_of))  # by slice, then index; stable
            idx, val = idx[order], val[order]
        return ptr, idx, val
    n_minor = shape[1] if layout == "vcsr" else shape[0]
    return transpose_csr(n_minor, ptr, idx, val, lib=lib)


def transpose_csr(n_minor, ptr, idx, val, lib=None):
    """Exact transpose by the stable two-pass counting sort; the payload
    (float32 or float64) is copied bit for bit."""
    lib = lib or load()
    ptr, idx = _i32(ptr), _i32(idx)
    val = np.ascontiguousarray(val)
    if val.dtype not in (np.float32, np.float64):
        raise TypeError(val.dtype)
    n_major = ptr.size - 1
    t_ptr = np.empty(n_minor + 1, dtype=np.int32)
    t_idx = np.empty(idx.size, dtype=np.int32)
    t_val = np.empty(idx.size, dtype=val.dtype)
    lib.orc_transpose_csr(n_major, n_minor, _p(ptr), _p(idx), _p(val), val.itemsize,
                          _p(t_ptr), _p(t_idx), _p(t_val))
    return t_ptr, t_idx, t_val


def transpose_csr_scaled(n_minor, ptr, idx, val, factor, lib=None):
    """The exact transpose with each entry scaled by a factor of its own
    (regridding page, section "API": the conservative transpose scales each
    entry of the exact transpose by its own element's cells and shares .T's
    indices): entry p becomes val[p] * factor[p], one rounding to val's type
    (the product of two float32 numbers is exact in float64)."""
    val = np.ascontiguousarray(val)
    scaled = (val.astype(np.float64) * np.asarray(factor, dtype=np.float64)).astype(val.dtype)
    return transpose_csr(n_minor, ptr, idx, scaled, lib=lib)


ROLES = {"own": 0, "shared": 1, "summed": 2, "sum_of": 3}


def assembled_shape(role, n_elem, n_out, n_in):
    """(rows, columns) of the operator a role assembles."""
    r = ROLES[role]
    return (n_elem * n_out if r <= 1 else n_out, n_elem * n_in if r in (0, 2) else n_in)


def assemble_csr(role, n_elem, n_out, n_in, elem_ptr, out_idx, in_idx, weight, lib=None):
    """The regridder's operator from its elements' weights, by the two-pass
    counting sort (see orc_assemble_csr): (row_ptr, col, val) with val in
    weight's type (copied, not computed)."""
    lib = lib or load()
    elem_ptr, out_idx, in_idx = _i32(elem_ptr), _i32(out_idx), _i32(in_idx)
    weight = np.ascontiguousarray(weight)
    n_rows, _ = assembled_shape(role, n_elem, n_out, n_in)
    nnz = out_idx.size
    row_ptr = np.empty(n_rows + 1, dtype=np.int32)
    col = np.empty(nnz, dtype=np.int32)
    val = np.empty(nnz, dtype=np.float64)
    lib.orc_assemble_csr(ROLES[role], n_elem, n_out, n_in, _p(elem_ptr), _p(out_idx),
                         _p(in_idx), _p(_f64(weight)), n_rows, _p(row_ptr), _p(col), _p(val))
    return row_ptr, col, val.astype(weight.dtype)


def regroup_vcs(n_minor, major_ptr, values, value_ptr, indices, lib=None):
    """The same matrix in the opposite VCS layout, canonical order (groups by
    ascending value, entries of a group in stored order)."""
    lib = lib or load()
    major_ptr, value_ptr, indices = _i32(major_ptr), _i32(value_ptr), _i32(indices)
    values = np.ascontiguousarray(values, dtype=np.float32)
    n_major = major_ptr.size - 1
    nnz = indices.size
    t_major_ptr = np.empty(n_minor + 1, dtype=np.int32)
    t_values = np.empty(max(nnz, 1), dtype=np.float32)
    t_value_ptr = np.empty(nnz + 1, dtype=np.int32)
    t_indices = np.empty(nnz, dtype=np.int32)
    g = lib.orc_regroup_vcs(n_major, n_minor, _p(major_ptr), _p(values), _p(value_ptr),
                            _p(indices), _p(t_major_ptr), _p(t_values), _p(t_value_ptr),
                            _p(t_indices))
    return t_major_ptr, t_values[:g].copy(), t_value_ptr[:g + 1].copy(), t_indices


def max_rel_error(got, ref, scale):
    """max |got - ref| / scale over outputs with scale > 0, and whether every
    output with scale == 0 is exactly zero."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    pos = scale > 0
    rel = float((err[pos] / scale[pos]).max()) if pos.any() else 0.0
    zeros_ok = bool(np.all(got[~pos] == 0))
    return rel, zeros_ok
