"""Python binding of libvspmm (sparse x dense products over CSR, VCSR and VCSC
on MI355X).

Argument marshalling only: every product, transpose and regrouping runs in the
HIP kernels of ``libvspmm.so``. torch supplies device memory and the current
stream. There is no fallback: importing this package without the built library
raises ImportError, and a call that the library rejects raises VspmmError.

    A = VcsMatrix.from_arrays("vcsr", (m, n), major_ptr, values, value_ptr, indices)
    out = A @ B          # B: n x w (cuda, float32) -> m x w
    out = B @ A          # B: w x m -> w x n
    A.T                  # the transpose, a VCSC over the same arrays
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["VcsMatrix", "CsrMatrix", "Schedule", "VspmmError", "assemble_csr", "lib", "LIB_PATH",
           "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvspmm.so")

LAYOUTS = {"csr": 0, "vcsr": 1, "vcsc": 2}
DIRECTIONS = {"AB": 0, "BA": 1}
MODES = {"atomic": 0, "deterministic": 1}
# roles of a regridder's orthogonal axis (see vspmm_assemble_csr)
ROLES = {"own": 0, "shared": 1, "summed": 2, "sum_of": 3}
# normalized views the binding offers; the library must implement each one
VIEWS = {"identity": 0, "scale": 1}
SPLIT_WIDTH, SPLIT_MATRIX, VALIDATE = 1, 2, 4

_vp, _i64, _i32, _u32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                              ctypes.c_size_t)
_P = ctypes.POINTER

# name -> (argtypes, restype); mirrors include/vspmm.h
EXPORTS = {
    "vspmm_create_vcs": ([_P(_vp), ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _u32,
                          _i32, _vp], ctypes.c_int),
    "vspmm_create_csr": ([_P(_vp), _i64, _i64, _i64, _vp, _vp, _vp, ctypes.c_int, _u32, _i32, _vp],
                         ctypes.c_int),
    "vspmm_create_csr64": ([_P(_vp), _i64, _i64, _i64, _vp, _vp, _vp, ctypes.c_int, _u32, _i32,
                            _i64, _vp], ctypes.c_int),
    "vspmm_destroy": ([_vp], ctypes.c_int),
    "vspmm_spmm": ([_vp, _vp, _vp, _i64, ctypes.c_int, _vp], ctypes.c_int),
    "vspmm_workspace_size": ([_vp, ctypes.c_int, ctypes.c_int, _P(_sz)], ctypes.c_int),
    "vspmm_spmm_ex": ([_vp, _vp, _vp, _i64, ctypes.c_int, ctypes.c_int, _vp, _sz, _vp],
                      ctypes.c_int),
    "vspmm_spmm_noalloc": ([_vp, _vp, _vp, _i64, ctypes.c_int, ctypes.c_int, _vp], ctypes.c_int),
    "vspmm_schedule_create": ([_P(_vp), _vp, ctypes.c_int, _i64, _vp, _sz, _vp], ctypes.c_int),
    "vspmm_schedule_spmm": ([_vp, _vp, _vp, _i64, _vp], ctypes.c_int),
    "vspmm_schedule_bytes": ([_vp, _P(_sz)], ctypes.c_int),
    "vspmm_schedule_destroy": ([_vp], ctypes.c_int),
    "vspmm_validate": ([_vp, _vp], ctypes.c_int),
    "vspmm_transpose_csr": ([_vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "vspmm_transpose_csr_scaled": ([_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "vspmm_assemble_csr": ([_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                            _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "vspmm_assemble_workspace_size": ([_i32, _i64, _i64, _i64, _i64, _P(_sz)], ctypes.c_int),
    "vspmm_regroup_vcs": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "vspmm_expand_vcs": ([_vp, ctypes.c_int, _i32, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "vspmm_footprint": ([_vp, _P(_sz), _P(_sz)], ctypes.c_int),
    "vspmm_workspace_size_width": ([_vp, ctypes.c_int, ctypes.c_int, _i64, _P(_sz)],
                                   ctypes.c_int),
    "vspmm_plan_info": ([_vp, _i64, ctypes.c_int, ctypes.c_int, _P(_i32), _P(_i32), _P(_i32),
                         _P(_i32), _P(_i32), _P(_i32), _P(_i32)], ctypes.c_int),
    "vspmm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "vspmm_set_view": ([_vp, _i32, _vp, _vp, _i64], ctypes.c_int),
    "vspmm_view_name": ([_i32], ctypes.c_char_p),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m sparse_dense_matmul_amd.build`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (argtypes, restype) in EXPORTS.items():
        try:
            fn = getattr(handle, name)
        except AttributeError as e:
            raise ImportError(f"{LIB_PATH} lacks {name}: rebuild it with "
                              "`python -m sparse_dense_matmul_amd.build`") from e
        fn.argtypes = argtypes
        fn.restype = restype
    # every view the binding offers must be one the library implements:
    # otherwise fail here, loudly, instead of computing another product
    for name, code in VIEWS.items():
        got = handle.vspmm_view_name(code)
        if got is None or got.decode() != name:
            raise ImportError(f"{LIB_PATH} does not implement the normalized view '{name}' "
                              f"(code {code})")
    return handle


class _Lib:
    """The library, loaded on first use, so that importing the package (the
    build module included) works before the library is built; any call then
    fails loudly if it is missing or stale."""

    _handle = None

    def __getattr__(self, name):
        if _Lib._handle is None:
            _Lib._handle = _load()
        return getattr(_Lib._handle, name)


lib = _Lib()


class VspmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.vspmm_status_string(status).decode()} (status {status})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise VspmmError(status, where)


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _dev_tensor(t, dtype, device, name):
    t = torch.as_tensor(t)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.contiguous()


class SparseMatrix:
    """A handle over device arrays that it keeps alive (never copied)."""

    layout: str
    dtype: torch.dtype

    def __init__(self, handle, arrays, shape, layout, dtype, device, flags, force_group):
        self._h = handle
        self._arrays = arrays
        self.shape = tuple(int(x) for x in shape)
        self.layout = layout
        self.dtype = dtype
        self.device = device
        self.flags = flags
        self.force_group = force_group

    def __del__(self):
        h = getattr(self, "_h", None)
        # at interpreter exit the module's globals may already be gone; the
        # process is ending and the driver frees the device memory then
        if h and lib is not None:
            lib.vspmm_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    # ----------------------------------------------------------- products

    def _dense_in(self, B, rows, name="B"):
        B = _dev_tensor(B, self.dtype, self.device, name)
        if B.dim() == 1:
            B = B.unsqueeze(1)
        if B.dim() != 2 or B.shape[0] != rows:
            raise ValueError(f"{name} has shape {tuple(B.shape)}, expected ({rows}, width)")
        return B

    def _operands(self, B, direction, out):
        m, n = self.shape
        n_in, n_out = (n, m) if direction == "AB" else (m, n)
        B = self._dense_in(B, n_in)
        w = B.shape[1]
        if out is None:
            out = torch.empty((n_out, w), dtype=self.dtype, device=self.device)
        elif out.shape != (n_out, w) or not out.is_contiguous() or out.dtype != self.dtype:
            raise ValueError("out must be a contiguous (n_out, width) tensor of the matrix dtype")
        return B, out

    def spmm(self, B: torch.Tensor, direction: str = "AB", mode: str = "atomic",
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
        """``A @ B`` for ``direction="AB"`` (B: n x w, returns m x w), or
        ``(B @ A)`` transposed for ``direction="BA"`` (B given transposed,
        m x w; returns n x w). ``mode="deterministic"`` makes the misaligned
        directions repeat bit for bit (needs ``workspace``, see
        :meth:`workspace_size`); each such call builds its layout again, see
        :meth:`schedule` to build it once."""
        B, out = self._operands(B, direction, out)
        w = B.shape[1]
        d, md = DIRECTIONS[direction], MODES[mode]
        if md == 0:
            st = lib.vspmm_spmm(self._h, _ptr(B), _ptr(out), w, d, _stream(self.device))
        else:
            ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
            st = lib.vspmm_spmm_ex(self._h, _ptr(B), _ptr(out), w, d, md, _ptr(workspace),
                                   ws_bytes, _stream(self.device))
        _check(st, "vspmm_spmm")
        return out

    def __matmul__(self, B):
        B = torch.as_tensor(B)
        if B.dim() == 1:
            return self.spmm(B.unsqueeze(1), "AB")[:, 0]
        return self.spmm(B, "AB")

    def __rmatmul__(self, B):
        B = torch.as_tensor(B)
        if B.dim() == 1:
            return self.spmm(B.unsqueeze(1), "BA")[:, 0]
        return self.spmm(B.t().contiguous(), "BA").t()

    def workspace_size(self, direction: str = "BA", mode: str = "deterministic",
                       width: int | None = None) -> int:
        """Workspace bytes for ``spmm(..., mode=mode)``; with ``width``, enough for
        the tiled schedule at that width when one applies."""
        n = _sz(0)
        if width is None:
            _check(lib.vspmm_workspace_size(self._h, DIRECTIONS[direction], MODES[mode],
                                            ctypes.byref(n)), "vspmm_workspace_size")
        else:
            _check(lib.vspmm_workspace_size_width(self._h, DIRECTIONS[direction], MODES[mode],
                                                  width, ctypes.byref(n)),
                   "vspmm_workspace_size_width")
        return int(n.value)

    def workspace(self, direction: str = "BA", mode: str = "deterministic",
                  width: int | None = None) -> torch.Tensor:
        """A device workspace of the required size (torch's allocations are
        256-byte aligned)."""
        nbytes = self.workspace_size(direction, mode, width)
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)

    def schedule(self, direction: str, width: int,
                 workspace: torch.Tensor | None = None) -> "Schedule":
        """The deterministic product's layout for ``direction`` at ``width``,
        built once (``vspmm_schedule_create``); ``workspace`` is build scratch
        (``workspace_size(direction, "deterministic", width)`` bytes), or
        None for scratch the library allocates for the call."""
        h = _vp()
        nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        with torch.cuda.device(self.device):
            st = lib.vspmm_schedule_create(ctypes.byref(h), self._h, DIRECTIONS[direction],
                                           int(width), _ptr(workspace), nbytes,
                                           _stream(self.device))
        _check(st, "vspmm_schedule_create")
        return Schedule(h, self, direction, int(width))

    def normalized(self, view: str, row_stat=None, col_stat=None,
                   max_width: int = 64) -> "SparseMatrix":
        """A view of the same arrays whose stored entries (r, c, v) act as
        g(v, r, c): ``"identity"`` (v) or ``"scale"`` (v * row_stat[r] *
        col_stat[c], statistics of the dense operands' type on the device).
        Products up to ``max_width`` columns (see ``vspmm_set_view``)."""
        if view not in VIEWS:
            raise ValueError(f"unknown normalized view {view!r}; known: {sorted(VIEWS)}")
        m, n = self.shape
        stats = ()
        if view != "identity":
            row_stat = _dev_tensor(row_stat, self.dtype, self.device, "row_stat")
            col_stat = _dev_tensor(col_stat, self.dtype, self.device, "col_stat")
            if row_stat.numel() != m or col_stat.numel() != n:
                raise ValueError(f"statistics must have {m} and {n} entries")
            stats = (row_stat, col_stat)
        other = self._clone_handle()
        st = lib.vspmm_set_view(other._h, VIEWS[view], _ptr(stats[0]) if stats else None,
                                _ptr(stats[1]) if stats else None, int(max_width))
        _check(st, "vspmm_set_view")
        other._view = (view, stats, int(max_width))
        return other

    def validate(self) -> bool:
        st = lib.vspmm_validate(self._h, _stream(self.device))
        if st == 4:
            return False
        _check(st, "vspmm_validate")
        return True

    def footprint(self) -> tuple[int, int]:
        a, b = _sz(0), _sz(0)
        _check(lib.vspmm_footprint(self._h, ctypes.byref(a), ctypes.byref(b)), "vspmm_footprint")
        return int(a.value), int(b.value)

    def plan_info(self, width: int, direction: str = "AB", mode: str = "atomic") -> dict:
        vals = [_i32(0) for _ in range(7)]
        _check(lib.vspmm_plan_info(self._h, width, DIRECTIONS[direction], MODES[mode],
                                   *[ctypes.byref(v) for v in vals]), "vspmm_plan_info")
        keys = ("entry_lanes", "width_lanes", "vec", "slices_per_wave", "lds_staged", "kernel",
                "tiles")
        info = {k: int(v.value) for k, v in zip(keys, vals)}
        # the walked layout: the handle's own, or the opposite one in deterministic mode
        aligned = (self.layout != "vcsc") == (direction == "AB")
        walked = self.layout if aligned or mode == "atomic" or info["tiles"] else \
            {"vcsr": "vcsc", "vcsc": "vcsr", "csr": "csr"}[self.layout]
        vcs = walked != "csr"
        info["kernel_name"] = {0: "k_aligned", 1: "k_vcs_rows" if vcs else "k_short",
                               4: "k_vcs_seg",
                               2: "k_vcs_long" if vcs else "k_long",
                               3: "k_scatter"}[info["kernel"]]
        return info


class Schedule:
    """A built deterministic product (see ``vspmm_schedule_create``). Keeps its
    matrix alive; products through it must not overlap in time (one stream)."""

    def __init__(self, handle, matrix: SparseMatrix, direction: str, width: int):
        self._h = handle
        self.matrix = matrix
        self.direction = direction
        self.width = width

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and lib is not None:
            lib.vspmm_schedule_destroy(h)
            self._h = None

    @property
    def nbytes(self) -> int:
        n = _sz(0)
        _check(lib.vspmm_schedule_bytes(self._h, ctypes.byref(n)), "vspmm_schedule_bytes")
        return int(n.value)

    def spmm(self, B: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """The product in the schedule's direction (operands as
        :meth:`SparseMatrix.spmm`)."""
        B, out = self.matrix._operands(B, self.direction, out)
        st = lib.vspmm_schedule_spmm(self._h, _ptr(B), _ptr(out), B.shape[1],
                                     _stream(self.matrix.device))
        _check(st, "vspmm_schedule_spmm")
        return out


class VcsMatrix(SparseMatrix):
    """VCSR (``layout="vcsr"``) or VCSC over device arrays: for major slice i
    the distinct values are ``values[major_ptr[i]:major_ptr[i+1]]`` and value k
    is shared by ``indices[value_ptr[k]:value_ptr[k+1]]``."""

    @classmethod
    def from_arrays(cls, layout, shape, major_ptr, values, value_ptr, indices, flags=0,
                    force_group=0, validate=False):
        if layout not in ("vcsr", "vcsc"):
            raise ValueError(layout)
        dev = torch.as_tensor(major_ptr).device
        major_ptr = _dev_tensor(major_ptr, torch.int32, dev, "major_ptr")
        values = _dev_tensor(values, torch.float32, dev, "values")
        value_ptr = _dev_tensor(value_ptr, torch.int32, dev, "value_ptr")
        indices = _dev_tensor(indices, torch.int32, dev, "indices")
        m, n = (int(x) for x in shape)
        flags = flags | (VALIDATE if validate else 0)
        h = _vp()
        with torch.cuda.device(dev):
            st = lib.vspmm_create_vcs(ctypes.byref(h), LAYOUTS[layout], m, n, values.numel(),
                                      indices.numel(), _ptr(major_ptr), _ptr(values),
                                      _ptr(value_ptr), _ptr(indices), flags, force_group,
                                      _stream(dev))
        _check(st, "vspmm_create_vcs")
        return cls(h, (major_ptr, values, value_ptr, indices), (m, n), layout, torch.float32, dev,
                   flags, force_group)

    @property
    def major_ptr(self):
        return self._arrays[0]

    @property
    def values(self):
        return self._arrays[1]

    @property
    def value_ptr(self):
        return self._arrays[2]

    @property
    def indices(self):
        return self._arrays[3]

    @property
    def T(self) -> "VcsMatrix":
        """The transpose: the same arrays read as the other layout."""
        other = "vcsc" if self.layout == "vcsr" else "vcsr"
        t = VcsMatrix.from_arrays(other, (self.shape[1], self.shape[0]), *self._arrays,
                                  flags=self.flags & ~VALIDATE, force_group=self.force_group)
        view = getattr(self, "_view", None)
        if view is not None and view[0] != "identity":
            # the transposed view: the statistics change axes
            t = t.normalized(view[0], view[1][1], view[1][0], view[2])
        return t

    def _clone_handle(self) -> "VcsMatrix":
        return VcsMatrix.from_arrays(self.layout, self.shape, *self._arrays,
                                     flags=self.flags & ~VALIDATE, force_group=self.force_group)

    def regroup(self, workspace: torch.Tensor | None = None) -> "VcsMatrix":
        """The same matrix in the opposite layout (VCSR <-> VCSC), canonical."""
        m, n = self.shape
        n_minor = n if self.layout == "vcsr" else m
        nnz = self.indices.numel()
        dev = self.device
        t_mp = torch.empty(n_minor + 1, dtype=torch.int32, device=dev)
        t_v = torch.empty(max(nnz, 1), dtype=torch.float32, device=dev)
        t_vp = torch.empty(nnz + 1, dtype=torch.int32, device=dev)
        t_i = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        t_g = torch.empty(1, dtype=torch.int32, device=dev)
        ws = workspace if workspace is not None else self.workspace("BA" if self.layout == "vcsr"
                                                                    else "AB")
        st = lib.vspmm_regroup_vcs(self._h, _ptr(t_mp), _ptr(t_v), _ptr(t_vp), _ptr(t_i),
                                   _ptr(t_g), _ptr(ws), ws.numel(), _stream(dev))
        _check(st, "vspmm_regroup_vcs")
        g = int(t_g.item())
        other = "vcsc" if self.layout == "vcsr" else "vcsr"
        return VcsMatrix.from_arrays(other, self.shape, t_mp, t_v[:g].clone(),
                                     t_vp[:g + 1].clone(), t_i[:nnz].clone(), flags=self.flags,
                                     force_group=self.force_group)


    def expand(self, format: str = "csr", sort_indices: bool = True,
               workspace: torch.Tensor | None = None):
        """The matrix with one value per entry, as (ptr, idx, val) of its CSR
        (``format="csr"``) or CSC (``"csc"``), index-sorted by default; see
        ``vspmm_expand_vcs``."""
        if format not in ("csr", "csc"):
            raise ValueError("format must be 'csr' or 'csc'")
        m, n = self.shape
        nnz = self.indices.numel()
        dev = self.device
        ptr = torch.empty((m if format == "csr" else n) + 1, dtype=torch.int32, device=dev)
        idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        val = torch.empty(max(nnz, 1), dtype=torch.float32, device=dev)
        own = (format == "csr") == (self.layout == "vcsr")
        ws = workspace
        if ws is None and (sort_indices or not own):
            ws = self.workspace("BA" if self.layout == "vcsr" else "AB")
        st = lib.vspmm_expand_vcs(self._h, 0 if format == "csr" else 1, int(bool(sort_indices)),
                                  _ptr(ptr), _ptr(idx), _ptr(val), _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(dev))
        _check(st, "vspmm_expand_vcs")
        return ptr, idx[:nnz], val[:nnz]


class CsrMatrix(SparseMatrix):
    """CSR over device arrays: float32 or float64 values; the dense operands
    and the sums follow the values' type, or ``dtype=torch.float64`` with
    float32 values sums them in float64 (``VSPMM_F32_F64``). ``ptr64=True`` (implied
    past 2^31 - 1 entries) keeps int64 row pointers: the rows are cut into blocks
    of at most ``block_nnz`` entries (0: 2^30), each walked as an int32 CSR."""

    @classmethod
    def from_arrays(cls, shape, row_ptr, col, val, flags=0, force_group=0, validate=False,
                    dtype=None, ptr64=False, block_nnz=0):
        dev = torch.as_tensor(row_ptr).device
        val = torch.as_tensor(val)
        if val.dtype not in (torch.float32, torch.float64):
            raise TypeError(f"val must be float32 or float64, got {val.dtype}")
        dtype = val.dtype if dtype is None else dtype
        if dtype == val.dtype:
            code = 1 if val.dtype == torch.float64 else 0
        elif val.dtype == torch.float32 and dtype == torch.float64:
            code = 2  # float32 values, float64 operands and sums
        else:
            raise TypeError(f"{val.dtype} values cannot be summed in {dtype}")
        ptr64 = ptr64 or torch.as_tensor(col).numel() > 2**31 - 1
        row_ptr = _dev_tensor(row_ptr, torch.int64 if ptr64 else torch.int32, dev, "row_ptr")
        col = _dev_tensor(col, torch.int32, dev, "col")
        val = _dev_tensor(val, val.dtype, dev, "val")
        m, n = (int(x) for x in shape)
        flags = flags | (VALIDATE if validate else 0)
        h = _vp()
        with torch.cuda.device(dev):
            if ptr64:
                st = lib.vspmm_create_csr64(ctypes.byref(h), m, n, col.numel(), _ptr(row_ptr),
                                            _ptr(col), _ptr(val), code, flags, force_group,
                                            block_nnz, _stream(dev))
            else:
                st = lib.vspmm_create_csr(ctypes.byref(h), m, n, col.numel(), _ptr(row_ptr),
                                          _ptr(col), _ptr(val), code, flags, force_group,
                                          _stream(dev))
        _check(st, "vspmm_create_csr64" if ptr64 else "vspmm_create_csr")
        out = cls(h, (row_ptr, col, val), (m, n), "csr", dtype, dev, flags, force_group)
        out._block_nnz = block_nnz
        return out

    def _clone_handle(self) -> "CsrMatrix":
        return CsrMatrix.from_arrays(self.shape, *self._arrays, flags=self.flags & ~VALIDATE,
                                     force_group=self.force_group, dtype=self.dtype,
                                     ptr64=self.row_ptr.dtype == torch.int64,
                                     block_nnz=getattr(self, "_block_nnz", 0))

    @property
    def row_ptr(self):
        return self._arrays[0]

    @property
    def col(self):
        return self._arrays[1]

    @property
    def val(self):
        return self._arrays[2]

    def transpose_scaled(self, factor, workspace: torch.Tensor | None = None) -> "CsrMatrix":
        """The exact transpose with entry p's value multiplied by factor[p]
        (one factor per stored entry, in stored order; the indices are the
        exact transpose's), see ``vspmm_transpose_csr_scaled``."""
        m, n = self.shape
        nnz = self.col.numel()
        dev = self.device
        factor = _dev_tensor(factor, self.val.dtype, dev, "factor")
        if factor.numel() != nnz:
            raise ValueError(f"factor must have {nnz} entries")
        t_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
        t_col = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        t_val = torch.empty(max(nnz, 1), dtype=self.val.dtype, device=dev)
        ws = workspace if workspace is not None else self.workspace("BA")
        st = lib.vspmm_transpose_csr_scaled(self._h, _ptr(factor), _ptr(t_ptr), _ptr(t_col),
                                            _ptr(t_val), _ptr(ws), ws.numel(), _stream(dev))
        _check(st, "vspmm_transpose_csr_scaled")
        return CsrMatrix.from_arrays((n, m), t_ptr, t_col[:nnz], t_val[:nnz],
                                     flags=self.flags & ~VALIDATE, force_group=self.force_group,
                                     dtype=self.dtype)

    def transpose(self, workspace: torch.Tensor | None = None) -> "CsrMatrix":
        """The exact transpose (each new row lists its entries by ascending
        source row), bit-identical to a sequential counting sort."""
        m, n = self.shape
        nnz = self.col.numel()
        dev = self.device
        t_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
        t_col = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        t_val = torch.empty(max(nnz, 1), dtype=self.val.dtype, device=dev)
        ws = workspace if workspace is not None else self.workspace("BA")
        st = lib.vspmm_transpose_csr(self._h, _ptr(t_ptr), _ptr(t_col), _ptr(t_val), _ptr(ws),
                                     ws.numel(), _stream(dev))
        _check(st, "vspmm_transpose_csr")
        return CsrMatrix.from_arrays((n, m), t_ptr, t_col[:nnz], t_val[:nnz],
                                     flags=self.flags & ~VALIDATE, force_group=self.force_group,
                                     dtype=self.dtype)


def assemble_csr(role: str, n_out: int, n_in: int, elem_ptr, out_idx, in_idx, weight,
                 workspace: torch.Tensor | None = None, **kw) -> CsrMatrix:
    """A regridder's operator from its elements' weights (``vspmm_assemble_csr``):
    element e's entries are ``[elem_ptr[e], elem_ptr[e+1])`` of (out_idx,
    in_idx, weight), device arrays; ``role`` is one of ``ROLES``. Returns the
    assembled CSR (float32 or float64 like ``weight``); ``kw`` goes to
    :meth:`CsrMatrix.from_arrays`."""
    if role not in ROLES:
        raise ValueError(f"unknown role {role!r}; known: {sorted(ROLES)}")
    dev = torch.as_tensor(elem_ptr).device
    elem_ptr = _dev_tensor(elem_ptr, torch.int32, dev, "elem_ptr")
    out_idx = _dev_tensor(out_idx, torch.int32, dev, "out_idx")
    in_idx = _dev_tensor(in_idx, torch.int32, dev, "in_idx")
    weight = torch.as_tensor(weight)
    if weight.dtype not in (torch.float32, torch.float64):
        raise TypeError(f"weight must be float32 or float64, got {weight.dtype}")
    weight = _dev_tensor(weight, weight.dtype, dev, "weight")
    n_elem, nnz = elem_ptr.numel() - 1, out_idx.numel()
    if in_idx.numel() != nnz or weight.numel() != nnz:
        raise ValueError("out_idx, in_idx and weight must have the same length")
    r = ROLES[role]
    rows = n_elem * n_out if r <= 1 else n_out
    cols = n_elem * n_in if r in (0, 2) else n_in
    need = _sz(0)
    _check(lib.vspmm_assemble_workspace_size(r, n_elem, n_out, n_in, nnz, ctypes.byref(need)),
           "vspmm_assemble_workspace_size")
    ws = workspace if workspace is not None else \
        torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(nnz, 1), dtype=weight.dtype, device=dev)
    with torch.cuda.device(dev):
        st = lib.vspmm_assemble_csr(r, n_elem, n_out, n_in, nnz, _ptr(elem_ptr), _ptr(out_idx),
                                    _ptr(in_idx), _ptr(weight),
                                    1 if weight.dtype == torch.float64 else 0, _ptr(row_ptr),
                                    _ptr(col), _ptr(val), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "vspmm_assemble_csr")
    return CsrMatrix.from_arrays((rows, cols), row_ptr, col[:nnz], val[:nnz], **kw)
