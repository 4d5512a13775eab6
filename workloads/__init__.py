"""Seeded synthetic inputs for the sparse x dense product workloads.

This module only draws random matrices and lays them out; it holds none of the
product's arithmetic and imports neither the oracle nor the HIP library, so the
two sides that are compared against each other can both take their inputs from
here.

Layouts produced (all index arrays int32, as the device library takes them):

* CSR: ``row_ptr[m+1]``, ``col[nnz]``, ``val[nnz]``.
* VCSR / VCSC, the value-grouped layout of the vsparse page ("Add CUDA transfer
  and matmul kernels for the normalized views", section "The layout stays
  compressed"): for major slice ``i`` (a row for VCSR, a column for VCSC) the
  distinct values are ``values[major_ptr[i]:major_ptr[i+1]]`` and value ``k`` is
  shared by the minor indices ``indices[value_ptr[k]:value_ptr[k+1]]``.

Canonical order, used by every builder here: within a slice the groups are in
ascending value, and within a group the minor indices ascend.

Workloads (the shapes and distributions the pages describe; the pages' own
matrices and the regridding data are not available, so these stand in for
them):

* ``config1``: CSR 2,000 x 500, Poisson(10) entries per row, U(0,1) values.
* ``count_matrix(60_000, 2_000, 100, 64)``: the 60k x 2k, ~6M-entry count
  matrix the vsparse page benchmarks at width 16 (its "Benchmarks" table);
  stored as VCSR (``config2``) and VCSC (``config3``).
* ``config4``: a regridding-shaped CSR operator (regridding page, sections
  "How it is built" and "Performance"): 20,000 rows with log-normal row
  lengths (median 40, clipped to 1..4,000, ~5% empty rows), ~1.1M U(0,1)
  weights, n_cols = nnz/3 so that its transpose has ~3 entries per row.
* ``count_matrix(1_000_000, 20_000, 200, 255)``: the large count matrix
  (``config5``).
"""

from __future__ import annotations

import dataclasses
import numpy as np

SEED_BASE = 20261202


def rng_for(config_index: int, salt: int = 0) -> np.random.Generator:
    """The PCG64 stream for one workload (seed = 20261202 + config index)."""
    return np.random.Generator(np.random.PCG64([SEED_BASE + config_index, salt]))


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------


@dataclasses.dataclass
class Triplets:
    """A sparse matrix as coordinate triplets, without duplicates."""

    shape: tuple[int, int]
    rows: np.ndarray  # int64
    cols: np.ndarray  # int64
    vals: np.ndarray  # float32 or float64

    @property
    def nnz(self) -> int:
        return int(self.rows.size)


@dataclasses.dataclass
class Csr:
    shape: tuple[int, int]
    row_ptr: np.ndarray  # int32 [m+1]
    col: np.ndarray  # int32 [nnz]
    val: np.ndarray  # float32 / float64 [nnz]

    @property
    def nnz(self) -> int:
        return int(self.col.size)

    def nbytes(self) -> int:
        return self.row_ptr.nbytes + self.col.nbytes + self.val.nbytes


@dataclasses.dataclass
class Vcs:
    """VCSR (``layout == "vcsr"``, major = rows) or VCSC (major = columns)."""

    layout: str
    shape: tuple[int, int]
    major_ptr: np.ndarray  # int32 [n_major+1]
    values: np.ndarray  # float32 [n_groups]
    value_ptr: np.ndarray  # int32 [n_groups+1]
    indices: np.ndarray  # int32 [nnz]

    @property
    def nnz(self) -> int:
        return int(self.indices.size)

    @property
    def n_groups(self) -> int:
        return int(self.values.size)

    @property
    def n_major(self) -> int:
        return self.shape[0] if self.layout == "vcsr" else self.shape[1]

    @property
    def n_minor(self) -> int:
        return self.shape[1] if self.layout == "vcsr" else self.shape[0]

    def nbytes(self) -> int:
        return (self.major_ptr.nbytes + self.values.nbytes + self.value_ptr.nbytes
                + self.indices.nbytes)


def expanded_csr_nbytes(shape_major: int, nnz: int, val_bytes: int = 4) -> int:
    """Bytes of the equivalent one-value-per-entry CSR/CSC (int32 indices)."""
    return 4 * (shape_major + 1) + (4 + val_bytes) * nnz


# --------------------------------------------------------------------------
# sampling
# --------------------------------------------------------------------------


def sample_columns(rng: np.random.Generator, counts: np.ndarray, n: int):
    """Per row, ``counts[i]`` distinct columns drawn uniformly from ``[0, n)``.

    Draws with replacement and redraws every repeated (row, column) until none
    is left. The procedure treats all column labels alike, so each row's final
    set is a uniform random subset of its size. Returns (rows, cols) sorted by
    (row, col), int64.
    """
    counts = np.minimum(np.asarray(counts, dtype=np.int64), n)
    m = counts.size
    rows = np.repeat(np.arange(m, dtype=np.int64), counts)
    cols = rng.integers(0, n, size=rows.size, dtype=np.int64)
    while True:
        key = rows * n + cols
        order = np.argsort(key, kind="stable")
        ks = key[order]
        dup = np.zeros(ks.size, dtype=bool)
        dup[1:] = ks[1:] == ks[:-1]
        if not dup.any():
            return ks // n, ks % n
        redo = order[dup]
        cols[redo] = rng.integers(0, n, size=redo.size, dtype=np.int64)


def count_values(rng: np.random.Generator, size: int, cap: int) -> np.ndarray:
    """Counts 1 + Geometric(0.3) failures (support 1, 2, ...), capped, as float32.

    numpy's ``geometric(p)`` counts trials up to the first success, so its
    support starts at 1 with P(1) = p, which is "1 + failures".
    """
    return np.minimum(rng.geometric(0.3, size=size), cap).astype(np.float32)


# --------------------------------------------------------------------------
# layout builders (canonical order)
# --------------------------------------------------------------------------


def _order_by_major_value_minor(major, vals, minor):
    # float keys: ascending value; ties (equal values) by ascending minor index.
    return np.lexsort((minor, vals, major))


def build_csr(t: Triplets, by: str = "row") -> Csr:
    """CSR (``by="row"``) or CSC (``by="col"``, returned with the same fields:
    ``row_ptr`` = column pointers, ``col`` = row indices) in ascending index order."""
    m, n = t.shape
    major, minor, n_major = (t.rows, t.cols, m) if by == "row" else (t.cols, t.rows, n)
    order = np.lexsort((minor, major))
    ptr = np.zeros(n_major + 1, dtype=np.int64)
    np.cumsum(np.bincount(major, minlength=n_major), out=ptr[1:])
    return Csr(t.shape, ptr.astype(np.int32), minor[order].astype(np.int32), t.vals[order].copy())


def build_vcs(t: Triplets, layout: str) -> Vcs:
    """Canonical VCSR (``layout="vcsr"``) or VCSC from duplicate-free triplets."""
    m, n = t.shape
    if layout == "vcsr":
        major, minor, n_major = t.rows, t.cols, m
    elif layout == "vcsc":
        major, minor, n_major = t.cols, t.rows, n
    else:
        raise ValueError(layout)
    vals = t.vals.astype(np.float32)
    order = _order_by_major_value_minor(major, vals, minor)
    maj_s, val_s, min_s = major[order], vals[order], minor[order]
    nnz = maj_s.size
    start = np.ones(nnz, dtype=bool)
    if nnz:
        start[1:] = (maj_s[1:] != maj_s[:-1]) | (val_s[1:] != val_s[:-1])
    gstart = np.flatnonzero(start)
    values = val_s[gstart].astype(np.float32)
    value_ptr = np.empty(gstart.size + 1, dtype=np.int64)
    value_ptr[:-1] = gstart
    value_ptr[-1] = nnz
    major_ptr = np.zeros(n_major + 1, dtype=np.int64)
    np.cumsum(np.bincount(maj_s[gstart], minlength=n_major), out=major_ptr[1:])
    return Vcs(layout, t.shape, major_ptr.astype(np.int32), values,
               value_ptr.astype(np.int32), min_s.astype(np.int32))


# --------------------------------------------------------------------------
# dense operands
# --------------------------------------------------------------------------


def dense_normal(rng: np.random.Generator, rows: int, width: int, dtype=np.float32):
    """Row-major ``rows x width`` N(0,1) block."""
    return rng.standard_normal((rows, width)).astype(dtype)


def dense_int(rng: np.random.Generator, rows: int, width: int, lo: int = -4, hi: int = 4,
              dtype=np.float32):
    """Row-major integer-valued block in ``[lo, hi]`` (exact in float32 sums)."""
    return rng.integers(lo, hi + 1, size=(rows, width)).astype(dtype)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------


def count_matrix(m: int, n: int, lam: float, cap: int, rng: np.random.Generator) -> Triplets:
    """Count matrix: Poisson(lam) distinct uniform columns per row, values
    ``min(1 + Geometric(0.3), cap)`` stored as float32."""
    counts = rng.poisson(lam, size=m)
    rows, cols = sample_columns(rng, counts, n)
    return Triplets((m, n), rows, cols, count_values(rng, rows.size, cap))


def config1(seed_salt: int = 0):
    """CSR 2,000 x 500 workload: returns (triplets, csr) in float32."""
    rng = rng_for(1, seed_salt)
    m, n = 2000, 500
    counts = rng.poisson(10, size=m)
    rows, cols = sample_columns(rng, counts, n)
    vals = rng.random(rows.size).astype(np.float32)
    t = Triplets((m, n), rows, cols, vals)
    return t, build_csr(t)


def count_60k(seed_salt: int = 0) -> Triplets:
    """The 60,000 x 2,000 count matrix (~6M entries, values capped at 64)."""
    return count_matrix(60_000, 2_000, 100.0, 64, rng_for(2, seed_salt))


def config2(seed_salt: int = 0):
    t = count_60k(seed_salt)
    return t, build_vcs(t, "vcsr")


def config3(seed_salt: int = 0):
    t = count_60k(seed_salt)
    return t, build_vcs(t, "vcsc")


REGRID_ROWS = 20_000
REGRID_SIGMA = 0.85
REGRID_PLANTED = 8
REGRID_MAX = 4_000


def config4_lengths(rng: np.random.Generator) -> np.ndarray:
    """Row lengths of the regridding operator: lognormal(ln 40, 0.85) rounded and
    clipped to [1, 4000], ~5% of rows emptied, 8 rows planted at 4,000."""
    lengths = np.rint(rng.lognormal(np.log(40.0), REGRID_SIGMA, size=REGRID_ROWS))
    lengths = np.clip(lengths, 1, REGRID_MAX).astype(np.int64)
    empty = rng.choice(REGRID_ROWS, size=REGRID_ROWS // 20, replace=False)
    lengths[empty] = 0
    live = np.flatnonzero(lengths)
    planted = rng.choice(live, size=REGRID_PLANTED, replace=False)
    lengths[planted] = REGRID_MAX
    return lengths


def config4(dtype=np.float64, seed_salt: int = 0):
    """Regridding-shaped CSR forward operator; returns (triplets, csr)."""
    rng = rng_for(4, seed_salt)
    lengths = config4_lengths(rng)
    n = int(round(lengths.sum() / 3.0))
    rows, cols = sample_columns(rng, lengths, n)
    vals = rng.random(rows.size).astype(dtype)
    t = Triplets((REGRID_ROWS, n), rows, cols, vals)
    return t, build_csr(t)


def config5(seed_salt: int = 0) -> Triplets:
    """The 1,000,000 x 20,000 count matrix (~200M entries, values capped at 255)."""
    return count_matrix(1_000_000, 20_000, 200.0, 255, rng_for(5, seed_salt))


def _vcsr_chunk(job):
    """One chunk of count_vcsr_chunked (a process-pool task)."""
    seed, rows_n, n, lam, cap = job
    rng = np.random.Generator(np.random.PCG64(seed))
    counts = rng.poisson(lam, size=rows_n)
    rows, cols = sample_columns(rng, counts, n)
    vals = count_values(rng, rows.size, cap)
    # canonical order inside the chunk: row, value, column (one int64 key)
    key = (rows * (cap + 1) + vals.astype(np.int64)) * n + cols
    order = np.argsort(key, kind="stable")
    rows, cols, vals = rows[order], cols[order], vals[order]
    start = np.ones(rows.size, dtype=bool)
    start[1:] = (rows[1:] != rows[:-1]) | (vals[1:] != vals[:-1])
    gstart = np.flatnonzero(start)
    groups_per_row = np.bincount(rows[gstart], minlength=rows_n)
    return (vals[gstart].astype(np.float32), gstart.astype(np.int64), cols.astype(np.int32),
            groups_per_row)


def count_vcsr_chunked(m: int, n: int, lam: float, cap: int, seed: list, chunk: int = 50_000,
                       workers: int = 1, log=None) -> Vcs:
    """Canonical VCSR of a count matrix built ``chunk`` rows at a time: per row
    Poisson(lam) distinct uniform columns (``sample_columns``) and
    ``min(1 + Geometric(0.3), cap)`` values, grouped by value (ascending value,
    then ascending column). Chunk c draws from its own stream
    PCG64(seed + [c]), so chunks can be built in parallel (``workers``
    processes) with the same result."""
    jobs = [(list(seed) + [c], min(chunk, m - r0), n, lam, cap)
            for c, r0 in enumerate(range(0, m, chunk))]
    if workers > 1:
        import concurrent.futures as cf
        import multiprocessing as mp
        with cf.ProcessPoolExecutor(max_workers=workers,
                                    mp_context=mp.get_context("fork")) as pool:
            parts = list(pool.map(_vcsr_chunk, jobs))
    else:
        parts = [_vcsr_chunk(j) for j in jobs]
    major_ptr = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(np.concatenate([p[3] for p in parts]), out=major_ptr[1:])
    e_off, value_ptr = 0, []
    for vals, gstart, cols, _ in parts:
        value_ptr.append(gstart + e_off)
        e_off += cols.size
    value_ptr.append(np.array([e_off], dtype=np.int64))
    if log:
        log(f"{m} rows, {e_off} entries")
    return Vcs("vcsr", (m, n), major_ptr.astype(np.int32),
               np.concatenate([p[0] for p in parts]),
               np.concatenate(value_ptr).astype(np.int32),
               np.concatenate([p[2] for p in parts]))


def config5_vcsr(seed_salt: int = 0, workers: int = 1, log=None) -> Vcs:
    """The 1,000,000 x 20,000 count matrix (~200M entries, values capped at
    255) as a canonical VCSR, built in chunks of 50,000 rows."""
    return count_vcsr_chunked(1_000_000, 20_000, 200.0, 255, [SEED_BASE + 5, seed_salt],
                              workers=workers, log=log)


def tiny_count(m: int, n: int, density: float, cap: int, rng: np.random.Generator) -> Triplets:
    """Small count matrix for brute-force checks (Bernoulli(density) pattern)."""
    mask = rng.random((m, n)) < density
    rows, cols = np.nonzero(mask)
    vals = count_values(rng, rows.size, cap)
    return Triplets((m, n), rows.astype(np.int64), cols.astype(np.int64), vals)


def tiny_real(m: int, n: int, density: float, rng: np.random.Generator, dtype=np.float64):
    """Small matrix with U(0,1) values for brute-force checks."""
    mask = rng.random((m, n)) < density
    rows, cols = np.nonzero(mask)
    vals = rng.random(rows.size).astype(dtype)
    return Triplets((m, n), rows.astype(np.int64), cols.astype(np.int64), vals)


def shuffled_vcs(L: Vcs, rng: np.random.Generator, n_dup: int = 0) -> Vcs:
    """The same matrix stored in another order the layout allows: the value
    groups of each slice permuted, and the indices of each group permuted.
    With ``n_dup`` > 0, that many entries are also repeated: an index of one
    group is appended to another group of the same slice, so that slice holds
    the index twice, under two values (stored entries add, as a COO sum does;
    this changes the matrix)."""
    n_major = L.major_ptr.size - 1
    G = L.values.size
    sizes = np.diff(L.value_ptr.astype(np.int64))
    slice_of_group = np.repeat(np.arange(n_major), np.diff(L.major_ptr.astype(np.int64)))
    perm = np.lexsort((rng.random(G), slice_of_group))  # new group k = old group perm[k]
    newpos = np.empty(G, dtype=np.int64)
    newpos[perm] = np.arange(G)
    group_of_entry = np.repeat(np.arange(G), sizes)
    ent_group = newpos[group_of_entry]
    ent_idx = L.indices.astype(np.int64)
    ent_key = rng.random(ent_idx.size)
    if n_dup and G:
        # entries whose slice has at least two groups
        n_groups_of_slice = np.diff(L.major_ptr.astype(np.int64))
        ok = np.flatnonzero(n_groups_of_slice[slice_of_group[group_of_entry]] >= 2)
        pick = rng.choice(ok, size=min(n_dup, ok.size), replace=False)
        extra_group, extra_idx = [], []
        for e in pick:
            g = group_of_entry[e]
            s = slice_of_group[g]
            g0, g1 = int(L.major_ptr[s]), int(L.major_ptr[s + 1])
            other = int(rng.integers(g0, g1 - 1))
            other += other >= g  # any group of the slice but g
            extra_group.append(newpos[other])
            extra_idx.append(ent_idx[e])
        ent_group = np.concatenate([ent_group, np.array(extra_group, np.int64)])
        ent_idx = np.concatenate([ent_idx, np.array(extra_idx, np.int64)])
        ent_key = np.concatenate([ent_key, rng.random(len(extra_idx))])
    order = np.lexsort((ent_key, ent_group))
    new_sizes = np.bincount(ent_group, minlength=G)
    value_ptr = np.zeros(G + 1, dtype=np.int64)
    np.cumsum(new_sizes, out=value_ptr[1:])
    return Vcs(L.layout, L.shape, L.major_ptr.copy(), L.values[perm].copy(),
               value_ptr.astype(np.int32), ent_idx[order].astype(np.int32))
