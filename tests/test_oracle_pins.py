"""Pins for the float64 oracle: each test ties it to something other than
itself (brute force, scipy.sparse, closed forms, identities, hand-worked
examples, numbers the vsparse page prints). CPU only."""

import json
import os

import numpy as np
import pytest
import scipy.sparse as sp

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense_of(t: W.Triplets) -> np.ndarray:
    """Dense matrix straight from the generator's triplets (not from any
    compressed layout), float64."""
    A = np.zeros(t.shape, dtype=np.float64)
    np.add.at(A, (t.rows, t.cols), t.vals.astype(np.float64))
    return A


def layouts_of(t: W.Triplets):
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc"),
            "csr": W.build_csr(t)}


def brute(A: np.ndarray, direction: str, B: np.ndarray) -> np.ndarray:
    """Triple loop over the dense matrix (tiny inputs only)."""
    m, n = A.shape
    w = B.shape[1]
    if direction == "AB":
        out = np.zeros((m, w))
        for i in range(m):
            for j in range(n):
                for c in range(w):
                    out[i, c] += A[i, j] * B[j, c]
    else:
        out = np.zeros((n, w))
        for j in range(n):
            for i in range(m):
                for c in range(w):
                    out[j, c] += A[i, j] * B[i, c]
    return out


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(12))
def test_brute_force_integer_exact(orc, seed):
    """Integer counts times integer B: every sum is exact, so all layouts and
    both directions must equal the triple loop exactly."""
    rng = np.random.default_rng(1000 + seed)
    m, n = rng.integers(1, 13, size=2)
    t = W.tiny_count(int(m), int(n), rng.uniform(0.1, 0.9), 64, rng)
    A = dense_of(t)
    w = int(rng.integers(1, 6))
    for direction, rows in (("AB", n), ("BA", m)):
        B = W.dense_int(rng, int(rows), w, dtype=np.float64)
        want = brute(A, direction, B)
        for name, L in layouts_of(t).items():
            got = orc.spmm(L, direction, B)
            assert np.array_equal(got, want), (name, direction)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_real(orc, seed):
    rng = np.random.default_rng(2000 + seed)
    m, n = rng.integers(1, 13, size=2)
    t = W.tiny_real(int(m), int(n), 0.5, rng)
    A = dense_of(t)
    csr = W.build_csr(t)
    for direction, rows in (("AB", n), ("BA", m)):
        B = rng.standard_normal((int(rows), 3))
        want = brute(A, direction, B)
        got = orc.spmm(csr, direction, B)
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_handmade_worked_example(orc):
    """Repeated index in a slice, one value in two groups, an empty group, a
    stored zero, an empty slice: the hand-worked dense matrix."""
    g = json.load(open(os.path.join(GOLDEN, "handmade_vcs.json")))
    v = g["vcsr"]
    A = np.array(g["dense"])
    m, n = g["shape"]
    args = [np.array(v[k], dtype=np.int32) if k != "values" else np.array(v[k], np.float32)
            for k in ("major_ptr", "values", "value_ptr", "indices")]
    eye_n, eye_m = np.eye(n), np.eye(m)
    got = orc.spmm_vcs("vcsr", "AB", (m, n), *args, eye_n)  # A @ I = A
    assert np.array_equal(got, A)
    got = orc.spmm_vcs("vcsr", "BA", (m, n), *args, eye_m)  # (I @ A)^T = A^T
    assert np.array_equal(got, A.T)
    # the regrouped (VCSC) layout worked out by hand
    r = g["regrouped_vcsc"]
    t_mp, t_v, t_vp, t_i = orc.regroup_vcs(n, *args)
    assert t_mp.tolist() == r["major_ptr"]
    assert t_v.tolist() == r["values"]
    assert t_vp.tolist() == r["value_ptr"]
    assert t_i.tolist() == r["indices"]
    got = orc.spmm_vcs("vcsc", "AB", (m, n), t_mp, t_v, t_vp, t_i, eye_n)
    assert np.array_equal(got, A)


# --------------------------------------------------------------- scipy.sparse

def test_scipy_csr_config1(orc):
    t, csr = W.config1()
    rng = np.random.default_rng(7)
    S = sp.csr_matrix((csr.val.astype(np.float64), csr.col, csr.row_ptr), shape=csr.shape)
    B = rng.standard_normal((500, 8))
    np.testing.assert_allclose(orc.spmm(csr, "AB", B), S @ B, rtol=1e-13, atol=1e-12)
    Bt = rng.standard_normal((2000, 8))
    np.testing.assert_allclose(orc.spmm(csr, "BA", Bt), (Bt.T @ S).T, rtol=1e-13, atol=1e-12)
    x = rng.standard_normal((500, 1))
    np.testing.assert_allclose(orc.spmm(csr, "AB", x), S @ x, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_scipy_vcs_medium(orc, layout):
    rng = W.rng_for(99)
    t = W.count_matrix(3000, 400, 20.0, 64, rng)
    L = W.build_vcs(t, layout)
    S = sp.coo_matrix((t.vals.astype(np.float64), (t.rows, t.cols)), shape=t.shape).tocsr()
    B = rng.standard_normal((400, 16))
    np.testing.assert_allclose(orc.spmm(L, "AB", B), S @ B, rtol=1e-12, atol=1e-10)
    Bt = rng.standard_normal((3000, 16))
    np.testing.assert_allclose(orc.spmm(L, "BA", Bt), S.T @ Bt, rtol=1e-12, atol=1e-10)


# ------------------------------------------------------ own expansion, layouts

def test_vcs_equals_its_expansion_exact(orc):
    rng = W.rng_for(98)
    t = W.count_matrix(500, 300, 30.0, 64, rng)
    for layout in ("vcsr", "vcsc"):
        L = W.build_vcs(t, layout)
        ptr, idx, val = orc.expand_vcs(L.major_ptr, L.values, L.value_ptr, L.indices)
        assert ptr[-1] == t.nnz and np.array_equal(idx, L.indices)
        n_in = {"vcsr": {"AB": 300, "BA": 500}, "vcsc": {"AB": 300, "BA": 500}}[layout]
        for direction in ("AB", "BA"):
            B = W.dense_int(rng, n_in[direction], 5, dtype=np.float64)
            got = orc.spmm(L, direction, B)
            if layout == "vcsr":
                want = orc.spmm_csr(direction, t.shape, ptr, idx, val, B)
            else:  # the expansion of a VCSC is a CSC: swap the directions' roles
                other = "BA" if direction == "AB" else "AB"
                want = orc.spmm_csr(other, (t.shape[1], t.shape[0]), ptr, idx, val, B)
            assert np.array_equal(got, want), (layout, direction)


def test_vcsr_equals_vcsc(orc):
    rng = W.rng_for(97)
    t = W.count_matrix(800, 200, 25.0, 64, rng)
    R, C = W.build_vcs(t, "vcsr"), W.build_vcs(t, "vcsc")
    for direction, rows in (("AB", 200), ("BA", 800)):
        B = rng.standard_normal((rows, 7))
        np.testing.assert_allclose(orc.spmm(R, direction, B), orc.spmm(C, direction, B),
                                   rtol=1e-13, atol=1e-11)


# ---------------------------------------------------------------- closed forms

def test_all_ones_row_and_column_sums(orc):
    """A @ 1 = row sums = sum_k values[k] * |group k| (integer arithmetic);
    1 @ A = column sums = bincount of indices weighted by each entry's value."""
    t = W.count_matrix(2000, 300, 40.0, 64, W.rng_for(96))
    R = W.build_vcs(t, "vcsr")
    sizes = np.diff(R.value_ptr.astype(np.int64))
    gv = R.values.astype(np.int64) * sizes
    row_sums = np.add.reduceat(np.concatenate([gv, [0]]), R.major_ptr[:-1].astype(np.int64))
    row_sums[np.diff(R.major_ptr) == 0] = 0
    got = orc.spmm(R, "AB", np.ones((300, 2)))
    assert np.array_equal(got[:, 0], row_sums.astype(np.float64))
    assert np.array_equal(got[:, 1], row_sums.astype(np.float64))
    per_entry = np.repeat(R.values.astype(np.int64), sizes)
    col_sums = np.bincount(R.indices, weights=per_entry, minlength=300)
    got = orc.spmm(R, "BA", np.ones((2000, 1)))
    assert np.array_equal(got[:, 0], col_sums)
    C = W.build_vcs(t, "vcsc")
    assert np.array_equal(orc.spmm(C, "AB", np.ones((300, 1)))[:, 0], row_sums.astype(np.float64))
    assert np.array_equal(orc.spmm(C, "BA", np.ones((2000, 1)))[:, 0], col_sums)


@pytest.mark.parametrize("kind", ["vcsr", "vcsc", "csr"])
def test_dot_product_identity(orc, kind):
    """<A x, y> = <x, A^T y>: ties the AB walk to the BA walk."""
    rng = np.random.default_rng(5)
    t = W.count_matrix(700, 250, 30.0, 64, W.rng_for(95))
    L = layouts_of(t)[kind]
    x = rng.standard_normal((250, 1))
    y = rng.standard_normal((700, 1))
    lhs = float(y[:, 0] @ orc.spmm(L, "AB", x)[:, 0])
    rhs = float(x[:, 0] @ orc.spmm(L, "BA", y)[:, 0])
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1.0)


# ------------------------------------------------------------------ transpose

@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_transpose_equals_scipy_tocsc(orc, dtype):
    """scipy's CSR->CSC conversion is a stable counting sort too: the arrays
    must agree bit for bit, and so must the transpose of the transpose."""
    t, csr = W.config1()
    val = csr.val.astype(dtype)
    S = sp.csr_matrix((val, csr.col, csr.row_ptr), shape=csr.shape)
    C = S.tocsc()
    tp, ti, tv = orc.transpose_csr(500, csr.row_ptr, csr.col, val)
    assert np.array_equal(tp, C.indptr) and np.array_equal(ti, C.indices)
    assert tv.dtype == dtype and np.array_equal(tv.view(np.uint8), C.data.view(np.uint8))
    bp, bi, bv = orc.transpose_csr(2000, tp, ti, tv)
    assert np.array_equal(bp, csr.row_ptr) and np.array_equal(bi, csr.col)
    assert np.array_equal(bv.view(np.uint8), val.view(np.uint8))


def test_transpose_regridding_operator(orc):
    t, csr = W.config4(np.float64)
    n = t.shape[1]
    tp, ti, tv = orc.transpose_csr(n, csr.row_ptr, csr.col, csr.val)
    S = sp.csr_matrix((csr.val, csr.col, csr.row_ptr), shape=csr.shape).tocsc()
    assert np.array_equal(tp, S.indptr) and np.array_equal(ti, S.indices)
    assert np.array_equal(tv, S.data)
    counts = np.diff(tp)
    assert 2.5 < counts.mean() < 3.5  # ~3 entries per transposed row
    assert 0.03 < (counts == 0).mean() < 0.08  # Poisson(3): ~5% empty


def test_transpose_unsorted_and_repeated(orc):
    """Stored order is kept within each source slice, repeats included."""
    ptr = np.array([0, 3, 3, 5], dtype=np.int32)
    idx = np.array([2, 0, 2, 1, 2], dtype=np.int32)
    val = np.array([1.0, 2.0, 3.0, 4.0, 5.0])
    tp, ti, tv = orc.transpose_csr(3, ptr, idx, val)
    assert tp.tolist() == [0, 1, 2, 5]
    assert ti.tolist() == [0, 2, 0, 0, 2]
    assert tv.tolist() == [2.0, 4.0, 1.0, 3.0, 5.0]


# ------------------------------------------------------------------- regroup

def test_regroup_matches_generator_layouts(orc):
    """Regrouping the generator's canonical VCSR gives its canonical VCSC (two
    independent constructions), and back again."""
    t = W.count_matrix(1500, 250, 30.0, 64, W.rng_for(94))
    R, C = W.build_vcs(t, "vcsr"), W.build_vcs(t, "vcsc")
    mp, v, vp, ix = orc.regroup_vcs(250, R.major_ptr, R.values, R.value_ptr, R.indices)
    assert np.array_equal(mp, C.major_ptr) and np.array_equal(vp, C.value_ptr)
    assert np.array_equal(v, C.values) and np.array_equal(ix, C.indices)
    mp, v, vp, ix = orc.regroup_vcs(1500, C.major_ptr, C.values, C.value_ptr, C.indices)
    assert np.array_equal(mp, R.major_ptr) and np.array_equal(vp, R.value_ptr)
    assert np.array_equal(v, R.values) and np.array_equal(ix, R.indices)


def test_regroup_value_order_total():
    """-0 sorts before +0 and they stay separate groups; negatives ascend."""
    import oracle as orc
    major_ptr = np.array([0, 4], dtype=np.int32)
    values = np.array([0.0, -0.0, 3.5, -2.0], dtype=np.float32)
    value_ptr = np.array([0, 1, 2, 3, 4], dtype=np.int32)
    indices = np.array([0, 0, 0, 0], dtype=np.int32)
    mp, v, vp, ix = orc.regroup_vcs(1, major_ptr, values, value_ptr, indices)
    assert mp.tolist() == [0, 4]
    assert [float(x) for x in v] == [-2.0, -0.0, 0.0, 3.5]
    assert np.signbit(v[1]) and not np.signbit(v[2])


# -------------------------------------------------------------- special cases

def test_special_cases(orc):
    # empty slices give zero rows; one entry scales one row of B
    mp = np.array([0, 0, 1, 1], dtype=np.int32)
    vals = np.array([3.0], dtype=np.float32)
    vp = np.array([0, 1], dtype=np.int32)
    ix = np.array([2], dtype=np.int32)
    B = np.arange(12, dtype=np.float64).reshape(4, 3)
    out = orc.spmm_vcs("vcsr", "AB", (3, 4), mp, vals, vp, ix, B)
    assert np.array_equal(out, np.array([[0, 0, 0], 3 * B[2], [0, 0, 0]]))
    # nnz = 0: all zeros
    z = orc.spmm_vcs("vcsr", "AB", (3, 4), np.zeros(4, np.int32), np.zeros(0, np.float32),
                     np.zeros(1, np.int32), np.zeros(0, np.int32), B)
    assert z.shape == (3, 3) and not z.any()
    # width 0
    z = orc.spmm_vcs("vcsr", "AB", (3, 4), mp, vals, vp, ix, np.zeros((4, 0)))
    assert z.shape == (3, 0)
    # m = 0 and n = 0
    z = orc.spmm_csr("AB", (0, 5), np.zeros(1, np.int32), np.zeros(0, np.int32),
                     np.zeros(0), np.ones((5, 2)))
    assert z.shape == (0, 2)
    z = orc.spmm_csr("BA", (0, 5), np.zeros(1, np.int32), np.zeros(0, np.int32),
                     np.zeros(0), np.ones((0, 2)))
    assert z.shape == (5, 2) and not z.any()
    z = orc.spmm_csr("AB", (3, 0), np.zeros(4, np.int32), np.zeros(0, np.int32),
                     np.zeros(0), np.ones((0, 2)))
    assert z.shape == (3, 2) and not z.any()


def test_want_subset_matches_full(orc):
    t = W.count_matrix(900, 120, 20.0, 64, W.rng_for(93))
    rng = np.random.default_rng(3)
    for layout in ("vcsr", "vcsc"):
        L = W.build_vcs(t, layout)
        for direction, rows, n_out in (("AB", 120, 900), ("BA", 900, 120)):
            B = rng.standard_normal((rows, 4))
            full = orc.spmm(L, direction, B)
            pick = rng.choice(n_out, size=17, replace=False)
            part = orc.spmm(L, direction, B, want=pick)
            assert np.array_equal(part[pick], full[pick])
            rest = np.setdiff1d(np.arange(n_out), pick)
            assert not part[rest].any()


# ----------------------------------------------------------------- validation

def test_validate(orc):
    ok = orc.validate_vcs(2, 3, np.array([0, 1, 2], np.int32), np.array([0, 2, 3], np.int32),
                          np.array([0, 2, 1], np.int32))
    assert ok == 0
    assert orc.validate_vcs(2, 3, np.array([1, 1, 2], np.int32), np.array([0, 2, 3], np.int32),
                            np.array([0, 2, 1], np.int32)) == 1
    assert orc.validate_vcs(2, 3, np.array([0, 2, 1], np.int32), np.array([0, 2, 3], np.int32),
                            np.array([0, 2, 1], np.int32)) == 2
    assert orc.validate_vcs(2, 3, np.array([0, 1, 2], np.int32), np.array([0, 2, 4], np.int32),
                            np.array([0, 2, 1], np.int32)) == 3
    assert orc.validate_vcs(2, 3, np.array([0, 1, 2], np.int32), np.array([0, 2, 3], np.int32),
                            np.array([0, 3, 1], np.int32)) == 4
    assert orc.validate_csr(2, 3, np.array([0, 2, 3], np.int32), np.array([0, -1, 1], np.int32)) == 4
    assert orc.validate_csr(2, 3, np.array([0, 2, 3], np.int32), np.array([0, 1, 2], np.int32)) == 0


# --------------------------------------------------- numbers the page prints

def test_footprint_ratios_printed_on_page():
    """The vsparse page's benchmark table gives device bytes vs CSR of 0.62
    (VCSR) and 0.51 (VCSC) at 60k x 2k, 6M nonzeros; the generator's reading of
    the count-matrix workload must reproduce both to two decimals."""
    g = json.load(open(os.path.join(GOLDEN, "vcs_footprint_ratios.json")))
    t = W.count_60k()
    assert 5.9e6 < t.nnz < 6.1e6
    R, C = W.build_vcs(t, "vcsr"), W.build_vcs(t, "vcsc")
    csr = W.expanded_csr_nbytes(60_000, t.nnz)
    csc = W.expanded_csr_nbytes(2_000, t.nnz)
    assert round(R.nbytes() / csr, 2) == g["printed_to_two_decimals"]["vcsr"]
    assert round(C.nbytes() / csc, 2) == g["printed_to_two_decimals"]["vcsc"]


@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_expand_formats_match_scipy(orc, layout):
    """VCS -> CSR / CSC of A, index-sorted: on a matrix without repeated
    (row, column) pairs the sorted expansion is unique, and equals scipy's
    (csr_matrix(...).sort_indices() in the layout's own format, .tocsc() /
    .tocsr() of the stored-order expansion in the other)."""
    t = W.count_matrix(300, 170, 12.0, 9, W.rng_for(71))
    L = W.build_vcs(t, layout)
    m, n = t.shape
    own = "csr" if layout == "vcsr" else "csc"
    other = "csc" if own == "csr" else "csr"
    ptr, idx, val = orc.expand_vcs(L.major_ptr, L.values, L.value_ptr, L.indices)
    M = (sp.csr_matrix if own == "csr" else sp.csc_matrix)((val, idx, ptr), shape=(m, n))
    S = M.copy()
    S.sort_indices()
    got = orc.expand_vcs_format(layout, (m, n), L.major_ptr, L.values, L.value_ptr, L.indices,
                                own, True)
    assert np.array_equal(got[0], S.indptr) and np.array_equal(got[1], S.indices)
    assert np.array_equal(got[2], S.data)
    T = M.tocsc() if other == "csc" else M.tocsr()
    T.sort_indices()
    got = orc.expand_vcs_format(layout, (m, n), L.major_ptr, L.values, L.value_ptr, L.indices,
                                other, True)
    assert np.array_equal(got[0], T.indptr) and np.array_equal(got[1], T.indices)
    assert np.array_equal(got[2], T.data)
    # unsorted, own format: the stored order itself
    got = orc.expand_vcs_format(layout, (m, n), L.major_ptr, L.values, L.value_ptr, L.indices,
                                own, False)
    assert np.array_equal(got[1], idx) and np.array_equal(got[2], val)


def test_expand_sorted_repeated_indices(orc):
    """Worked by hand: a 2 x 6 VCSR whose row 0 holds index 1 in two groups.
    Row 0: value 2 at [5, 1], value 3 at [1]; row 1: value 7 at [4, 0].
    Stored order: (5, 2) (1, 2) (1, 3) | (4, 7) (0, 7). Sorted by index, equal
    indices in stored order: (1, 2) (1, 3) (5, 2) | (0, 7) (4, 7). The CSC: column
    0: (1, 7); column 1: (0, 2) (0, 3); column 4: (1, 7); column 5: (0, 2)."""
    major_ptr = np.array([0, 2, 3], np.int32)
    values = np.array([2, 3, 7], np.float32)
    value_ptr = np.array([0, 2, 3, 5], np.int32)
    indices = np.array([5, 1, 1, 4, 0], np.int32)
    ptr, idx, val = orc.expand_vcs_format("vcsr", (2, 6), major_ptr, values, value_ptr, indices,
                                          "csr", True)
    assert ptr.tolist() == [0, 3, 5]
    assert idx.tolist() == [1, 1, 5, 0, 4] and val.tolist() == [2, 3, 2, 7, 7]
    ptr, idx, val = orc.expand_vcs_format("vcsr", (2, 6), major_ptr, values, value_ptr, indices,
                                          "csc", True)
    assert ptr.tolist() == [0, 1, 3, 3, 3, 4, 5]
    assert idx.tolist() == [1, 0, 0, 1, 0] and val.tolist() == [7, 2, 3, 7, 2]


# ------------------------------------------------------------ the comparator

def test_max_rel_error_hand_computed(orc):
    """The float parity criterion on arrays worked by hand: the largest
    |got - ref| / S over outputs with S > 0 (errors 0, 0.5, 1.0 over scales
    1, 1, 4 give 0, 0.5, 0.25: the maximum is 0.5, the mean would be 0.25)."""
    got = np.array([1.0, 2.0, 3.0])
    ref = np.array([1.0, 2.5, 2.0])
    scale = np.array([1.0, 1.0, 4.0])
    rel, zeros_ok = orc.max_rel_error(got, ref, scale)
    assert rel == 0.5 and zeros_ok


def test_max_rel_error_cancellation(orc):
    """A cancelled output (reference 0, |A||B| = 2) judged against S, not
    against |ref|: an error of 1e-7 is 5e-8 relative, not infinite."""
    rel, zeros_ok = orc.max_rel_error(np.array([1e-7, 3.0]), np.array([0.0, 3.0]),
                                      np.array([2.0, 3.0]))
    assert rel == pytest.approx(5e-8, rel=1e-12) and zeros_ok


def test_max_rel_error_zero_scale(orc):
    """Outputs whose |A||B| is 0 must be exactly 0: any nonzero value there
    fails, however small, and does not enter the relative error (which comes
    from the S > 0 outputs alone)."""
    scale = np.array([0.0, 2.0, 0.0])
    ref = np.array([0.0, 1.0, 0.0])
    rel, zeros_ok = orc.max_rel_error(np.array([0.0, 3.0, 0.0]), ref, scale)
    assert rel == 1.0 and zeros_ok
    rel, zeros_ok = orc.max_rel_error(np.array([1e-30, 1.0, 0.0]), ref, scale)
    assert rel == 0.0 and not zeros_ok
    rel, zeros_ok = orc.max_rel_error(np.array([0.0, 1.0, -0.0]), ref, scale)
    assert rel == 0.0 and zeros_ok  # -0 equals 0
    rel, zeros_ok = orc.max_rel_error(np.zeros(3), np.zeros(3), np.zeros(3))
    assert rel == 0.0 and zeros_ok


def _signed_hand_matrix():
    """A = [[1, 2], [1, -2]] as triplets, B = [[1, 3], [-1, 1]] (hand-picked
    so that |A||B|, |A|B and A|B| all differ): A B = [[-1, 5], [3, 1]],
    |A||B| = [[3, 5], [3, 5]]; for B A (B given transposed as Bt = [[1, -1],
    [3, 1]] over the rows of A): (B A)^T = [[4, 0], [-4, -4]] and
    |A|^T |Bt| = [[4, 2], [8, 4]]."""
    t = W.Triplets((2, 2), np.array([0, 0, 1, 1]), np.array([0, 1, 0, 1]),
                   np.array([1.0, 2.0, 1.0, -2.0], dtype=np.float32))
    B = np.array([[1.0, 3.0], [-1.0, 1.0]])
    Bt = np.array([[1.0, -1.0], [3.0, 1.0]])
    return t, B, Bt


@pytest.mark.parametrize("kind", ["vcsr", "vcsc", "csr"])
def test_abs_scale_hand_computed(orc, kind):
    """S = |A| |B| in the output's layout, worked by hand (a dropped absolute
    value on A or on B changes some entry)."""
    t, B, Bt = _signed_hand_matrix()
    L = layouts_of(t)[kind]
    assert np.array_equal(orc.spmm(L, "AB", B), [[-1.0, 5.0], [3.0, 1.0]])
    assert np.array_equal(orc.abs_scale(L, "AB", B), [[3.0, 5.0], [3.0, 5.0]])
    assert np.array_equal(orc.spmm(L, "BA", Bt), [[4.0, 0.0], [-4.0, -4.0]])
    assert np.array_equal(orc.abs_scale(L, "BA", Bt), [[4.0, 2.0], [8.0, 4.0]])


# ---------------------------------------------------------- threaded mode

@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threaded_integer_exact(orc, threads):
    """The timed mode on integer data: every partial sum is exact, so each
    layout and direction equals the triple loop exactly at any thread count
    (more threads than slices included)."""
    for seed in range(4):
        rng = np.random.default_rng(3000 + seed)
        m, n = (int(x) for x in rng.integers(1, 30, size=2))
        t = W.tiny_count(m, n, rng.uniform(0.1, 0.9), 64, rng)
        A = dense_of(t)
        for direction, rows in (("AB", n), ("BA", m)):
            B = W.dense_int(rng, rows, 3, dtype=np.float64)
            want = brute(A, direction, B)
            for name, L in layouts_of(t).items():
                got = orc.spmm_threaded(L, direction, B, threads)
                assert np.array_equal(got, want), (name, direction, threads)


@pytest.mark.parametrize("threads", [2, 7])
def test_threaded_real_data(orc, threads):
    """Real data: where the output rows are the slices each row is summed by
    one thread in the sequential order (bitwise equal); elsewhere the private
    outputs regroup the additions, within 1e-13 of |A||B|."""
    rng = W.rng_for(96)
    t = W.count_matrix(1500, 300, 20.0, 64, rng)
    t = W.Triplets(t.shape, t.rows, t.cols, (t.vals * 0.37).astype(np.float32))
    for name, L in layouts_of(t).items():
        for direction, rows in (("AB", 300), ("BA", 1500)):
            B = rng.standard_normal((rows, 5))
            seq = orc.spmm(L, direction, B)
            got = orc.spmm_threaded(L, direction, B, threads)
            rows_are_slices = (name != "vcsc") == (direction == "AB")
            if rows_are_slices:
                assert np.array_equal(got, seq), (name, direction)
            else:
                rel, zeros_ok = orc.max_rel_error(got, seq, orc.abs_scale(L, direction, B))
                assert rel <= 1e-13 and zeros_ok, (name, direction, rel)


# ------------------------------------------------------ normalized view

@pytest.mark.parametrize("seed", range(8))
def test_view_brute_force_integer_exact(orc, seed):
    """The "scale" view's product equals the triple loop over the dense
    matrix with every entry multiplied by its row's and its column's
    statistic (integer statistics, zeros and negatives included, so every
    sum is exact): all layouts, both directions."""
    rng = np.random.default_rng(3000 + seed)
    m, n = (int(x) for x in rng.integers(1, 11, size=2))
    t = W.tiny_count(m, n, rng.uniform(0.2, 0.9), 16, rng)
    r = rng.integers(-3, 4, size=m).astype(np.float64)
    c = rng.integers(-3, 4, size=n).astype(np.float64)
    G = dense_of(t) * r[:, None] * c[None, :]
    w = int(rng.integers(1, 5))
    for direction, rows in (("AB", n), ("BA", m)):
        B = W.dense_int(rng, rows, w, dtype=np.float64)
        want = brute(G, direction, B)
        for name, L in layouts_of(t).items():
            assert np.array_equal(orc.spmm_view(L, direction, B, r, c), want), (name, direction)


def test_view_hand_worked(orc):
    """A = [[1, 2], [1, -2]], row statistics (2, -1), column statistics (3,
    0.5): the transformed entries are [[6, 2], [-3, 1]]. By hand: G B =
    [[4, 20], [-4, -8]], |G||B| = [[8, 20], [4, 10]]; for B G (B given
    transposed): [[-3, -9], [5, -1]], with scale [[15, 9], [5, 3]]."""
    t, B, Bt = _signed_hand_matrix()
    r, c = np.array([2.0, -1.0]), np.array([3.0, 0.5])
    for name, L in layouts_of(t).items():
        assert np.array_equal(orc.spmm_view(L, "AB", B, r, c), [[4.0, 20.0], [-4.0, -8.0]]), name
        assert np.array_equal(orc.abs_scale_view(L, "AB", B, r, c), [[8.0, 20.0], [4.0, 10.0]])
        assert np.array_equal(orc.spmm_view(L, "BA", Bt, r, c), [[-3.0, -9.0], [5.0, -1.0]]), name
        assert np.array_equal(orc.abs_scale_view(L, "BA", Bt, r, c), [[15.0, 9.0], [5.0, 3.0]])


def test_view_unit_statistics_is_the_product(orc):
    """Statistics of 1 leave every value as stored: the view's product is the
    plain product, bit for bit, on real data."""
    rng = np.random.default_rng(41)
    t = W.tiny_real(9, 7, 0.5, rng)
    for name, L in layouts_of(t).items():
        for direction, rows in (("AB", 7), ("BA", 9)):
            B = rng.standard_normal((rows, 3))
            got = orc.spmm_view(L, direction, B, np.ones(9), np.ones(7))
            assert np.array_equal(got, orc.spmm(L, direction, B)), (name, direction)


# ------------------------------------------------------------- assembly

def _elements(rng, n_elem, n_out, n_in, max_nnz):
    """Random elements with integer weights (repeated coordinates and empty
    elements included) and each element's dense matrix."""
    sizes = rng.integers(0, max_nnz + 1, n_elem)
    sizes[rng.random(n_elem) < 0.2] = 0
    elem_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    nnz = int(elem_ptr[-1])
    out_idx = rng.integers(0, n_out, nnz).astype(np.int32)
    in_idx = rng.integers(0, n_in, nnz).astype(np.int32)
    weight = rng.integers(1, 10, nnz).astype(np.float64)
    dense = np.zeros((n_elem, n_out, n_in))
    for e in range(n_elem):
        for p in range(elem_ptr[e], elem_ptr[e + 1]):
            dense[e, out_idx[p], in_idx[p]] += weight[p]
    return elem_ptr, out_idx, in_idx, weight, dense


def _role_dense(role, dense):
    """The operator each role of the regridding page's table describes,
    written with dense blocks: own = block diagonal, shared = elements
    stacked over one input, summed = elements side by side, sum_of = their
    sum."""
    import scipy.linalg
    if role == "own":
        return scipy.linalg.block_diag(*dense)
    if role == "shared":
        return np.vstack(list(dense))
    if role == "summed":
        return np.hstack(list(dense))
    return dense.sum(axis=0)


def _csr_dense(shape, row_ptr, col, val):
    A = np.zeros(shape)
    for r in range(shape[0]):
        for p in range(row_ptr[r], row_ptr[r + 1]):
            A[r, col[p]] += val[p]
    return A


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("role", ["own", "shared", "summed", "sum_of"])
def test_assembly_is_the_role_operator(orc, role, seed):
    rng = np.random.default_rng(4000 + seed)
    n_elem, n_out, n_in = (int(x) for x in rng.integers(1, 6, size=3))
    ep, oi, ii, wt, dense = _elements(rng, n_elem, n_out, n_in, 7)
    row_ptr, col, val = orc.assemble_csr(role, n_elem, n_out, n_in, ep, oi, ii, wt)
    shape = orc.assembled_shape(role, n_elem, n_out, n_in)
    assert shape == _role_dense(role, dense).shape
    assert np.array_equal(_csr_dense(shape, row_ptr, col, val), _role_dense(role, dense))


@pytest.mark.parametrize("role", ["own", "shared", "summed", "sum_of"])
def test_assembly_rows_keep_element_order(orc, role):
    """Weights that number the entries (their position in the element
    lists): every row must list them in increasing order, so by element and
    then as given; and the row counts are the rows' entry counts."""
    rng = np.random.default_rng(77)
    n_elem, n_out, n_in = 5, 4, 3
    ep, oi, ii, _, _ = _elements(rng, n_elem, n_out, n_in, 9)
    nnz = int(ep[-1])
    tag = np.arange(nnz, dtype=np.float64)
    row_ptr, col, val = orc.assemble_csr(role, n_elem, n_out, n_in, ep, oi, ii, tag)
    for r in range(row_ptr.size - 1):
        assert np.all(np.diff(val[row_ptr[r]:row_ptr[r + 1]]) > 0), r
    elem = np.repeat(np.arange(n_elem), np.diff(ep))
    rows = elem * n_out + oi if role in ("own", "shared") else oi
    assert np.array_equal(np.diff(row_ptr), np.bincount(rows, minlength=row_ptr.size - 1))


def test_scaled_transpose_hand_worked(orc):
    """A = [[1, 2], [0, 3]] with entry factors 10, 100, 1000 (stored order):
    the scaled transpose holds [[10, 0], [200, 3000]] with .T's indices."""
    ptr, idx = np.array([0, 2, 3], np.int32), np.array([0, 1, 1], np.int32)
    val = np.array([1.0, 2.0, 3.0], np.float32)
    t = orc.transpose_csr_scaled(2, ptr, idx, val, np.array([10.0, 100.0, 1000.0], np.float32))
    assert t[0].tolist() == [0, 1, 3] and t[1].tolist() == [0, 0, 1]
    assert t[2].tolist() == [10.0, 200.0, 3000.0]
    plain = orc.transpose_csr(2, ptr, idx, val)
    assert np.array_equal(plain[0], t[0]) and np.array_equal(plain[1], t[1])


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_scaled_transpose_brute_force(orc, dtype):
    """Against the dense transpose of the matrix whose entries are scaled
    (numpy's .T); unit factors give the exact transpose bit for bit."""
    rng = np.random.default_rng(5)
    t = W.tiny_real(11, 7, 0.4, rng, dtype=dtype)
    C = W.build_csr(t)
    f = rng.uniform(0.5, 2.0, C.nnz).astype(dtype)
    tp, ti, tv = orc.transpose_csr_scaled(7, C.row_ptr, C.col, C.val, f)
    D = np.zeros(C.shape)
    for r in range(C.shape[0]):
        for p in range(C.row_ptr[r], C.row_ptr[r + 1]):
            D[r, C.col[p]] += float(dtype(float(C.val[p]) * float(f[p])))
    assert np.array_equal(_csr_dense((7, 11), tp, ti, tv.astype(np.float64)), D.T)
    ones = orc.transpose_csr_scaled(7, C.row_ptr, C.col, C.val, np.ones(C.nnz, dtype))
    plain = orc.transpose_csr(7, C.row_ptr, C.col, C.val)
    for a, b in zip(ones, plain):
        assert np.array_equal(a, b)
