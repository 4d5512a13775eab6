/*
 * Float64 CPU oracle for the sparse x dense product over CSR and the
 * value-grouped VCSR/VCSC layouts.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product library
 * never calls it, and the two share no code: this file is written from the
 * definitions alone, plainly and without any blocking, fusion or reordering.
 *
 * Sources (the pages these definitions come from):
 *  - vsparse, "Add CUDA transfer and matmul kernels for the normalized views",
 *    section "The layout stays compressed" (the VCS arrays major_ptr, values,
 *    value_ptr, indices) and section "The kernels" (the four directions: the
 *    output's disjoint axis is the major axis or it is not).
 *  - regridding, "Regridder", section "How it is built" (a CSR operator built
 *    by a two-pass counting sort in which each row keeps its entries in
 *    source order; the exact transpose, section "API"; the roles of the
 *    orthogonal axis, the table in section "API").
 *
 * Semantics (COO sum): a stored entry (r, c, v) adds v to A[r][c]. Repeated
 * coordinates, empty groups and explicit zeros are all legal; repeats sum.
 *   VCSR: slice i is row i; entry p of group k is (i, indices[p], values[k]).
 *   VCSC: slice j is column j; entry p of group k is (indices[p], j, values[k]).
 *   CSR : slice i is row i; entry p is (i, col[p], val[p]).
 *
 * Products, with dense operands row-major and the width contiguous:
 *   AB: out[r][0:w] = sum over entries (r, c, v) of v * B[c][0:w]
 *       (B is n x w, out is m x w; out = A @ B).
 *   BA: out[c][0:w] = sum over entries (r, c, v) of v * Bt[r][0:w]
 *       (Bt is m x w holding B transposed, out is n x w holding (B @ A)
 *       transposed).
 * All arithmetic is in double. Float32 inputs are widened by the caller, which
 * is exact, so every single product v * b is exact and only the additions
 * round.
 *
 * The threaded mode (orc_spmm_*_threaded) is the timed CPU baseline: the
 * same loops with the slices split over host threads, private float64
 * outputs where the output rows are not the slices (vsparse, "The kernels").
 * The parity checks use the sequential functions.
 *
 * Parity pins: see the tests that exercise this file (brute-force dense
 * products, scipy.sparse, the all-ones closed forms, the dot-product identity,
 * the transpose involution, page 1's footprint ratios; the threaded mode
 * against the sequential one).
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_PTR0 1       /* pointer array does not start at 0 */
#define ORC_BAD_MONOTONE 2   /* pointer array decreases */
#define ORC_BAD_LAST 3       /* last pointer differs from the array length */
#define ORC_BAD_INDEX 4      /* minor index outside [0, n_minor) */
#define ORC_BAD_DIM 5        /* negative extent */

/* ---------------------------------------------------------------- validation */

static int check_ptr(int64_t n, const int32_t *ptr, int64_t count) {
    if (ptr[0] != 0) return ORC_BAD_PTR0;
    for (int64_t i = 0; i < n; ++i)
        if (ptr[i + 1] < ptr[i]) return ORC_BAD_MONOTONE;
    if ((int64_t)ptr[n] != count) return ORC_BAD_LAST;
    return ORC_OK;
}

static int check_idx(int64_t nnz, const int32_t *idx, int64_t n_minor) {
    for (int64_t p = 0; p < nnz; ++p)
        if (idx[p] < 0 || (int64_t)idx[p] >= n_minor) return ORC_BAD_INDEX;
    return ORC_OK;
}

int orc_validate_csr(int64_t n_major, int64_t n_minor, int64_t nnz,
                     const int32_t *ptr, const int32_t *idx) {
    if (n_major < 0 || n_minor < 0 || nnz < 0) return ORC_BAD_DIM;
    int st = check_ptr(n_major, ptr, nnz);
    if (st) return st;
    return check_idx(nnz, idx, n_minor);
}

int orc_validate_vcs(int64_t n_major, int64_t n_minor, int64_t n_groups, int64_t nnz,
                     const int32_t *major_ptr, const int32_t *value_ptr,
                     const int32_t *indices) {
    if (n_major < 0 || n_minor < 0 || n_groups < 0 || nnz < 0) return ORC_BAD_DIM;
    int st = check_ptr(n_major, major_ptr, n_groups);
    if (st) return st;
    st = check_ptr(n_groups, value_ptr, nnz);
    if (st) return st;
    return check_idx(nnz, indices, n_minor);
}

/* ------------------------------------------------------------------ products */

/* Add v * src[0:w] to dst[0:w]. */
static void axpy(double v, const double *src, double *dst, int64_t w) {
    for (int64_t c = 0; c < w; ++c) dst[c] += v * src[c];
}

/* One stored entry (r, c, v) of A contributes to the product. want, when not
 * NULL, selects the output rows to compute (others are left untouched). */
static void entry(int dir, int64_t r, int64_t c, double v, const double *B, int64_t w,
                  double *out, const uint8_t *want) {
    if (dir == 0) { /* AB: out[r] += v * B[c] */
        if (!want || want[r]) axpy(v, B + c * w, out + r * w, w);
    } else { /* BA: out[c] += v * Bt[r] */
        if (!want || want[c]) axpy(v, B + r * w, out + c * w, w);
    }
}

/* layout: 1 = VCSR, 2 = VCSC. dir: 0 = A@B, 1 = B@A. out must be zeroed by the
 * caller (m x w for AB, n x w for BA). */
void orc_spmm_vcs(int layout, int dir, int64_t n_major,
                  const int32_t *major_ptr, const double *values,
                  const int32_t *value_ptr, const int32_t *indices,
                  const double *B, int64_t w, double *out, const uint8_t *want) {
    for (int64_t s = 0; s < n_major; ++s)
        for (int64_t k = major_ptr[s]; k < major_ptr[s + 1]; ++k)
            for (int64_t p = value_ptr[k]; p < value_ptr[k + 1]; ++p) {
                int64_t r = layout == 1 ? s : indices[p];
                int64_t c = layout == 1 ? indices[p] : s;
                entry(dir, r, c, values[k], B, w, out, want);
            }
}

/* CSR with rows as the major axis. */
void orc_spmm_csr(int dir, int64_t n_rows, const int32_t *row_ptr, const int32_t *col,
                  const double *val, const double *B, int64_t w, double *out,
                  const uint8_t *want) {
    for (int64_t r = 0; r < n_rows; ++r)
        for (int64_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p)
            entry(dir, r, col[p], val[p], B, w, out, want);
}

/* --------------------------------------------- products, normalized view */

/* The product of a normalized view (vsparse page, introduction: a view
 * transforms each stored value on the fly; section "The layout stays
 * compressed": it carries O(n_rows + n_cols) statistics). The page does not
 * give its transforms; this is the library's one closed form: a stored entry
 * (r, c, v) contributes g = v * row_stat[r] * col_stat[c] in place of v.
 * Otherwise as orc_spmm_vcs and orc_spmm_csr (out zeroed by the caller). */
void orc_spmm_vcs_scaled(int layout, int dir, int64_t n_major,
                         const int32_t *major_ptr, const double *values,
                         const int32_t *value_ptr, const int32_t *indices,
                         const double *row_stat, const double *col_stat,
                         const double *B, int64_t w, double *out) {
    for (int64_t s = 0; s < n_major; ++s)
        for (int64_t k = major_ptr[s]; k < major_ptr[s + 1]; ++k)
            for (int64_t p = value_ptr[k]; p < value_ptr[k + 1]; ++p) {
                int64_t r = layout == 1 ? s : indices[p];
                int64_t c = layout == 1 ? indices[p] : s;
                double g = values[k] * row_stat[r] * col_stat[c];
                entry(dir, r, c, g, B, w, out, NULL);
            }
}

void orc_spmm_csr_scaled(int dir, int64_t n_rows, const int32_t *row_ptr, const int32_t *col,
                         const double *val, const double *row_stat, const double *col_stat,
                         const double *B, int64_t w, double *out) {
    for (int64_t r = 0; r < n_rows; ++r)
        for (int64_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p) {
            double g = val[p] * row_stat[r] * col_stat[col[p]];
            entry(dir, r, col[p], g, B, w, out, NULL);
        }
}

/* ------------------------------------------------- products, threaded mode */

/* The timed mode of the same products, on n_threads host threads (OpenMP).
 * It follows the host product of vsparse, section "The kernels": the major
 * slices are split over the threads, and in a direction whose output rows
 * are not the slices each thread adds into an accumulator of its own.
 *  - Output rows are the slices (VCSR or CSR times B, B times VCSC): thread t
 *    walks the t-th of n_threads contiguous ranges of slices and writes their
 *    rows. Every row is summed by one thread in the order of the sequential
 *    functions above, so the result equals theirs bit for bit.
 *  - Otherwise: thread t walks its range of slices into a private zeroed
 *    n_out x w float64 copy of out; then every output element is the sum of
 *    the copies taken in thread order. The additions are regrouped by thread,
 *    so the result may differ from the sequential one in the last bits
 *    (exactly equal when every partial sum is exact, e.g. integer data).
 * out must be zeroed by the caller. Returns 0, or 1 if the private copies
 * could not be allocated. */

static void slice_vcs(int layout, int dir, int64_t s, const int32_t *major_ptr,
                      const double *values, const int32_t *value_ptr, const int32_t *indices,
                      const double *B, int64_t w, double *out) {
    for (int64_t k = major_ptr[s]; k < major_ptr[s + 1]; ++k)
        for (int64_t p = value_ptr[k]; p < value_ptr[k + 1]; ++p) {
            int64_t r = layout == 1 ? s : indices[p];
            int64_t c = layout == 1 ? indices[p] : s;
            entry(dir, r, c, values[k], B, w, out, NULL);
        }
}

static void slice_csr(int dir, int64_t r, const int32_t *row_ptr, const int32_t *col,
                      const double *val, const double *B, int64_t w, double *out) {
    for (int64_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p)
        entry(dir, r, col[p], val[p], B, w, out, NULL);
}

/* kind 0 = CSR (rows are slices), 1 = VCSR, 2 = VCSC. */
static int spmm_threaded(int kind, int dir, int64_t n_major, int64_t n_out,
                         const int32_t *sptr, const double *vals, const int32_t *vptr,
                         const int32_t *idx, const double *B, int64_t w, double *out,
                         int n_threads) {
    const int rows_are_slices = (kind != 2) == (dir == 0);
    const int64_t n_el = n_out * w;
    double *priv = NULL;
    if (n_threads < 1) n_threads = 1;
    if (!rows_are_slices) {
        priv = (double *)calloc((size_t)n_threads * (size_t)(n_el > 0 ? n_el : 1), sizeof(double));
        if (!priv) return 1;
    }
#pragma omp parallel num_threads(n_threads)
    {
        const int64_t t = omp_get_thread_num(), nt = omp_get_num_threads();
        const int64_t s0 = n_major * t / nt, s1 = n_major * (t + 1) / nt;
        double *dst = rows_are_slices ? out : priv + t * n_el;
        for (int64_t s = s0; s < s1; ++s) {
            if (kind == 0) slice_csr(dir, s, sptr, idx, vals, B, w, dst);
            else slice_vcs(kind, dir, s, sptr, vals, vptr, idx, B, w, dst);
        }
        if (!rows_are_slices) {
#pragma omp barrier
            const int64_t e0 = n_el * t / nt, e1 = n_el * (t + 1) / nt;
            for (int64_t e = e0; e < e1; ++e)
                for (int64_t u = 0; u < nt; ++u) out[e] += priv[u * n_el + e];
        }
    }
    free(priv);
    return 0;
}

int orc_spmm_vcs_threaded(int layout, int dir, int64_t n_major, int64_t n_out,
                          const int32_t *major_ptr, const double *values,
                          const int32_t *value_ptr, const int32_t *indices, const double *B,
                          int64_t w, double *out, int n_threads) {
    return spmm_threaded(layout, dir, n_major, n_out, major_ptr, values, value_ptr, indices, B,
                         w, out, n_threads);
}

int orc_spmm_csr_threaded(int dir, int64_t n_rows, int64_t n_out, const int32_t *row_ptr,
                          const int32_t *col, const double *val, const double *B, int64_t w,
                          double *out, int n_threads) {
    return spmm_threaded(0, dir, n_rows, n_out, row_ptr, val, NULL, col, B, w, out, n_threads);
}

/* ---------------------------------------------------------------- expansion */

/* VCS -> one value per entry, keeping the stored order: ptr[s] is the first
 * entry of slice s, idx = indices, val[p] = values of the group holding p. */
void orc_expand_vcs(int64_t n_major, const int32_t *major_ptr, const float *values,
                    const int32_t *value_ptr, const int32_t *indices,
                    int32_t *ptr, int32_t *idx, float *val) {
    for (int64_t s = 0; s <= n_major; ++s) ptr[s] = value_ptr[major_ptr[s]];
    for (int64_t s = 0; s < n_major; ++s)
        for (int64_t k = major_ptr[s]; k < major_ptr[s + 1]; ++k)
            for (int64_t p = value_ptr[k]; p < value_ptr[k + 1]; ++p) {
                idx[p] = indices[p];
                val[p] = values[k];
            }
}

/* ---------------------------------------------------------------- transpose */

/* Exact transpose by a two-pass counting sort (regridding page, "How it is
 * built"): count the entries of each minor index, turn the counts into
 * starts, then place every entry at its minor index's cursor in stored order,
 * so each output slice lists its entries by ascending source slice and, inside
 * a slice, in stored order. The value payload is copied byte for byte
 * (val_bytes = 4 or 8). */
void orc_transpose_csr(int64_t n_major, int64_t n_minor, const int32_t *ptr,
                       const int32_t *idx, const void *val, int val_bytes,
                       int32_t *t_ptr, int32_t *t_idx, void *t_val) {
    int64_t *cursor = (int64_t *)calloc((size_t)n_minor + 1, sizeof(int64_t));
    int64_t nnz = ptr[n_major];
    for (int64_t p = 0; p < nnz; ++p) cursor[idx[p] + 1] += 1;
    for (int64_t j = 0; j < n_minor; ++j) cursor[j + 1] += cursor[j];
    for (int64_t j = 0; j <= n_minor; ++j) t_ptr[j] = (int32_t)cursor[j];
    for (int64_t s = 0; s < n_major; ++s)
        for (int64_t p = ptr[s]; p < ptr[s + 1]; ++p) {
            int64_t at = cursor[idx[p]]++;
            t_idx[at] = (int32_t)s;
            memcpy((char *)t_val + at * val_bytes, (const char *)val + p * val_bytes,
                   (size_t)val_bytes);
        }
    free(cursor);
}

/* ---------------------------------------------------------------- assembly */

/* A regridder's operator assembled from its elements (regridding page,
 * section "API", the roles of the orthogonal axis; section "How it is
 * built", the two-pass counting sort). Element e holds entries [elem_ptr[e],
 * elem_ptr[e + 1]) of (out_idx, in_idx, weight). The role places entry
 * (e, o, i): role 0 (each element its own input and output) at row
 * e * n_out + o, column e * n_in + i; role 1 (one shared input) at row
 * e * n_out + o, column i; role 2 (outputs summed) at row o, column
 * e * n_in + i; role 3 (the elements' sum) at row o, column i. Pass one
 * counts each row's entries; pass two walks the elements in order and puts
 * each entry at its row's cursor, so a row lists its entries by element and
 * then in the order given. row_ptr has n_rows + 1 entries. */
static int64_t assembled_row(int role, int64_t e, int64_t o, int64_t n_out) {
    return role <= 1 ? e * n_out + o : o;
}

static int64_t assembled_col(int role, int64_t e, int64_t i, int64_t n_in) {
    return (role == 0 || role == 2) ? e * n_in + i : i;
}

void orc_assemble_csr(int role, int64_t n_elem, int64_t n_out, int64_t n_in,
                      const int32_t *elem_ptr, const int32_t *out_idx, const int32_t *in_idx,
                      const double *weight, int64_t n_rows, int32_t *row_ptr, int32_t *col,
                      double *val) {
    int64_t *cursor = (int64_t *)calloc((size_t)n_rows + 1, sizeof(int64_t));
    for (int64_t e = 0; e < n_elem; ++e)
        for (int64_t p = elem_ptr[e]; p < elem_ptr[e + 1]; ++p)
            cursor[assembled_row(role, e, out_idx[p], n_out) + 1] += 1;
    for (int64_t r = 0; r < n_rows; ++r) cursor[r + 1] += cursor[r];
    for (int64_t r = 0; r <= n_rows; ++r) row_ptr[r] = (int32_t)cursor[r];
    for (int64_t e = 0; e < n_elem; ++e)
        for (int64_t p = elem_ptr[e]; p < elem_ptr[e + 1]; ++p) {
            int64_t at = cursor[assembled_row(role, e, out_idx[p], n_out)]++;
            col[at] = (int32_t)assembled_col(role, e, in_idx[p], n_in);
            val[at] = weight[p];
        }
    free(cursor);
}

/* -------------------------------------------------------------- regrouping */

/* The order used to group a slice's entries by value: ascending float value,
 * as the total order on IEEE-754 single bit patterns (-0 before +0; NaNs
 * outside +-inf, ordered by payload). Two entries share a group exactly when
 * their values have the same bits. */
static uint32_t value_order(uint32_t bits) {
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

typedef struct {
    uint32_t key;   /* value_order of the entry's value */
    int64_t src;    /* position of the entry in the transposed (stored) order */
} keyed;

static int keyed_cmp(const void *a, const void *b) {
    const keyed *x = (const keyed *)a, *y = (const keyed *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return (x->src > y->src) - (x->src < y->src);
}

/* The same matrix in the opposite VCS layout (VCSR <-> VCSC), canonical for
 * the stored input: each new slice (an old minor index) holds its entries
 * grouped by value, groups in ascending value, and within a group the old
 * major indices in stored order (the order the counting sort above leaves).
 * Outputs: t_major_ptr[n_minor+1], t_values[<= nnz], t_value_ptr[<= nnz+1],
 * t_indices[nnz]; returns the number of groups. */
int64_t orc_regroup_vcs(int64_t n_major, int64_t n_minor, const int32_t *major_ptr,
                        const float *values, const int32_t *value_ptr,
                        const int32_t *indices, int32_t *t_major_ptr, float *t_values,
                        int32_t *t_value_ptr, int32_t *t_indices) {
    int64_t nnz = value_ptr[major_ptr[n_major]];
    int32_t *ptr = (int32_t *)malloc(sizeof(int32_t) * ((size_t)n_major + 1));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * ((size_t)nnz + 1));
    float *val = (float *)malloc(sizeof(float) * ((size_t)nnz + 1));
    int32_t *tptr = (int32_t *)malloc(sizeof(int32_t) * ((size_t)n_minor + 1));
    int32_t *tidx = (int32_t *)malloc(sizeof(int32_t) * ((size_t)nnz + 1));
    float *tval = (float *)malloc(sizeof(float) * ((size_t)nnz + 1));
    orc_expand_vcs(n_major, major_ptr, values, value_ptr, indices, ptr, idx, val);
    orc_transpose_csr(n_major, n_minor, ptr, idx, val, 4, tptr, tidx, tval);

    int64_t longest = 0;
    for (int64_t j = 0; j < n_minor; ++j)
        if (tptr[j + 1] - tptr[j] > longest) longest = tptr[j + 1] - tptr[j];
    keyed *seg = (keyed *)malloc(sizeof(keyed) * ((size_t)longest + 1));

    int64_t g = 0;
    for (int64_t j = 0; j < n_minor; ++j) {
        int64_t a = tptr[j], b = tptr[j + 1];
        for (int64_t e = a; e < b; ++e) {
            uint32_t bits;
            memcpy(&bits, &tval[e], 4);
            seg[e - a].key = value_order(bits);
            seg[e - a].src = e;
        }
        qsort(seg, (size_t)(b - a), sizeof(keyed), keyed_cmp);
        t_major_ptr[j] = (int32_t)g;
        for (int64_t e = a; e < b; ++e) {
            const keyed *x = &seg[e - a];
            if (e == a || x->key != seg[e - a - 1].key) {
                t_values[g] = tval[x->src];
                t_value_ptr[g] = (int32_t)e;
                ++g;
            }
            t_indices[e] = tidx[x->src];
        }
    }
    t_major_ptr[n_minor] = (int32_t)g;
    t_value_ptr[g] = (int32_t)nnz;
    free(seg); free(ptr); free(idx); free(val); free(tptr); free(tidx); free(tval);
    return g;
}
