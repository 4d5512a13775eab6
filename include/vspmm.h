/*
 * libvspmm: row-segmented sparse x dense products (SpMM, and SpMV at width 1)
 * over CSR and the value-grouped VCSR/VCSC layouts, for AMD Instinct MI355X
 * (gfx950).
 *
 * Layouts
 *  - VCSR / VCSC, defined on the vsparse page ("Add CUDA transfer and matmul
 *    kernels for the normalized views", section "The layout stays
 *    compressed"): for major slice i (row i of a VCSR, column i of a VCSC) the
 *    distinct values are values[major_ptr[i] .. major_ptr[i+1]) and value k is
 *    shared by the minor indices indices[value_ptr[k] .. value_ptr[k+1]).
 *    Values are float32 on the device (same page, opening paragraph).
 *  - CSR, the single-matrix operator of the regridding page ("Regridder",
 *    sections "How it is built" and "API"): row i holds col[row_ptr[i] ..
 *    row_ptr[i+1]) with one value each, float32 or float64.
 *  Every stored entry (r, c, v) adds v to A[r][c]: repeated indices, empty
 *  groups and explicit zeros are legal and sum. The matrix is never expanded:
 *  a handle borrows the caller's arrays as they are.
 *
 * Directions (vsparse page, section "The kernels"): out = A @ B (VSPMM_AB) and
 * out = B @ A (VSPMM_BA). Dense operands are row-major with the width
 * contiguous and indexed by the sparse axis they meet:
 *  - VSPMM_AB: B is n_cols x width, out is n_rows x width.
 *  - VSPMM_BA: B is passed transposed, n_rows x width, and out is written
 *    transposed, n_cols x width.
 * A direction is "aligned" when the output's rows are the layout's major
 * slices (VCSR @ B, B @ VCSC, CSR @ B) and "misaligned" otherwise (B @ VCSR,
 * VCSC @ B, B @ CSR). Aligned products accumulate per slice in registers and
 * repeat bit for bit. Misaligned products scatter with hardware float atomics
 * (VSPMM_ATOMIC; last bits vary run to run) or, with VSPMM_DETERMINISTIC, first
 * build the matrix in the opposite layout in a caller-owned workspace and then
 * run the aligned walk over it, which repeats bit for bit.
 *
 * Conventions
 *  - All pointers passed as "device" must be device memory of the current HIP
 *    device (e.g. torch CUDA tensors); host pointers are marked "host".
 *  - Index and pointer arrays are int32. Pointer arrays start at 0 and do not
 *    decrease; indices lie in [0, n_minor). Those rules are only checked by
 *    vspmm_validate (or VSPMM_VALIDATE at create); a product over a structure
 *    that breaks them is undefined.
 *  - out is overwritten, never accumulated into. width == 0 or an empty
 *    output returns VSPMM_OK without a launch; nnz == 0 zero-fills out.
 *  - Every call returns a status; nothing throws across this interface.
 *    Argument checks run on the host before anything is enqueued; a failed
 *    check enqueues nothing. Launch errors return VSPMM_ERR_HIP.
 *  - Work is enqueued on the given stream and returns before it finishes,
 *    except vspmm_validate, which waits for its result, and
 *    vspmm_create_csr, which waits once for its list of long rows.
 *  - A handle changes after creation only through vspmm_set_view. Products
 *    on different streams may run concurrently if their outputs and
 *    workspaces are distinct, except on a handle with a SCALE view, whose
 *    products share the handle's scaled-input buffer.
 *  - Non-finite values spread only through stored entries: an element of out
 *    is NaN or +-Inf exactly when IEEE arithmetic over the entries of its own
 *    slice makes it so (a lane that a walk pads with another slice's entry
 *    keeps its sum, never adding zero times a non-finite B element).
 */
#ifndef VSPMM_H
#define VSPMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vspmm_matrix_s *vspmm_matrix; /* opaque handle */
typedef struct vspmm_schedule_s *vspmm_schedule; /* opaque: a built pass-2 layout */

typedef enum {
    VSPMM_OK = 0,
    VSPMM_ERR_NULL = 1,        /* a required pointer is NULL */
    VSPMM_ERR_DIM = 2,         /* negative or inconsistent extent, or above int32 */
    VSPMM_ERR_ENUM = 3,        /* unknown layout, direction, dtype, mode or flag */
    VSPMM_ERR_STRUCTURE = 4,   /* vspmm_validate found a malformed structure */
    VSPMM_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    VSPMM_ERR_UNSUPPORTED = 6, /* valid request this library does not serve */
    VSPMM_ERR_HIP = 7,         /* a HIP call or kernel launch failed */
    VSPMM_ERR_ALLOC = 8        /* host allocation failed */
} vspmm_status;

typedef enum { VSPMM_CSR = 0, VSPMM_VCSR = 1, VSPMM_VCSC = 2 } vspmm_layout;
typedef enum { VSPMM_AB = 0, VSPMM_BA = 1 } vspmm_direction;
/* Element types of a CSR handle: VSPMM_F32 and VSPMM_F64 store values, take
 * dense operands and carry sums in that type; VSPMM_F32_F64 stores float32
 * values and takes float64 dense operands, with the sums in float64 (each
 * value widened exactly; regridding page, section "Why not cuSPARSE", on
 * summing float32 entries in float64). VCS handles are float32. */
typedef enum { VSPMM_F32 = 0, VSPMM_F64 = 1, VSPMM_F32_F64 = 2 } vspmm_dtype;
typedef enum { VSPMM_ATOMIC = 0, VSPMM_DETERMINISTIC = 1 } vspmm_mode;

/* Creation flags. The lane split (vsparse page, section "The kernels";
 * regridding page, section "How it is built") picks, per product, how many
 * lanes of a 64-lane wave cover the dense width and how many walk the slice's
 * entries.
 *  - VSPMM_SPLIT_WIDTH: the split follows the width (the default for VCS).
 *  - VSPMM_SPLIT_MATRIX: the number of entry lanes follows the matrix, the
 *    power of two at or below its mean entries per slice, at most 64 (the
 *    default for CSR). It does not depend on the width, so each column of a
 *    batch gets exactly the bits it gets alone.
 *  - VSPMM_VALIDATE: run vspmm_validate during creation. */
enum { VSPMM_SPLIT_WIDTH = 1u, VSPMM_SPLIT_MATRIX = 2u, VSPMM_VALIDATE = 4u };

/* Create a handle over a VCSR or VCSC held in device memory.
 *  layout      VSPMM_VCSR (major = rows) or VSPMM_VCSC (major = columns).
 *  n_rows, n_cols  shape of A; n_groups = length of values; nnz = length of
 *              indices. All must fit in int32.
 *  major_ptr   device int32[n_major + 1]; values device float[n_groups];
 *  value_ptr   device int32[n_groups + 1]; indices device int32[nnz].
 *              Borrowed: they must stay alive and unchanged until
 *              vspmm_destroy. May be NULL only when their length is 0.
 *  flags       VSPMM_SPLIT_* / VSPMM_VALIDATE.
 *  force_group 0, or a power of two 1..64 fixing the number of entry lanes
 *              per slice (tests use it to cover every split).
 *  stream      stream used by VSPMM_VALIDATE (and, for CSR, the row ranges
 *              and the long-row list).
 * Errors: VSPMM_ERR_NULL, _DIM, _ENUM, _STRUCTURE (with VSPMM_VALIDATE),
 * _HIP, _ALLOC. *h is set only on success. */
vspmm_status vspmm_create_vcs(vspmm_matrix *h, vspmm_layout layout, int64_t n_rows,
                              int64_t n_cols, int64_t n_groups, int64_t nnz,
                              const int32_t *major_ptr, const float *values,
                              const int32_t *value_ptr, const int32_t *indices,
                              uint32_t flags, int32_t force_group, hipStream_t stream);

/* Create a handle over a CSR held in device memory (rows are the major axis).
 *  row_ptr device int32[n_rows + 1]; col device int32[nnz];
 *  val device float[nnz] (VSPMM_F32, VSPMM_F32_F64) or double[nnz]
 *  (VSPMM_F64). The dense operands of every product on this handle are
 *  float32 (VSPMM_F32) or float64 (VSPMM_F64, VSPMM_F32_F64), and the sums
 *  are carried in that type. Other arguments as vspmm_create_vcs.
 *  The handle also holds, in device memory it owns (freed by vspmm_destroy):
 *  - one row range per wave of the short walk's grid (16 waves per CU), cut
 *    so the ranges hold about equal numbers of entries (a binary search over
 *    row_ptr per range), int32[16 * CUs + 1];
 *  - the list of long rows: rows longer than one wave's share of the entries
 *    (nnz / (16 * CUs), at least 64) or than one round of the short walk
 *    (1,536 entries float32, 768 float64), whichever is smaller. Products
 *    walk those rows with a block of waves each instead of inside one wave's
 *    range, so a few long rows do not hold up the rest (regridding page,
 *    section "How it is built", on giving a row a group of threads sized to
 *    it).
 *  Both are built from row_ptr on `stream`; counting the long rows waits for
 *  it once. Which rows are long is fixed at creation, so it does not depend
 *  on the width of a product. */
vspmm_status vspmm_create_csr(vspmm_matrix *h, int64_t n_rows, int64_t n_cols, int64_t nnz,
                              const int32_t *row_ptr, const int32_t *col, const void *val,
                              vspmm_dtype dtype, uint32_t flags, int32_t force_group,
                              hipStream_t stream);

/* Create a handle over a CSR with int64 row pointers and int32 column
 * indices, for matrices of more than 2^31 - 1 entries (regridding page,
 * section "Why not cuSPARSE": row pointers must be int64 past 2^31 entries,
 * while the column indices can stay int32).
 *  row_ptr device int64[n_rows + 1]; col device int32[nnz]; val device
 *  float[nnz] or double[nnz] as for vspmm_create_csr. nnz may exceed int32;
 *  n_rows and n_cols may not.
 *  block_nnz   0, or 1 .. 2^30: entries per row block (0 = 2^30).
 * The rows are cut into blocks of whole rows, each of at most block_nnz
 * entries (a single longer row forms a block of its own, up to 2^30 entries),
 * and each block becomes an int32 CSR handle over the same col and val arrays
 * from its first entry on (rebased row pointers in device memory the handle
 * owns). Creation copies row_ptr to the host (one wait on `stream`), checks
 * that it starts at 0, does not decrease and ends at nnz, and creates the
 * blocks as vspmm_create_csr does (flags and force_group apply to each).
 * Products:
 *  - A @ B: each block writes its own rows of out; rows repeat bit for bit and
 *    equal the int32 handle's over the same rows when the blocks cut nothing.
 *  - B @ A, atomic: out is zeroed once and every block scatters into it.
 *  - B @ A, deterministic: block 0's product is written to out and each later
 *    block's product (into the workspace) is added to it in block order, so
 *    the result repeats bit for bit. The workspace holds 256 bytes, each
 *    block's exact transpose and, with two or more non-empty blocks, an
 *    n_cols x width buffer: vspmm_workspace_size_width gives the whole;
 *    vspmm_workspace_size gives it without the buffer (enough for one
 *    non-empty block).
 * vspmm_validate checks every block; vspmm_plan_info reports block 0's plan;
 * vspmm_transpose_csr returns VSPMM_ERR_UNSUPPORTED (its row pointers are
 * int32). Errors: as vspmm_create_csr, plus _STRUCTURE (row_ptr as above) and
 * _UNSUPPORTED (a row of more than 2^30 entries). */
vspmm_status vspmm_create_csr64(vspmm_matrix *h, int64_t n_rows, int64_t n_cols, int64_t nnz,
                                const int64_t *row_ptr, const int32_t *col, const void *val,
                                vspmm_dtype dtype, uint32_t flags, int32_t force_group,
                                int64_t block_nnz, hipStream_t stream);

/* Release the handle: its host metadata and, for CSR, the device arrays it
 * owns (row ranges and long-row list). The borrowed arrays are untouched: the
 * handle never held a copy of them (vsparse page, section "The layout stays
 * compressed": the device view is the arrays themselves, never an expanded
 * copy). Errors: _NULL. */
vspmm_status vspmm_destroy(vspmm_matrix h);

/* out = A @ B or B @ A (see Directions), atomic mode for misaligned
 * directions, no workspace. B and out: device arrays of the handle's dtype,
 * row-major with `width` contiguous elements per row; they must not overlap.
 * Errors: _NULL, _DIM (width < 0), _ENUM, _HIP. */
vspmm_status vspmm_spmm(vspmm_matrix h, const void *B, void *out, int64_t width,
                        vspmm_direction dir, hipStream_t stream);

/* Bytes of workspace vspmm_spmm_ex needs for (dir, mode) (0 when none):
 * for a deterministic misaligned product, the matrix in the opposite layout
 * plus the scratch of the counting sort that builds it (regridding page,
 * section "How it is built": a two-pass counting sort; vsparse page, section
 * "The kernels": the misaligned directions are the ones needing more than a
 * plain walk). bytes: host. Errors: _NULL, _ENUM. */
vspmm_status vspmm_workspace_size(vspmm_matrix h, vspmm_direction dir, vspmm_mode mode,
                                  size_t *bytes);

/* vspmm_spmm with a mode. VSPMM_DETERMINISTIC on a misaligned direction
 * builds the matrix in the opposite layout (CSR: its exact transpose;
 * VCSR/VCSC: the same matrix regrouped by the other axis) inside ws, and runs
 * the aligned walk over it. Every call builds it again: ws holds nothing from
 * one call to the next. To build once and run many products, use a schedule
 * (vspmm_schedule_create).
 *
 * Tiled schedule (VCSR/VCSC, float, either direction): when B's rows do not
 * fit in a CU's LDS and ws holds at least vspmm_workspace_size_width bytes
 * for this width, deterministic mode instead builds a tiled copy of the
 * matrix: B's rows are cut into tiles and each output row's entries are split
 * by tile, every (tile, output row) part grouped by value as in the pages'
 * value-grouped layouts. With rows of up to 64 bytes, B is cut into tiles
 * that fit in LDS and each block stages its tile there, as long as the
 * partial rows the tiles write and read back stay within half the matrix's
 * own bytes: the fewest such tiles, rounded up to a multiple of 8 (each XCD
 * then owns whole tiles) when there are four or more, or left as they are
 * when only that count keeps the partial rows within bounds; where the fewest
 * tiles would leave (tile, output row) parts of 1,024 entries or more on
 * average, the tile count rises to a multiple of 8 until the mean is at most
 * 512. Otherwise (wider rows, or LDS tiles that do not pay) a B larger than
 * 4 MB is cut into tiles of about 2 MB, a multiple of 8 of them, each fitting
 * one XCD's L2: the blocks of a tile, all on one XCD and as many as the XCD
 * holds at once, gather it from global memory; a smaller B is gathered
 * untiled from L2. The product writes one partial row per (tile, output row)
 * into ws and adds them in a fixed order; it repeats bit for bit. A smaller ws
 * falls back to the path above (aligned: the plain walk, ws unused).
 *
 * ws: device, 256-byte aligned, at least vspmm_workspace_size bytes; unused
 * (may be NULL) when the size is 0. Errors: as vspmm_spmm, plus
 * _WORKSPACE. */
vspmm_status vspmm_spmm_ex(vspmm_matrix h, const void *B, void *out, int64_t width,
                           vspmm_direction dir, vspmm_mode mode, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* vspmm_spmm_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument, and the call allocates nothing. Its workspace is a
 * device array inside the library of VSPMM_NOALLOC_WS_BYTES (64 MiB), one
 * per device, held from the library's first use on that device until the
 * process ends. A product whose workspace
 * (vspmm_workspace_size; with the width for an int64 CSR) exceeds it
 * returns VSPMM_ERR_WORKSPACE and enqueues nothing; the tiled copy is taken
 * when it fits. Every call on a device shares that device's array and leaves
 * its contents behind (each call rebuilds what it reads): calls that overlap
 * in time on one device race and must not be issued so (one stream, or a
 * wait between them). Results equal vspmm_spmm_ex's bit for bit in
 * deterministic mode. Errors: as vspmm_spmm_ex. */
#define VSPMM_NOALLOC_WS_BYTES ((size_t)64 << 20)
vspmm_status vspmm_spmm_noalloc(vspmm_matrix h, const void *B, void *out, int64_t width,
                                vspmm_direction dir, vspmm_mode mode, hipStream_t stream);

/* Normalized views. On the vsparse page a view of the counts transforms each
 * stored value on the fly (introduction), carries O(n_rows + n_cols)
 * statistics beside the four arrays and never an expanded copy (section "The
 * layout stays compressed"), and a transform the device code does not know
 * fails loudly (section "Testing"). The page does not give its transforms;
 * this library offers the identity and one closed form:
 *   VSPMM_VIEW_SCALE: stored entry (r, c, v) acts as v * row_stat[r] * col_stat[c].
 * Every product on the handle (vspmm_spmm, _spmm_ex, _spmm_noalloc,
 * _schedule_spmm) then computes diag(out_stat) A diag(in_stat) B: B's rows
 * are scaled by their axis's statistic into a buffer the handle owns, the
 * walk runs over that, and out's rows are scaled by the other axis's
 * statistic; in exact arithmetic that is the product with every entry
 * transformed. */
typedef enum { VSPMM_VIEW_IDENTITY = 0, VSPMM_VIEW_SCALE = 1 } vspmm_view;

/* Sets the handle's view. row_stat: device [n_rows], col_stat: device
 * [n_cols], of the dense operands' type (float for VSPMM_F32 and VCS, double
 * otherwise), borrowed; ignored for VSPMM_VIEW_IDENTITY (which clears a
 * view). max_width: the widest product the view will serve; the handle
 * allocates max(n_rows, n_cols) x max_width elements for the scaled input,
 * and products wider than that return VSPMM_ERR_DIM. Products through one
 * handle with a SCALE view share that buffer: they must not overlap in time;
 * call this only while none is in flight. Errors: _NULL, _ENUM (unknown
 * view), _DIM, _HIP. */
vspmm_status vspmm_set_view(vspmm_matrix h, int32_t view, const void *row_stat,
                            const void *col_stat, int64_t max_width);

/* The name of a view code ("identity", "scale"), or NULL for a code this
 * library does not implement (bindings check their list against it). */
const char *vspmm_view_name(int32_t view);

/* Bytes of workspace for a product of the given width: in deterministic
 * mode, what the tiled schedule needs when it applies (see vspmm_spmm_ex),
 * else the same as vspmm_workspace_size. bytes: host. Errors: as
 * vspmm_workspace_size, plus _DIM (negative width). */
vspmm_status vspmm_workspace_size_width(vspmm_matrix h, vspmm_direction dir, vspmm_mode mode,
                                        int64_t width, size_t *bytes);

/* Schedules: the two-pass deterministic product with its first pass done
 * once. On the regridding page the exact transpose is kept once it has been
 * built (section "API"), the build is a two-pass counting sort (section "How
 * it is built") and every output row is summed in a fixed order (section
 * "Why"). A schedule holds such a built layout for one (handle, direction,
 * width): the opposite layout
 * of a misaligned direction, or the tiled copy where vspmm_spmm_ex would
 * take the tiled schedule, in device memory of its own sized to what the
 * product reads (the realized group count, not the worst case). Products
 * through it equal vspmm_spmm_ex's in deterministic mode bit for bit.
 *
 * vspmm_schedule_create builds it. build_ws: device, 256-byte aligned, at
 * least vspmm_workspace_size_width(h, dir, VSPMM_DETERMINISTIC, width) bytes,
 * used only during the call; or NULL, and the call allocates and frees a
 * build workspace of its own. Waits for `stream` (it reads back the group
 * count). Errors: _NULL, _ENUM, _DIM, _WORKSPACE (build_ws too small), _HIP,
 * _ALLOC.
 * For an aligned direction with no tiled copy (and for an empty matrix) the
 * schedule holds nothing and its products are the plain walk.
 *
 * The schedule reads the handle's arrays: destroy it before the handle. */
vspmm_status vspmm_schedule_create(vspmm_schedule *sc, vspmm_matrix h, vspmm_direction dir,
                                   int64_t width, void *build_ws, size_t build_ws_bytes,
                                   hipStream_t stream);

/* out = A @ B or B @ A through schedule sc, in its direction; width must equal
 * the schedule's. A tiled schedule keeps the product's partial rows in its
 * own memory: products through one schedule must not overlap in time (issue
 * them on one stream, or wait between them). Errors: as vspmm_spmm, plus _DIM
 * for another width. */
vspmm_status vspmm_schedule_spmm(vspmm_schedule sc, const void *B, void *out, int64_t width,
                                 hipStream_t stream);

/* Device bytes the schedule holds (vsparse page, section "Benchmarks": device
 * bytes are reported against the expanded form). bytes: host. Errors: _NULL. */
vspmm_status vspmm_schedule_bytes(vspmm_schedule sc, size_t *bytes);

/* Frees the schedule's memory (after its products have finished on the
 * device). Errors: _NULL. */
vspmm_status vspmm_schedule_destroy(vspmm_schedule sc);

/* Check the structure on the device: pointer arrays start at 0, do not
 * decrease and end at their array's length; every index is in range
 * (regridding page, section "Tests": invalid shapes are rejected; the array
 * meanings are those of vsparse, section "The layout stays compressed").
 * Waits on `stream` for the answer. Returns VSPMM_OK or VSPMM_ERR_STRUCTURE
 * (or _NULL, _HIP). */
vspmm_status vspmm_validate(vspmm_matrix h, hipStream_t stream);

/* The exact transpose of a CSR handle by a stable counting sort (regridding
 * page, section "How it is built": counts per row, then placement at the rows'
 * cursors in source order), equal bit for bit to a sequential counting sort.
 * Outputs (device): t_row_ptr int32[n_cols + 1], t_col int32[nnz], t_val of
 * the handle's value type [nnz] (float for VSPMM_F32_F64). ws: device, vspmm_workspace_size(h, VSPMM_BA,
 * VSPMM_DETERMINISTIC) bytes. Errors: _NULL, _ENUM (not CSR), _WORKSPACE,
 * _HIP. */
vspmm_status vspmm_transpose_csr(vspmm_matrix h, int32_t *t_row_ptr, int32_t *t_col,
                                 void *t_val, void *ws, size_t ws_bytes, hipStream_t stream);

/* The matrix of a VCSR handle as a VCSC, or of a VCSC handle as a VCSR,
 * canonical for the input: each new slice groups its entries by value, the
 * groups in ascending value (IEEE total order on the bits, -0 before +0) and
 * the entries of a group in stored order (ascending old slice). Outputs
 * (device): t_major_ptr int32[n_minor + 1], t_values float[nnz],
 * t_value_ptr int32[nnz + 1], t_indices int32[nnz], t_n_groups int32[1] (the
 * number of groups written). ws as for the deterministic misaligned product.
 * Errors: _NULL, _ENUM (not VCS), _WORKSPACE, _HIP. */
vspmm_status vspmm_regroup_vcs(vspmm_matrix h, int32_t *t_major_ptr, float *t_values,
                               int32_t *t_value_ptr, int32_t *t_indices,
                               int32_t *t_n_groups, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* Formats of an expanded matrix (one value per entry): the CSR of A (row
 * pointers over the rows, column indices) or its CSC (column pointers over
 * the columns, row indices). */
/* The exact transpose with every entry scaled by a factor of its own: the
 * shape of the regridding page's conservative transpose (section "API"),
 * which scales each entry of the exact transpose by its own element's cells
 * (not two diagonal scalings) and shares the indices of .T. The factors are
 * the caller's (the cell volumes behind them need grids the pages do not
 * give). factor: device [nnz] of the stored value type, one per stored entry
 * in the handle's order; entry p's value in the transpose is val[p] *
 * factor[p], rounded once. t_row_ptr and t_col equal vspmm_transpose_csr's.
 * Other arguments and errors as vspmm_transpose_csr. */
vspmm_status vspmm_transpose_csr_scaled(vspmm_matrix h, const void *factor, int32_t *t_row_ptr,
                                        int32_t *t_col, void *t_val, void *ws, size_t ws_bytes,
                                        hipStream_t stream);

/* Roles of a regridder's orthogonal axis (regridding page, section "API",
 * the roles table), for an operator of n_elem elements, each a sparse
 * matrix from n_in input cells to n_out output cells:
 *   VSPMM_ROLE_OWN     (weights N, input N, output N): each element applies
 *                      to its own input: rows e n_out + o, columns e n_in + i;
 *   VSPMM_ROLE_SHARED  (N, 1, N): every element applies to the same input:
 *                      rows e n_out + o, columns i;
 *   VSPMM_ROLE_SUMMED  (N, N, 1): the elements' outputs are summed: rows o,
 *                      columns e n_in + i;
 *   VSPMM_ROLE_SUM_OF  (N, 1, 1): the sum of the elements applies: rows o,
 *                      columns i.
 * The table's batch axis (weights 1, input M, output M: the same matrix
 * applied to every input) is the width of the dense operands. */
typedef enum {
    VSPMM_ROLE_OWN = 0,
    VSPMM_ROLE_SHARED = 1,
    VSPMM_ROLE_SUMMED = 2,
    VSPMM_ROLE_SUM_OF = 3
} vspmm_role;

/* Assembles the elements' weights into one CSR operator (regridding page,
 * section "How it is built": a two-pass counting sort in which every row
 * keeps its entries in the order of the elements), so that one product
 * applies them all. Element e's weights are entries [elem_ptr[e],
 * elem_ptr[e + 1]) of (out_idx, in_idx, weight): device arrays, out_idx in
 * [0, n_out), in_idx in [0, n_in), weight float (VSPMM_F32) or double
 * (VSPMM_F64). Output (device): row_ptr [rows + 1], col [nnz], val [nnz] of
 * the weight type, rows and columns as the role gives; a row lists its
 * entries by element, then in the order given (repeated coordinates stay
 * separate entries, which products add). Malformed element pointers or
 * indices give an undefined operator (nothing is written out of range).
 * ws: device, 256-byte aligned, vspmm_assemble_workspace_size bytes. Errors:
 * _NULL, _ENUM, _DIM (rows + 1 or columns above int32), _WORKSPACE, _HIP. */
vspmm_status vspmm_assemble_csr(int32_t role, int64_t n_elem, int64_t n_out, int64_t n_in,
                                int64_t nnz, const int32_t *elem_ptr, const int32_t *out_idx,
                                const int32_t *in_idx, const void *weight, vspmm_dtype dtype,
                                int32_t *row_ptr, int32_t *col, void *val, void *ws,
                                size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of vspmm_assemble_csr. bytes: host. Errors: _NULL, _ENUM,
 * _DIM. */
vspmm_status vspmm_assemble_workspace_size(int32_t role, int64_t n_elem, int64_t n_out,
                                           int64_t n_in, int64_t nnz, size_t *bytes);

typedef enum { VSPMM_FORMAT_CSR = 0, VSPMM_FORMAT_CSC = 1 } vspmm_format;

/* A VCS handle expanded to one value per entry (vsparse page, section
 * "Benchmarks": the expansion its baseline runs on is index-sorted by
 * default, with an opt-out, and takes a format so a VCSC-backed matrix can be
 * expanded to CSR).
 *  - The layout's own format (CSR from a VCSR, CSC from a VCSC): with
 *    sort_indices == 0 the entries in stored order (each slice's groups in
 *    turn, the group's value repeated on each of its entries); otherwise each
 *    slice's entries ordered by index, repeated indices in stored order.
 *  - The other format: the exact transpose of the stored-order expansion;
 *    each slice lists its entries by ascending index (sort_indices has no
 *    effect), repeated pairs in stored order.
 * Outputs (device): ptr int32[n_rows + 1] (CSR) or int32[n_cols + 1] (CSC),
 * idx int32[nnz], val float[nnz]. ws: device, 256-byte aligned, at least
 * vspmm_workspace_size(h, dir, VSPMM_DETERMINISTIC) bytes for the handle's
 * misaligned direction (VSPMM_BA for a VCSR, VSPMM_AB for a VCSC), needed
 * unless the format is the layout's own and sort_indices == 0 (then it may
 * be NULL). A workspace holding a built schedule is overwritten (the next
 * deterministic product on it rebuilds). Bit-exact: the same entries and
 * values as the definition, in the order above.
 * Errors: _NULL, _ENUM (not VCS, unknown format), _WORKSPACE, _HIP. */
vspmm_status vspmm_expand_vcs(vspmm_matrix h, vspmm_format format, int32_t sort_indices,
                              int32_t *ptr, int32_t *idx, float *val, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* Device bytes the handle's arrays occupy, and what the same matrix would take
 * expanded to one value per entry in the same major order (int32 pointers and
 * indices): the comparison of vsparse page, section "Benchmarks", which
 * states the value-grouped layouts' device bytes as a fraction of the
 * expanded CSR's (0.62 for VCSR, 0.51 for VCSC on its 60k x 2k matrix). Both
 * host. Errors: _NULL. */
vspmm_status vspmm_footprint(vspmm_matrix h, size_t *bytes, size_t *expanded_bytes);

/* Kernel family a product's walk runs in (reported by vspmm_plan_info). */
typedef enum {
    VSPMM_KERNEL_PLAIN = 0,   /* slices side by side, one lane group each */
    VSPMM_KERNEL_SHORT = 1,   /* a wave walks a block of short slices in register rounds */
    VSPMM_KERNEL_LONG = 2,    /* a block of waves walks one long slice */
    VSPMM_KERNEL_SCATTER = 3, /* misaligned walk with float atomics */
    VSPMM_KERNEL_SEG = 4      /* VCS: each wave walks a planned run of entries across slices */
} vspmm_kernel;

/* The lane split a product would use (host outputs, any may be NULL):
 * entry lanes per slice, width lanes, elements per lane, slices per wave,
 * whether the gathered operand is staged in LDS, and the kernel family
 * (vspmm_kernel). The scatter walk balances entries rather than slices over
 * its waves (slices per wave 0), takes its entry lanes as entries added side
 * by side, and reports as LDS-staged the copy of the output each block adds
 * into when the output fits in LDS. tiles: in deterministic mode, the tiles of
 * B a tiled schedule would use (0 when none applies); the other outputs then
 * describe the walk over the tiled copy. In deterministic mode a misaligned product reports its
 * second pass, the aligned walk over the opposite layout. The caller's buffer
 * alignment is not known here, so 16-byte aligned operands are assumed. */
vspmm_status vspmm_plan_info(vspmm_matrix h, int64_t width, vspmm_direction dir,
                             vspmm_mode mode, int32_t *entry_lanes, int32_t *width_lanes,
                             int32_t *vec, int32_t *slices_per_wave, int32_t *lds_staged,
                             int32_t *kernel, int32_t *tiles);

/* A static string naming the status. */
const char *vspmm_status_string(vspmm_status st);

#ifdef __cplusplus
}
#endif

#endif /* VSPMM_H */
