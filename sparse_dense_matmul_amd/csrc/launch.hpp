// Launch plans and the launchers of each kernel family. Each family lives in
// a translation unit of its own (walk_*.hip) so the library's kernels compile
// in parallel; the host code in vspmm.hip sees only these declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vspmm {

struct Split {
    int log_ww;  // width lanes per entry lane (log2)
    int log_g;   // entry lanes per slice (log2)
};

enum Kind { kPlain = 0, kShort = 1, kLong = 2 };

constexpr int kRing = 128;              // k_short: ring positions per wave (two windows)
// k_short with 64 entry lanes, where a step is a whole window: a ring of eight
// windows, filled four at a time, so four steps' gathers go out together
constexpr int kRingDeep = 512;

// How one walk is launched: the lane split, the kernel family and its grid.
struct Plan {
    Split sp{0, 0};
    int vec = 1;         // elements per width lane (one 4-, 8- or 16-byte access)
    int R = 1;           // slices per wave in the plain walk
    int kind = kPlain;
    bool lds = false;    // dense operand staged in LDS
    size_t lds_bytes = 0;
    int grid = 0;
    int block = 256;
    int wps = 8;         // k_vcs_long, k_long: waves per slice
    int ring = kRing;    // k_short (CSR): ring positions per wave
};

constexpr size_t kLdsMax = 160 * 1024;  // LDS per CU on gfx950
// k_vcs_rows: entry windows and group windows per round (two rounds are held
// in registers at once), and the per-wave LDS they need (a mark byte per round
// position, a float per round group)
constexpr int kRowsNWR = 8;
constexpr int kRowsGWR = 2;
constexpr int kRowsWaveLds = 64 * kRowsNWR + 256 * kRowsGWR;
// k_vcs_rows: slices per unit of work, and the block's slice-header table
// (entries per array: the block's slice count plus the end pointer, rounded)
constexpr int kRowsChunk = 4;
__host__ __device__ inline int rows_header_cap(int n_slices, int n_blocks) {
    return ((n_slices + n_blocks - 1) / n_blocks + 2 + 3) & ~3;
}
// k_vcs_long: the same per pass of a slice piece
constexpr int kPieceNWR = 16;
constexpr int kPieceGWR = 4;
constexpr int kPieceWaveLds = 64 * kPieceNWR + 256 * kPieceGWR;

// k_vcs_seg: where one wave of a launch starts. Its run is the slices
// [s_a, s_b), entries [E_a, E_b) and groups [K_a, K_b), with K_a the group
// holding entry E_a (past any empty groups starting there). Built once per
// layout and launch shape by k_seg_plan.
struct SegDesc {
    int s_a, s_b, E_a, E_b, K_a, K_b, pad0, pad1;
};

// The slices [bb, be) that block blk of a k_vcs_rows / k_vcs_seg launch of
// `grid` blocks owns, and its tile: the slices are `tiles` runs of
// n_slices / tiles (one per tile of B), each cut into grid / tiles parts;
// with a multiple of 8 tiles, the blocks of a tile share an XCD (blocks go
// to the 8 XCDs round robin, block b to XCD b % 8), so a tile of B is
// fetched into one L2.
__host__ __device__ inline void seg_block_range(int blk, int grid, int tiles, int n_slices,
                                                int &bb, int &be, int &tile) {
    const int bpt = grid / tiles;  // blocks per tile
    int part;
    tile = blk / bpt;
    part = blk - tile * bpt;
    if (tiles % 8 == 0) {
        const int x = blk & 7, j = blk >> 3;
        tile = x * (tiles >> 3) + j / bpt;
        part = j - (j / bpt) * bpt;
    }
    const int n_run = n_slices / tiles;
    bb = tile * n_run + (int)((long long)part * n_run / bpt);
    be = tile * n_run + (int)((long long)(part + 1) * n_run / bpt);
}

// The operands of one aligned walk (slices of the walked layout = rows of out).
template <typename T>
struct WalkArgs {
    int n_slices;
    const int *sptr;  // slice pointers: CSR row_ptr or VCS major_ptr
    const int *vptr;  // VCS value_ptr (null for CSR)
    const T *vals;    // CSR values or VCS group values
    const int *idx;   // minor indices
    const T *B;       // dense input, n_in x w, row-major
    T *out;           // dense output, n_slices x w, row-major
    int w;
    int n_in;
    // k_vcs_rows only: the slices as `tiles` runs, each over n_in rows of B
    // (the last one cut at n_b_rows); 1 and n_in for an untiled walk
    int tiles = 1;
    int n_b_rows = 0;
    // CSR short/plain walks: slices longer than long_len are left to k_long
    // over long_list (n_long slices); a huge long_len skips nothing
    int long_len = 0x7fffffff;
    const int *long_list = nullptr;
    int n_long = 0;
    // CSR short walk: with n_parts equal to the grid's waves, wave k walks
    // the rows [parts[k], parts[k + 1]) (about equal entry counts), else an
    // equal share of the rows
    const int *parts = nullptr;
    int n_parts = 0;
    // CSR short walk: blocks added in front of the grid that walk the long
    // slices (kLongWaves waves per slice) in the same launch
    int long_blocks = 0;
    // float32 CSR values with T = double: the sums run in float64 over the
    // widened values (vals unused)
    const float *vals32 = nullptr;
    // VCS short walks: each slice's first entry (n_slices + 1) and the
    // per-wave starts of a k_vcs_seg launch of seg_grid blocks of seg_wpb
    // waves (null: walk with k_vcs_rows)
    const int *he = nullptr;
    const SegDesc *seg = nullptr;
    int seg_grid = 0;
    int seg_wpb = 0;
};

// Values of one type read as another (float32 CSR values summed in float64):
// indexing widens each value; used as the `vals` operand where the walks take
// a value-array type VP (a plain `const T *` otherwise).
template <typename T, typename V>
struct Widen {
    const V *p;
    __device__ __forceinline__ T operator[](int i) const { return T(p[i]); }
};

// Calls f with the walk's value array: the plain pointer, or, for float32
// CSR values summed in float64 (T = double with vals32 set), a Widen view.
template <typename T, typename Args, typename F>
void with_vals(const Args &a, F &&f) {
    if constexpr (sizeof(T) == 8) {
        if (a.vals32) return f(Widen<T, float>{a.vals32});
    }
    f(a.vals);
}

// The operands of one scatter walk (slices of the walked layout = rows of B).
template <typename T>
struct ScatterArgs {
    int n_slices;
    int n_groups;     // VCS groups (unused for CSR)
    int nnz;
    const int *sptr;  // slice pointers: CSR row_ptr or VCS major_ptr
    const int *vptr;  // VCS value_ptr (null for CSR)
    const T *vals;    // CSR values or VCS group values
    const int *idx;   // minor indices (rows of out)
    const T *B;       // dense input, n_slices x w, row-major
    T *out;           // dense output, n_out x w, row-major, zeroed by the caller
    int w;
    int n_out;
    const float *vals32 = nullptr;  // float32 CSR values with T = double (vals unused)
};

// Raises a kernel's dynamic LDS limit to a whole CU (once per kernel).
void allow_lds(const void *fn);

// walk_vcs_rows.hip: short VCS slices, float (one object per VEC).
template <int VEC>
void launch_vcs_rows(const Plan &pl, const WalkArgs<float> &a, hipStream_t s);

// walk_vcs_long.hip: long VCS slices, float (one object per VEC).
template <int VEC>
void launch_vcs_long(const Plan &pl, const WalkArgs<float> &a, hipStream_t s);

// walk_short.hip: short CSR slices.
template <typename T>
void launch_short(const Plan &pl, const WalkArgs<T> &a, hipStream_t s);

// walk_long.hip: long CSR slices, a block per slice.
template <bool VCS, typename T>
void launch_long(const Plan &pl, const WalkArgs<T> &a, hipStream_t s);

// walk_plain.hip: the plain slice-per-lane-group walk.
template <bool VCS, typename T>
void launch_plain(const Plan &pl, const WalkArgs<T> &a, hipStream_t s);

// walk_scatter.hip: the atomic scatter walk (pl.vec, pl.sp.log_ww, grid,
// block; pl.lds adds through an LDS copy of out of pl.lds_bytes).
template <bool VCS, typename T>
void launch_scatter(const Plan &pl, const ScatterArgs<T> &a, hipStream_t s);

}  // namespace vspmm
