// libvspmm: the C interface declared in include/vspmm.h. Host-side checks,
// the per-call plan (lane split, grid), kernel launches, and the device
// builders of the opposite layout for the deterministic misaligned products.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "vspmm.h"
#include "launch.hpp"
#include "schedule.hpp"

using namespace vspmm;

// ------------------------------------------------------------------ handle

struct vspmm_matrix_s {
    int layout;  // vspmm_layout
    int64_t n_rows, n_cols, n_groups, nnz;
    const int32_t *sptr;   // CSR row_ptr or VCS major_ptr
    const void *vals;      // CSR val or VCS values
    const int32_t *vptr;   // VCS value_ptr
    const int32_t *idx;    // minor indices
    int dtype;             // vspmm_dtype
    uint32_t flags;
    int force_group;
    int device;
    // CSR: rows longer than long_len (device list, owned), walked by k_long
    // apart from the short walks so one long row does not hold up a wave
    int32_t *long_rows = nullptr;
    int64_t n_long = 0;
    int long_len = 0x7fffffff;
    // CSR: entry-balanced row ranges for the short walk, one per wave of its
    // grid (16 waves per CU), device array of n_parts + 1 (owned)
    int32_t *parts = nullptr;
    int n_parts = 0;
    // CSR created with int64 row pointers: the rows are cut into blocks of at
    // most 2^30 entries, each an int32 CSR handle (owned) over the same col
    // and val arrays from its first entry on; block_row0 holds each block's
    // first row and then n_rows, block_ptr the blocks' rebased row pointers
    bool ptr64 = false;
    // VCS: each slice's first entry and the per-wave starts of the k_vcs_seg
    // walk over the handle's own layout (device, owned; one block of
    // kSegWaves waves per CU)
    int32_t *seg_he = nullptr;
    SegDesc *seg_desc = nullptr;
    int seg_grid = 0;
    std::vector<vspmm_matrix_s *> blocks;
    std::vector<int64_t> block_row0;
    int32_t *block_ptr = nullptr;
    // normalized view (VSPMM_VIEW_SCALE): entry (r, c, v) acts as
    // v * row_stat[r] * col_stat[c]; statistics borrowed, in the dense
    // operands' type; view_buf (owned) holds the scaled dense input of up to
    // view_width columns
    int view = VSPMM_VIEW_IDENTITY;
    const void *row_stat = nullptr, *col_stat = nullptr;
    void *view_buf = nullptr;
    int64_t view_width = 0;
    int64_t n_major() const { return layout == VSPMM_VCSC ? n_cols : n_rows; }
    int64_t n_minor() const { return layout == VSPMM_VCSC ? n_rows : n_cols; }
    // bytes of a dense element (the type the sums run in) and of a stored value
    size_t elt() const { return dtype == VSPMM_F32 ? 4 : 8; }
    size_t val_elt() const { return dtype == VSPMM_F64 ? 8 : 4; }
};

// Lets a kernel use up to the whole LDS of a CU as dynamic shared memory
// (once per kernel; a fixed table, so a product allocates no host memory).
void vspmm::allow_lds(const void *fn) {
    static std::mutex mu;
    static const void *done[1024];
    static int n_done = 0;
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < n_done; ++i)
        if (done[i] == fn) return;
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsMax));
    if (n_done < 1024) done[n_done++] = fn;
}

// The workspace of vspmm_spmm_noalloc: a file-scope device array, one copy
// per device, held from the library's first use on a device until the
// process ends. On the host its name is only a stand-in for the symbol: host
// code takes each device's address of it with hipGetSymbolAddress and passes
// that, never the name.
constexpr size_t kStaticScratchBytes = VSPMM_NOALLOC_WS_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

struct DeviceInfo {
    int n_cu = 0;
    bool ok = false;
};
std::mutex g_dev_mutex;
DeviceInfo g_dev[64];

DeviceInfo device_info(int dev) {
    std::lock_guard<std::mutex> lk(g_dev_mutex);
    if (dev < 0 || dev >= 64) return DeviceInfo{};
    if (!g_dev[dev].ok) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            g_dev[dev].n_cu = prop.multiProcessorCount;
            g_dev[dev].ok = true;
        }
    }
    return g_dev[dev];
}

constexpr int64_t kI32Max = 2147483647;

// Each device's address of `scratch`, taken once per device with that device
// current (at handle creation, or at the first no-alloc product).
std::mutex g_scratch_mutex;
void *g_scratch[64] = {};

vspmm_status static_scratch(int dev, void **p) {
    if (dev < 0 || dev >= 64) return VSPMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mutex);
    if (!g_scratch[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return VSPMM_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return VSPMM_ERR_HIP;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr) return VSPMM_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *p = g_scratch[dev];
    return VSPMM_OK;
}

// Waves per block of the k_vcs_seg walks over a layout's own slices.
constexpr int kSegWaves = 16;

bool fits_i32(int64_t x) { return x >= 0 && x <= kI32Max; }

int ilog2_floor(int64_t x) {
    int l = 0;
    while ((int64_t(1) << (l + 1)) <= x) ++l;
    return l;
}

int ilog2_ceil(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

int key_bits(int64_t n_keys) {  // bits holding every key in [0, n_keys)
    return n_keys <= 1 ? 0 : ilog2_ceil(n_keys);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Entries per row block of an int64 CSR at most (int32 offsets inside a
// block keep clear of overflow, e.g. a position plus a round of windows).
constexpr int64_t kBlockMaxNnz = int64_t(1) << 30;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Direction geometry: aligned when the output's rows are the major slices.
bool is_aligned(const vspmm_matrix_s &h, int dir) {
    return (h.layout != VSPMM_VCSC) == (dir == VSPMM_AB);
}

int64_t n_in(const vspmm_matrix_s &h, int dir) { return dir == VSPMM_AB ? h.n_cols : h.n_rows; }
int64_t n_out(const vspmm_matrix_s &h, int dir) { return dir == VSPMM_AB ? h.n_rows : h.n_cols; }

// ------------------------------------------------------------------- plan

constexpr int64_t kLongMean = 1024;        // mean entries per slice for k_vcs_long

// Entries in one round of the short CSR walk (64 times its windows per round:
// 24 when the sums run in float32, 12 in float64). A CSR whose mean row is at
// least this long is walked by k_long (a group of waves per row); shorter rows
// fit a round of the short walk.
constexpr int64_t csr_round_entries(size_t elt) { return elt == 8 ? 64 * 12 : 64 * 24; }

// The lane split of one walk over a matrix with n_slices slices and nnz
// entries, at width w. Entry lanes G and width lanes WW are powers of two with
// G * WW <= 64; R = 64 / (G * WW) slices share a wave.
Plan make_plan(int64_t n_slices, int64_t nnz, int64_t w, size_t elt, bool split_matrix,
               int force_group, const void *B, const void *out, int n_cu,
               int64_t n_in = 0, bool vcs = false) {
    Plan pl;
    int vec = 1;
    for (int v = int(16 / elt); v > 1; v >>= 1) {
        if (w % v == 0 && aligned(B, v * elt) && aligned(out, v * elt)) {
            vec = v;
            break;
        }
    }
    pl.vec = vec;
    const int64_t units = (w + vec - 1) / vec;
    const int log_need = std::min(6, ilog2_ceil(std::max<int64_t>(units, 1)));
    int log_g, log_ww;
    if (force_group > 0) {
        log_g = ilog2_floor(force_group);
        log_ww = std::min(log_need, 6 - log_g);
    } else if (split_matrix) {
        const int64_t mean = n_slices > 0 ? nnz / n_slices : 0;
        log_g = std::min(6, ilog2_floor(std::max<int64_t>(mean, 1)));
        log_ww = std::min(log_need, 6 - log_g);
        // CSR with 16 or more entry lanes: idle width lanes fill the wave so
        // the short walk (one slice per wave, entry-balanced row ranges)
        // takes it; the entry lanes, and so a column's arithmetic, are the same
        if (!vcs && log_g >= 4) log_ww = 6 - log_g;
    } else {
        log_ww = log_need;
        log_g = 6 - log_ww;
    }
    pl.sp.log_g = log_g;
    pl.sp.log_ww = log_ww;
    pl.R = 64 >> (log_g + log_ww);
    const int64_t mean = n_slices > 0 ? nnz / n_slices : 0;
    const size_t b_bytes = size_t(n_in) * size_t(w) * elt;
    // the VCS walks address B with 32-bit byte offsets: a row number and the
    // row stride (w * elt bytes) each multiply in 24 bits
    const bool small_b = b_bytes < (size_t(1) << 32) && n_in < (int64_t(1) << 24) &&
                         size_t(w) * elt < (size_t(1) << 24);
    if (pl.R == 1 && (!vcs || small_b)) {
        if (mean >= (vcs ? kLongMean : csr_round_entries(elt))) {
            pl.kind = kLong;
            pl.block = 512;
            if (vcs) {
                // k_vcs_long: waves per slice so that the grid's waves fill the
                // chip (16 per CU) about once; twice over for rows of at most
                // 16 bytes, whose gathers are cheap enough that shorter pieces
                // pay (at wider rows the extra waves cost more L2 traffic)
                const int64_t target = int64_t(std::max(n_cu, 1)) *
                                       (size_t(w) * elt <= 16 ? 32 : 16);
                int wps = 1;
                while (wps < 8 && n_slices * wps * 2 <= target) wps *= 2;
                pl.wps = wps;
                const int64_t spb = 8 / wps;
                const int64_t blocks = (n_slices + spb - 1) / spb;
                pl.grid = int(std::max<int64_t>(1, std::min<int64_t>(blocks, int64_t(n_cu) * 8)));
            } else {
                // k_long: as many waves per row as the mean row fills passes of
                // the walk's windows, at most 8 (rows of ~1,000 entries get one
                // wave each); it follows the matrix, not the width
                const int64_t pass = csr_round_entries(elt);
                int wps = 1;
                while (wps < 8 && mean >= pass * wps * 2) wps *= 2;
                pl.wps = wps;
                const int64_t spb = 8 / wps;
                const int64_t blocks = (n_slices + spb - 1) / spb;
                pl.grid = int(std::max<int64_t>(1, std::min<int64_t>(blocks, int64_t(n_cu) * 16)));
            }
            return pl;
        }
        pl.kind = kShort;
        // dynamic LDS: the staged B (16-byte aligned) and per wave either a
        // ring of (index, value) pairs (CSR) or the round's group marks and
        // values (VCS)
        // CSR with 64 entry lanes takes the deep ring when B is staged in LDS
        // beside it (with B gathered from L2 it measured no better)
        const size_t ring_el = elt == 8 ? 16 : 8;  // bytes of a ring entry
        auto ring_of = [&](int n) { return vcs ? size_t(kRowsWaveLds) : size_t(n) * ring_el; };
        const size_t b_al = (b_bytes + 15) & ~size_t(15);
        if (!vcs && log_g == 6 && b_bytes > 0 && aligned(B, 16) &&
            b_al + 16 * ring_of(kRingDeep) <= kLdsMax)
            pl.ring = kRingDeep;
        const size_t ring = ring_of(pl.ring);
        // VCS: the block's slice-header table (two int arrays) and a counter
        auto extra = [&](int64_t grid) -> size_t {
            if (!vcs) return 0;
            return size_t(8) * size_t(rows_header_cap(int(n_slices), int(grid))) + 16;
        };
        const int64_t g1 = std::max(n_cu, 1);
        if (b_bytes > 0 && b_al + 16 * ring + extra(g1) <= kLdsMax && aligned(B, 16)) {
            pl.lds = true;
            pl.lds_bytes = b_al + 16 * ring + extra(g1);
            pl.block = 1024;
            pl.grid = int(g1);
        } else {
            // enough blocks that a block's header table stays small
            const int64_t g4 = std::max<int64_t>(g1 * 4, vcs ? (n_slices + 2047) / 2048 : 0);
            pl.lds_bytes = 4 * ring + extra(g4);
            pl.block = 256;
            pl.grid = int(g4);
            if (!vcs) {  // CSR: blocks of 8 waves, so a long-slice group fits one
                pl.lds_bytes = 8 * ring;
                pl.block = 512;
                pl.grid = int(g1 * 2);
            }
        }
        return pl;
    }
    const int64_t per_block = int64_t(pl.block / 64) * pl.R;
    const int64_t want = (n_slices + per_block - 1) / per_block;
    const int64_t cap = int64_t(std::max(n_cu, 1)) * 8;
    pl.grid = int(std::max<int64_t>(1, std::min(want, cap)));
    return pl;
}

// --------------------------------------------------------------- launches

vspmm_status hip_status() {
    return hipGetLastError() == hipSuccess ? VSPMM_OK : VSPMM_ERR_HIP;
}

void launch_zero(void *p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (!words) return;
    const size_t blocks = std::min<size_t>((words / 4 + 255) / 256 + 1, 4096);
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)p, words);
}

// Each slice's first entry (he) and the starts of the waves of a k_vcs_seg
// launch of `grid` blocks of `wpb` waves over a VCS (as `tiles` runs).
void seg_plan(int64_t n_slices, int64_t n_groups, const int32_t *sptr, const int32_t *vptr,
              int tiles, int grid, int wpb, int32_t *he, SegDesc *desc, int n_cu, hipStream_t s) {
    const int64_t n = n_slices + 1;
    const int g1 = int(std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, int64_t(n_cu) * 16)));
    hipLaunchKernelGGL(k_slice_starts, dim3(g1), dim3(256), 0, s, int(n_slices), int(n_groups),
                       sptr, vptr, he);
    const int nw = grid * wpb;
    hipLaunchKernelGGL(k_seg_plan, dim3((nw + 255) / 256), dim3(256), 0, s, int(n_slices),
                       int(n_groups), sptr, vptr, he, tiles, grid, wpb, desc);
}

// Attaches a k_vcs_seg plan to the walk's arguments.
template <typename T>
void with_seg(WalkArgs<T> &a, const int32_t *he, const SegDesc *desc, int grid, int wpb) {
    a.he = he;
    a.seg = desc;
    a.seg_grid = grid;
    a.seg_wpb = wpb;
}

template <typename T>
WalkArgs<T> walk_args(int64_t n_slices, const int32_t *sptr, const int32_t *vptr, const void *vals,
                      const int32_t *idx, const void *B, void *out, int w, int64_t n_in) {
    WalkArgs<T> a{int(n_slices), sptr, vptr, static_cast<const T *>(vals), idx,
                  static_cast<const T *>(B), static_cast<T *>(out), w, int(n_in)};
    a.n_b_rows = int(n_in);
    return a;
}

// For a float32-value CSR summed in float64: the walk reads its values (the
// handle's, or the built transpose's) as float32 and widens each one.
WalkArgs<double> values_of(const vspmm_matrix_s &h, WalkArgs<double> a) {
    if (h.dtype == VSPMM_F32_F64) {
        a.vals32 = reinterpret_cast<const float *>(a.vals);
        a.vals = nullptr;
    }
    return a;
}

// Dispatches one aligned walk to its kernel family.
template <typename T>
void launch_aligned(bool vcs, const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    if (pl.kind == kLong) {
        if constexpr (sizeof(T) == 4) {
            if (vcs) {
                if (pl.vec == 4) return launch_vcs_long<4>(pl, a, s);
                if (pl.vec == 2) return launch_vcs_long<2>(pl, a, s);
                return launch_vcs_long<1>(pl, a, s);
            }
        }
        return launch_long<false, T>(pl, a, s);
    }
    if (pl.kind == kShort) {
        if constexpr (sizeof(T) == 4) {
            if (vcs) {
                if (pl.vec == 4) return launch_vcs_rows<4>(pl, a, s);
                if (pl.vec == 2) return launch_vcs_rows<2>(pl, a, s);
                return launch_vcs_rows<1>(pl, a, s);
            }
        }
        return launch_short<T>(pl, a, s);
    }
    if constexpr (sizeof(T) == 4) {
        if (vcs) return launch_plain<true, T>(pl, a, s);
    }
    launch_plain<false, T>(pl, a, s);
}

// An aligned walk over the handle's own layout. For CSR with long rows, the
// short or plain walk leaves the rows longer than long_len to the long walk,
// which gives each listed row 8 waves (the same matrix-driven entry lanes and
// the same pieces in either form, so a column's arithmetic does not depend on
// the width): blocks of its own in front of the short walk's grid (same
// launch), or k_long after the plain walk.
template <typename T>
void launch_csr_or_vcs(const vspmm_matrix_s &h, bool vcs, const Plan &pl, WalkArgs<T> a,
                       int n_cu, hipStream_t s) {
    const bool split_long = !vcs && pl.kind != kLong && h.n_long > 0;
    if (split_long) {
        a.long_len = h.long_len;
        a.long_list = h.long_rows;
        a.n_long = int(h.n_long);
    }
    if (!vcs) {
        a.parts = h.parts;
        a.n_parts = h.n_parts;
    }
    if (split_long && pl.kind == kShort) {
        // the long slices get blocks of their own in the short walk's launch
        const int groups = pl.block / 512;
        a.long_blocks = int(std::min<int64_t>((h.n_long + groups - 1) / groups, n_cu));
        launch_aligned<T>(vcs, pl, a, s);
        return;
    }
    launch_aligned<T>(vcs, pl, a, s);
    if (split_long) {
        Plan pl2 = pl;
        pl2.kind = kLong;
        pl2.sp.log_ww = 6 - pl.sp.log_g;
        pl2.R = 1;
        pl2.lds = false;
        pl2.lds_bytes = 0;
        pl2.block = 512;
        pl2.grid = int(std::max<int64_t>(1, std::min<int64_t>(h.n_long, int64_t(n_cu) * 16)));
        launch_long<false, T>(pl2, a, s);
    }
}

// The scatter walk's plan: one column per lane, WW = w lanes per entry
// rounded up to a power of two (at most 64), a wave per balanced entry range.
// The adds' cost is set by the hardware's atomic rates: an L2 float atomic
// instruction costs about the same per 64-byte run it touches whether one
// lane or sixteen add into that run, while LDS float atomics go about one
// lane per three clocks per CU (measured: 12 G width-16 entries per second
// over the chip against 20 G for L2 atomics). So a block adds into a private LDS copy
// of out (then once per element into out) only when out fits in LDS, its
// rows are narrow (at most 32 bytes, where most of an L2 request would be
// idle) and enough blocks share the entries (32 per 4 bytes of row: with
// fewer CUs adding, the LDS adds fall behind the L2's). The copy's flush is
// coalesced, so a full grid costs it little.
Plan scatter_plan(int64_t nnz, int64_t w, int64_t no, size_t elt, int n_cu, int force_group) {
    Plan pl;
    pl.vec = 1;
    pl.sp.log_ww = std::min(6, ilog2_ceil(std::max<int64_t>(w, 1)));
    if (force_group > 0) pl.sp.log_ww = 6 - std::min(6, ilog2_floor(force_group));
    pl.sp.log_g = 6 - pl.sp.log_ww;
    pl.R = 0;  // entries, not slices, are balanced over the waves
    n_cu = std::max(n_cu, 1);
    const size_t out_bytes = size_t(no) * size_t(w) * elt;
    const int64_t priv_grid = std::min<int64_t>(n_cu, nnz / (2 * std::max<int64_t>(no, 1)));
    if (out_bytes > 0 && out_bytes <= kLdsMax && size_t(w) * elt <= 32 &&
        priv_grid >= int64_t(w) * int64_t(elt) * 8) {
        pl.lds = true;
        pl.lds_bytes = out_bytes;
        pl.block = 1024;
        pl.grid = int(priv_grid);
        return pl;
    }
    // waves of at least 8 windows, 16 waves per CU at most
    const int64_t waves = std::max<int64_t>(1, std::min<int64_t>((nnz + 511) / 512, int64_t(n_cu) * 16));
    pl.block = 256;
    pl.grid = int((waves + 3) / 4);
    return pl;
}

template <typename T>
void launch_scatter_any(bool vcs, const Plan &pl, const vspmm_matrix_s &h, const void *B,
                        void *out, int w, int64_t no, hipStream_t s) {
    ScatterArgs<T> a{int(h.n_major()), int(h.n_groups), int(h.nnz), h.sptr, h.vptr,
                     static_cast<const T *>(h.vals), h.idx, static_cast<const T *>(B),
                     static_cast<T *>(out), w, int(no)};
    if (h.dtype == VSPMM_F32_F64) {  // float32 values summed in float64
        a.vals32 = static_cast<const float *>(h.vals);
        a.vals = nullptr;
    }
    if constexpr (sizeof(T) == 4) {
        if (vcs) return launch_scatter<true, T>(pl, a, s);
    }
    launch_scatter<false, T>(pl, a, s);
}

// ------------------------------------------------------------- workspace

// Carves 256-byte aligned arrays out of a workspace (or only counts bytes
// when base is null).
struct Bump {
    char *base;
    size_t off = 0;
    template <typename T>
    T *take(size_t n) {
        off = align256(off);
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += std::max<size_t>(n, 1) * sizeof(T);
        return p;
    }
};

// A built layout (result, kept across calls) plus the build's scratch: the
// opposite layout (n_bins = the handle's minor count) or a tiled one (n_bins
// virtual slices, with a per-entry key array and the product's partial rows).
struct OppositeWs {
    // result
    int32_t *t_ptr = nullptr;      // n_bins + 1 (CSR row pointers / VCS major_ptr)
    void *t_vals = nullptr;        // CSR: nnz values; VCS: nnz group values (worst case)
    int32_t *t_vptr = nullptr;     // VCS: nnz + 1
    int32_t *t_idx = nullptr;      // nnz
    int32_t *t_ngroups = nullptr;  // VCS: 1
    float *partial = nullptr;      // tiled: the product's partial rows (n_bins x width)
    int32_t *t_he = nullptr;       // VCS: first entry of each new slice (n_bins + 1)
    SegDesc *t_seg = nullptr;      // VCS: the k_vcs_seg plan over it (seg_waves)
    // scratch
    int32_t *slice_of = nullptr, *group_of = nullptr, *vkey = nullptr;
    uint32_t *keys_a = nullptr, *keys_b = nullptr;
    int32_t *pay_a = nullptr, *pay_b = nullptr;
    int32_t *cnt = nullptr;
    int32_t *hist = nullptr, *bsums = nullptr, *scalars = nullptr;
    size_t bytes = 0;
};

OppositeWs carve_opposite(const vspmm_matrix_s &h, void *base, int64_t n_bins = -1,
                          int64_t partial_elems = 0, int64_t seg_waves = -1) {
    OppositeWs w;
    Bump b{static_cast<char *>(base)};
    const size_t nnz = size_t(h.nnz);
    const size_t nb = size_t(n_bins < 0 ? h.n_minor() : n_bins);
    const bool vcs = h.layout != VSPMM_CSR;
    const bool tiled = partial_elems > 0;
    w.t_ptr = b.take<int32_t>(nb + 1);
    w.t_vals = b.take<char>(nnz * h.val_elt());
    if (vcs) {
        w.t_vptr = b.take<int32_t>(nnz + 1);
        w.t_ngroups = b.take<int32_t>(1);
    }
    w.t_idx = b.take<int32_t>(nnz);
    if (tiled) w.partial = b.take<float>(size_t(partial_elems));
    if (vcs) {
        if (seg_waves < 0) {
            const DeviceInfo di = device_info(h.device);
            seg_waves = int64_t(di.ok ? di.n_cu : 256) * kSegWaves;
        }
        w.t_he = b.take<int32_t>(nb + 1);
        w.t_seg = b.take<SegDesc>(size_t(seg_waves));
    }
    w.slice_of = b.take<int32_t>(nnz);
    if (vcs) w.group_of = b.take<int32_t>(nnz);
    if (tiled) w.vkey = b.take<int32_t>(nnz);
    w.keys_a = b.take<uint32_t>(nnz);
    w.keys_b = b.take<uint32_t>(nnz);
    w.pay_a = b.take<int32_t>(nnz);
    w.pay_b = b.take<int32_t>(nnz);
    w.cnt = b.take<int32_t>(nb + 1);
    const size_t nblocks = (nnz + kSortTile - 1) / kSortTile;
    w.hist = b.take<int32_t>(256 * std::max<size_t>(nblocks, 1));
    const size_t scan_len = std::max({nnz, nb + 1, 256 * std::max<size_t>(nblocks, 1)});
    w.bsums = b.take<int32_t>((scan_len + kScanTile - 1) / kScanTile + 1);
    w.scalars = b.take<int32_t>(4);
    w.bytes = align256(b.off);
    return w;
}

// Exclusive scan of n ints (out may alias in); *total (device, optional) gets
// the sum.
void scan_excl(const int32_t *in, int32_t *out, int64_t n, int32_t *bsums, int32_t *total,
               hipStream_t s) {
    if (n <= 0) {
        if (total) launch_zero(total, 4, s);
        return;
    }
    const int nb = int((n + kScanTile - 1) / kScanTile);
    hipLaunchKernelGGL(k_scan_reduce, dim3(nb), dim3(256), 0, s, in, int(n), bsums);
    hipLaunchKernelGGL(k_scan_bsums, dim3(1), dim3(256), 0, s, bsums, nb, total);
    hipLaunchKernelGGL(k_scan_apply, dim3(nb), dim3(256), 0, s, in, int(n), bsums, out);
}

// Stable LSD radix sort of (keys, pay) on the low `bits` bits; the result ends
// in (*ka, *pa).
void radix_sort(uint32_t **ka, int32_t **pa, uint32_t **kb, int32_t **pb, int64_t n, int bits,
                int32_t *hist, int32_t *bsums, hipStream_t s) {
    if (n <= 0) return;
    const int nblocks = int((n + kSortTile - 1) / kSortTile);
    for (int shift = 0; shift < bits; shift += 8) {
        hipLaunchKernelGGL(k_radix_hist, dim3(nblocks), dim3(kSortThreads), 0, s, *ka, int(n),
                           shift, nblocks, hist);
        scan_excl(hist, hist, int64_t(256) * nblocks, bsums, nullptr, s);
        hipLaunchKernelGGL(k_radix_scatter, dim3(nblocks), dim3(kSortThreads), 0, s, *ka, *pa,
                           int(n), shift, nblocks, hist, *kb, *pb);
        std::swap(*ka, *kb);
        std::swap(*pa, *pb);
    }
}

int grid_for(int64_t n, int n_cu) {
    const int64_t want = (n + 255) / 256;
    return int(std::max<int64_t>(1, std::min<int64_t>(want, int64_t(std::max(n_cu, 1)) * 16)));
}

void expand_slices(const vspmm_matrix_s &h, const OppositeWs &w, int n_cu, hipStream_t s) {
    const int64_t nmaj = h.n_major();
    if (nmaj <= 0 || h.nnz <= 0) return;
    const int grid = int(std::max<int64_t>(1, std::min<int64_t>((nmaj + 3) / 4, n_cu * 16)));
    if (h.layout == VSPMM_CSR)
        hipLaunchKernelGGL(k_expand<false>, dim3(grid), dim3(256), 0, s, int(nmaj), h.sptr,
                           h.vptr, w.slice_of, w.group_of);
    else
        hipLaunchKernelGGL(k_expand<true>, dim3(grid), dim3(256), 0, s, int(nmaj), h.sptr,
                           h.vptr, w.slice_of, w.group_of);
}

// tptr[b] (b = 0 .. n_bins) = the first position of bin b in the sorted keys:
// the new slices' entry offsets, read off the sort instead of counted with
// atomics (nnz may be 0: then every offset is 0 and keys is not read).
void bin_starts(const uint32_t *keys, int64_t nnz, int64_t n_bins, int32_t *tptr, int n_cu,
                hipStream_t s) {
    hipLaunchKernelGGL(k_bin_starts, dim3(grid_for(nnz + 1, n_cu)), dim3(256), 0, s, int(nnz),
                       keys, int(n_bins), tptr);
}

// The exact CSR transpose into (t_ptr, t_idx, t_val); with factor (one per
// stored entry, in the handle's order), each value scaled by its own factor.
void build_transpose(const vspmm_matrix_s &h, const OppositeWs &w, int32_t *t_ptr,
                     int32_t *t_idx, void *t_val, int n_cu, hipStream_t s,
                     const void *factor = nullptr) {
    if (h.nnz <= 0) {
        bin_starts(nullptr, 0, h.n_minor(), t_ptr, n_cu, s);
        return;
    }
    expand_slices(h, w, n_cu, s);
    const int grid = grid_for(h.nnz, n_cu);
    uint32_t *ka = w.keys_a, *kb = w.keys_b;
    int32_t *pa = w.pay_a, *pb = w.pay_b;
    hipLaunchKernelGGL(k_index_keys, dim3(grid), dim3(256), 0, s, int(h.nnz), h.idx, ka, pa);
    radix_sort(&ka, &pa, &kb, &pb, h.nnz, key_bits(h.n_minor()), w.hist, w.bsums, s);
    bin_starts(ka, h.nnz, h.n_minor(), t_ptr, n_cu, s);
    if (h.val_elt() == 8)
        hipLaunchKernelGGL(k_transpose_emit<double>, dim3(grid), dim3(256), 0, s, int(h.nnz), pa,
                           w.slice_of, (const double *)h.vals, (const double *)factor, t_idx,
                           (double *)t_val);
    else
        hipLaunchKernelGGL(k_transpose_emit<float>, dim3(grid), dim3(256), 0, s, int(h.nnz), pa,
                           w.slice_of, (const float *)h.vals, (const float *)factor, t_idx,
                           (float *)t_val);
}

// A VCS expanded to one value per entry (vsparse page, section "Benchmarks":
// the expansion is index-sorted by default and takes a format). In the
// layout's own format: stored order, or each slice sorted by index (stable,
// so repeated indices keep their stored order) by one block per slice. In the
// other format: the exact transpose of the stored-order expansion (a global
// stable sort by index; each new slice lists its entries by ascending old
// slice).
void build_expand(const vspmm_matrix_s &h, bool own, bool sorted, const OppositeWs &w,
                  int32_t *ptr, int32_t *idx_out, float *val_out, int n_cu, hipStream_t s) {
    const int64_t nmaj = h.n_major(), nnz = h.nnz;
    const float *values = static_cast<const float *>(h.vals);
    const int grid = grid_for(std::max<int64_t>(nnz, 1), n_cu);
    if (own) {
        hipLaunchKernelGGL(k_expand_ptr, dim3(grid_for(nmaj + 1, n_cu)), dim3(256), 0, s,
                           int(nmaj), h.sptr, h.vptr, ptr);
        if (nnz <= 0) return;
        if (!sorted) {
            const int g = int(std::max<int64_t>(1, std::min<int64_t>((nmaj + 3) / 4, n_cu * 16)));
            hipLaunchKernelGGL(k_expand_copy, dim3(g), dim3(256), 0, s, int(nmaj), h.sptr, h.vptr,
                               values, h.idx, idx_out, val_out);
            return;
        }
        // sorted: each slice by one block (in LDS, or a block radix sort
        // through the workspace for a slice longer than the LDS holds)
        const bool small = nnz / std::max<int64_t>(nmaj, 1) <= 128;
        const int g = int(std::max<int64_t>(1, std::min<int64_t>(nmaj, int64_t(n_cu) *
                                                                     (small ? 32 : 8))));
        const int bits = key_bits(h.n_minor());
        float *vb = reinterpret_cast<float *>(w.group_of);
        if (small)
            hipLaunchKernelGGL((k_expand_sorted<64, 512>), dim3(g), dim3(64), 0, s, int(nmaj),
                               h.sptr, h.vptr, values, h.idx, bits, w.keys_a, w.pay_a, w.keys_b,
                               w.pay_b, vb, idx_out, val_out);
        else
            hipLaunchKernelGGL((k_expand_sorted<256, 2048>), dim3(g), dim3(256), 0, s, int(nmaj),
                               h.sptr, h.vptr, values, h.idx, bits, w.keys_a, w.pay_a, w.keys_b,
                               w.pay_b, vb, idx_out, val_out);
        return;
    } else if (nnz <= 0) {
        bin_starts(nullptr, 0, h.n_minor(), ptr, n_cu, s);
        return;
    }
    expand_slices(h, w, n_cu, s);
    uint32_t *ka = w.keys_a, *kb = w.keys_b;
    int32_t *pa = w.pay_a, *pb = w.pay_b;
    hipLaunchKernelGGL(k_index_keys, dim3(grid), dim3(256), 0, s, int(nnz), h.idx, ka, pa);
    radix_sort(&ka, &pa, &kb, &pb, nnz, key_bits(h.n_minor()), w.hist, w.bsums, s);
    bin_starts(ka, nnz, h.n_minor(), ptr, n_cu, s);
    hipLaunchKernelGGL(k_expand_emit, dim3(grid), dim3(256), 0, s, int(nnz), pa, w.slice_of,
                       w.group_of, values, idx_out, val_out);
}

// The VCS regrouped by the other axis into (t_major_ptr, t_values,
// t_value_ptr, t_indices, t_n_groups).
void build_regroup(const vspmm_matrix_s &h, const OppositeWs &w, int32_t *t_major_ptr,
                   float *t_values, int32_t *t_value_ptr, int32_t *t_indices,
                   int32_t *t_n_groups, int n_cu, hipStream_t s) {
    int32_t *tptr = w.cnt;  // entry offsets of the new slices
    const int64_t nnz = h.nnz;
    const int grid = grid_for(std::max<int64_t>(nnz, 1), n_cu);
    int32_t *n_groups = w.scalars;
    int32_t *gid = w.pay_b;  // (not read when nnz is 0)
    if (nnz > 0) {
        expand_slices(h, w, n_cu, s);
        uint32_t *ka = w.keys_a, *kb = w.keys_b;
        int32_t *pa = w.pay_a, *pb = w.pay_b;
        hipLaunchKernelGGL(k_value_keys, dim3(grid), dim3(256), 0, s, int(nnz), w.group_of,
                           (const float *)h.vals, ka, pa);
        radix_sort(&ka, &pa, &kb, &pb, nnz, 32, w.hist, w.bsums, s);
        hipLaunchKernelGGL(k_gather_index, dim3(grid), dim3(256), 0, s, int(nnz), pa, h.idx, ka);
        radix_sort(&ka, &pa, &kb, &pb, nnz, key_bits(h.n_minor()), w.hist, w.bsums, s);
        bin_starts(ka, nnz, h.n_minor(), tptr, n_cu, s);
        // the sort's other key and payload arrays are free now: group flags
        // and group numbers
        int32_t *flag = reinterpret_cast<int32_t *>(kb);
        gid = pb;
        hipLaunchKernelGGL(k_group_flags, dim3(grid), dim3(256), 0, s, int(nnz), pa, ka,
                           w.group_of, (const float *)h.vals, flag);
        scan_excl(flag, gid, nnz, w.bsums, n_groups, s);
        hipLaunchKernelGGL(k_group_emit, dim3(grid), dim3(256), 0, s, int(nnz), pa, w.slice_of,
                           w.group_of, (const float *)h.vals, flag, gid, t_values,
                           t_value_ptr, t_indices);
    } else {
        launch_zero(n_groups, 4, s);
        bin_starts(nullptr, 0, h.n_minor(), tptr, n_cu, s);
    }
    const int g2 = grid_for(h.n_minor() + 1, n_cu);
    hipLaunchKernelGGL(k_group_major_ptr, dim3(g2), dim3(256), 0, s, int(h.n_minor()), int(nnz),
                       tptr, gid, n_groups, t_major_ptr, t_value_ptr, t_n_groups);
}

// ------------------------------------------------------------ tiled layout

// A tiled walk: the product's input rows (B's rows) are cut into tiles of tr
// rows, each small enough for one CU's LDS next to the walk's own LDS, and
// every entry goes to the virtual slice (tile, output row). The virtual
// slices form a VCS of tiles x n_out slices with tile-local indices, walked by
// k_vcs_rows with each block staging its tile of B; the tiles' partial rows
// are then added in a fixed order. It pays where the untiled walks are bound
// by L2 gather requests: B does not fit in LDS whole, B's rows are at most 64
// bytes (one request each; wider rows gather from L2 at a better rate per
// byte, and there the tiles measured slower) and the virtual slices keep at
// least 16 entries on average, so the partial rows cost little next to the
// entries.
struct TilePlan {
    bool ok = false;
    int tr = 0;          // B rows per tile (a multiple of 4)
    int tiles = 0;
    int64_t n_out = 0;   // output rows (virtual slices per tile)
    int64_t n_in = 0;    // B's rows
    Plan pl;             // the short walk's launch over the tiled layout
    int64_t n_bins() const { return int64_t(tiles) * n_out; }
};

// A B larger than one XCD's L2 (4 MB) is fetched from the Infinity Cache by
// every XCD when the walk gathers from global memory, and cut into LDS tiles
// it may need so many tiles that their partial rows (written and read back
// per (tile, output row)) outweigh the matrix, or its rows may be too wide for
// LDS tiles to pay. L2 tiles: B cut into a multiple of 8 tiles of about 2 MB,
// the blocks of a tile on one XCD (as for LDS tiles), as many blocks per tile
// as one XCD holds at once, so an XCD walks its tiles one after another with
// one tile in its L2; the walk gathers from global memory.
TilePlan tile_plan_l2(const vspmm_matrix_s &h, int64_t no, int64_t ni, int64_t w, int n_cu,
                      bool split_matrix, const void *B, const void *part) {
    TilePlan tp;
    const size_t row_bytes = size_t(w) * 4;
    constexpr size_t kL2Tile = size_t(2) << 20;
    const size_t b_bytes = size_t(ni) * row_bytes;
    if (b_bytes <= 2 * kL2Tile) return tp;  // B fits one XCD's L2 already
    int64_t tiles = int64_t((b_bytes + kL2Tile - 1) / kL2Tile);
    tiles = (tiles + 7) / 8 * 8;
    int64_t tr = (((ni + tiles - 1) / tiles) + 3) & ~int64_t(3);
    tiles = (ni + tr - 1) / tr;
    if (tiles % 8 != 0) return tp;  // the XCD mapping needs whole tiles per XCD
    const int64_t nv = tiles * no;
    if (!fits_i32(nv + 1) || ni >= (int64_t(1) << 24)) return tp;
    const int64_t mean = h.nnz / nv;
    if (mean < 16 || mean >= kLongMean) return tp;
    // blocks of 4 waves, four per CU: a tile gets one XCD's worth (its CUs
    // are an eighth of the chip), and at most 2,048 slices per block
    const int64_t bpt = std::max<int64_t>({int64_t(1), 4 * n_cu / 8, (no + 2047) / 2048});
    const int64_t grid = tiles * bpt;
    if (!fits_i32(grid)) return tp;
    Plan pl = make_plan(nv, h.nnz, w, 4, split_matrix, h.force_group, B, part, n_cu, tr, true);
    if (pl.kind != kShort || pl.R != 1) return tp;
    pl.lds = false;
    pl.block = 256;
    pl.grid = int(grid);
    pl.lds_bytes = size_t(4) * kRowsWaveLds + 16 + 8 * size_t(rows_header_cap(int(nv), int(grid)));
    tp.ok = true;
    tp.tr = int(tr);
    tp.tiles = int(tiles);
    tp.n_out = no;
    tp.n_in = ni;
    tp.pl = pl;
    return tp;
}

TilePlan tile_plan(const vspmm_matrix_s &h, int dir, int64_t w, int n_cu, bool split_matrix,
                   const void *B, const void *part) {
    TilePlan tp;
    if (h.layout == VSPMM_CSR || h.dtype != VSPMM_F32 || w <= 0 || h.nnz <= 0) return tp;
    n_cu = std::max(n_cu, 1);
    const int64_t no = n_out(h, dir), ni = n_in(h, dir);
    const size_t row_bytes = size_t(w) * 4;
    // rows over 64 bytes gather from L2 at a better rate per byte: L2 tiles
    // (for a B over 4 MB); rows of up to 64 bytes: LDS tiles, or L2 tiles for
    // a B over 4 MB when LDS tiles do not pay (1M x 20k, B @ A at width 8:
    // 248 LDS tiles, 0.76 ms, against 16 L2 tiles, 1.04 ms)
    if (row_bytes > 64) return tile_plan_l2(h, no, ni, w, n_cu, split_matrix, B, part);
    const bool big_b = size_t(ni) * row_bytes > (size_t(4) << 20);
    const size_t fixed = size_t(16) * kRowsWaveLds + 16;
    // B fits whole: the plain walks stage it already
    if (size_t(ni) * row_bytes + fixed + 8 * size_t(rows_header_cap(int(std::min<int64_t>(no, kI32Max)), n_cu)) <= kLdsMax)
        return tp;
    // the block's slice-header table: 8 bytes per slice, at most 2,048 slices
    // per block (blocks per tile are chosen below to keep it so)
    const size_t header_margin = 8 * (2048 + 8);
    const int64_t tr_max = int64_t((kLdsMax - fixed - header_margin) / row_bytes) & ~int64_t(3);
    if (tr_max < 64) return tp;  // rows too wide for a useful tile
    // the plan for a given least tile count (false when tiles do not pay)
    int64_t tr = 0, tiles = 0;
    Plan pl;
    auto try_tiles = [&](int64_t t0, bool whole_xcds) -> bool {
        tiles = t0;
        // a multiple of 8 tiles lets each XCD (8 on the chip) own whole
        // tiles, so a tile of B is fetched into one XCD's L2 instead of all
        // eight
        if (whole_xcds) tiles = (tiles + 7) / 8 * 8;
        tr = (((ni + tiles - 1) / tiles) + 3) & ~int64_t(3);  // balanced tiles
        // virtual slices too long for the short walk (a narrow B makes few,
        // large tiles): more tiles, a multiple of 8, until their mean is at
        // most 512 entries
        if (h.nnz / std::max<int64_t>(tiles * no, 1) >= kLongMean) {
            tiles = std::max<int64_t>(tiles, (h.nnz + no * 512 - 1) / (no * 512));
            tiles = (tiles + 7) / 8 * 8;
            tr = (((ni + tiles - 1) / tiles) + 3) & ~int64_t(3);
            if (tr < 64) return false;
        }
        tiles = (ni + tr - 1) / tr;  // (rounding tr may drop one)
        // B fits an XCD's L2 here, where the untiled walk gathers it at a
        // fair rate: tiles pay only while their partial rows (written, then
        // read back to be added) stay within half the matrix's own bytes (1M
        // x 20k at width 8: 8 tiles of 1M partial rows, 512 MB, against 0.9
        // GB, measured 1.24 ms tiled and 0.98 ms untiled)
        const size_t partial_traffic = 2 * size_t(tiles) * size_t(no) * row_bytes;
        const size_t matrix_bytes = 4 * size_t(h.n_major() + 1) + 8 * size_t(h.n_groups) + 4 +
                                    4 * size_t(h.nnz);
        if (2 * partial_traffic > matrix_bytes) return false;
        const int64_t nv = tiles * no;
        if (!fits_i32(nv + 1) || ni >= (int64_t(1) << 24)) return false;
        const int64_t mean = h.nnz / nv;
        if (mean < 16 || mean >= kLongMean) return false;
        // blocks per tile: enough to fill the chip, and enough that a block's
        // slice-header table (8 bytes per slice, in LDS) stays at 2,048
        // slices
        const int64_t bpt = std::max<int64_t>({int64_t(1), n_cu / tiles, (no + 2047) / 2048});
        const int64_t grid = tiles * bpt;
        if (!fits_i32(grid)) return false;
        const size_t b_al = (size_t(tr) * row_bytes + 15) & ~size_t(15);
        const size_t lds = b_al + fixed + 8 * size_t(rows_header_cap(int(nv), int(grid)));
        if (lds > kLdsMax) return false;
        pl = make_plan(nv, h.nnz, w, 4, split_matrix, h.force_group, B, part, n_cu, tr, true);
        if (pl.kind != kShort || pl.R != 1) return false;
        pl.lds = true;
        pl.lds_bytes = lds;
        pl.block = 1024;
        pl.grid = int(grid);
        return true;
    };
    // the fewest tiles that fit LDS, as a multiple of 8 where four or more;
    // when the partial rows of that many outweigh the matrix (a B of a few
    // hundred KB over a million output rows), the fewest tiles as they are:
    // such a B is cheap to fetch into every XCD's L2 (1M x 20k at width 8:
    // 5 tiles against 8; on a 100,000 x 20,000 matrix 84 us tiled against
    // 108 untiled)
    const int64_t t_min = (ni + tr_max - 1) / tr_max;
    if (!try_tiles(t_min, t_min >= 4) && !(t_min >= 4 && t_min % 8 != 0 && try_tiles(t_min, false)))
        return big_b ? tile_plan_l2(h, no, ni, w, n_cu, split_matrix, B, part) : tp;
    tp.ok = true;
    tp.tr = int(tr);
    tp.tiles = int(tiles);
    tp.n_out = no;
    tp.n_in = ni;
    tp.pl = pl;
    return tp;
}

// Workspace bytes of a tiled product at width w.
// Waves of a tiled walk's launch (one k_vcs_seg start each).
int64_t tiled_waves(const TilePlan &tp) { return int64_t(tp.pl.grid) * (tp.pl.block / 64); }

size_t tiled_ws_bytes(const vspmm_matrix_s &h, const TilePlan &tp, int64_t w) {
    return carve_opposite(h, nullptr, tp.n_bins(), tp.n_bins() * w, tiled_waves(tp)).bytes;
}

// Builds the tiled layout of a VCS handle into w: entries keyed by virtual
// slice, each slice's entries grouped by value (stable radix sorts by value,
// then by virtual slice), tile-local indices.
void build_tiled(const vspmm_matrix_s &h, const OppositeWs &w, const TilePlan &tp,
                 bool major_is_out, int n_cu, hipStream_t s) {
    const int64_t nnz = h.nnz, nb = tp.n_bins();
    const int grid = grid_for(nnz, n_cu);
    const float *vals = static_cast<const float *>(h.vals);
    int32_t *n_groups = w.scalars;
    expand_slices(h, w, n_cu, s);
    if (major_is_out)
        hipLaunchKernelGGL(k_tile_keys<true>, dim3(grid), dim3(256), 0, s, int(nnz), h.idx,
                           w.slice_of, tp.tr, int(tp.n_out), w.vkey);
    else
        hipLaunchKernelGGL(k_tile_keys<false>, dim3(grid), dim3(256), 0, s, int(nnz), h.idx,
                           w.slice_of, tp.tr, int(tp.n_out), w.vkey);
    uint32_t *ka = w.keys_a, *kb = w.keys_b;
    int32_t *pa = w.pay_a, *pb = w.pay_b;
    hipLaunchKernelGGL(k_value_keys, dim3(grid), dim3(256), 0, s, int(nnz), w.group_of, vals, ka,
                       pa);
    radix_sort(&ka, &pa, &kb, &pb, nnz, 32, w.hist, w.bsums, s);
    hipLaunchKernelGGL(k_gather_index, dim3(grid), dim3(256), 0, s, int(nnz), pa, w.vkey, ka);
    radix_sort(&ka, &pa, &kb, &pb, nnz, key_bits(nb), w.hist, w.bsums, s);
    bin_starts(ka, nnz, nb, w.cnt, n_cu, s);
    // group flags and numbers in the sort's free key and payload arrays
    int32_t *flag = reinterpret_cast<int32_t *>(kb), *gid = pb;
    hipLaunchKernelGGL(k_group_flags, dim3(grid), dim3(256), 0, s, int(nnz), pa, ka, w.group_of,
                       vals, flag);
    scan_excl(flag, gid, nnz, w.bsums, n_groups, s);
    hipLaunchKernelGGL(k_group_emit, dim3(grid), dim3(256), 0, s, int(nnz), pa, w.slice_of,
                       w.group_of, vals, flag, gid, (float *)w.t_vals, w.t_vptr, w.t_idx);
    hipLaunchKernelGGL(k_group_major_ptr, dim3(grid_for(nb + 1, n_cu)), dim3(256), 0, s, int(nb),
                       int(nnz), w.cnt, gid, n_groups, w.t_ptr, w.t_vptr, w.t_ngroups);
    // (the tiled copy holds at most nnz groups; its pointers bound the reads)
    seg_plan(nb, nnz, w.t_ptr, w.t_vptr, tp.tiles, tp.pl.grid, tp.pl.block / 64, w.t_he, w.t_seg,
             n_cu, s);
}

// The tiled product over a built tiled copy L: the walk writes one partial
// row per (tile, output row) into L.partial, then the tiles' partial rows are
// added in tile order into out.
vspmm_status walk_tiled(const TilePlan &tp, const OppositeWs &L, const void *B, void *out, int w,
                        int n_cu, hipStream_t s) {
    WalkArgs<float> a = walk_args<float>(tp.n_bins(), L.t_ptr, L.t_vptr, L.t_vals, L.t_idx, B,
                                         L.partial, w, tp.tr);
    a.tiles = tp.tiles;
    a.n_b_rows = int(tp.n_in);
    with_seg(a, L.t_he, L.t_seg, tp.pl.grid, tp.pl.block / 64);
    launch_aligned<float>(true, tp.pl, a, s);
    const size_t n = size_t(tp.n_out) * size_t(w);
    const int grid = int(std::min<size_t>((n + 63) / 64, size_t(n_cu) * 16));
    hipLaunchKernelGGL(k_tile_sum, dim3(grid), dim3(256), 0, s, L.partial, (float *)out,
                       tp.tiles, n);
    return hip_status();
}

// Whether the walks split entry lanes by the matrix (a CSR's default) or by
// the width (a VCS's default).
bool split_of(const vspmm_matrix_s &h) {
    return (h.flags & VSPMM_SPLIT_MATRIX) ||
           (h.layout == VSPMM_CSR && !(h.flags & VSPMM_SPLIT_WIDTH));
}

// The opposite layout of h built into L: a CSR's exact transpose, or a VCS
// regrouped by the other axis with the k_vcs_seg plan over its slices.
void build_opposite(const vspmm_matrix_s &h, const OppositeWs &L, int n_cu, hipStream_t s) {
    if (h.layout == VSPMM_CSR) {
        build_transpose(h, L, L.t_ptr, L.t_idx, L.t_vals, n_cu, s);
        return;
    }
    build_regroup(h, L, L.t_ptr, (float *)L.t_vals, L.t_vptr, L.t_idx, L.t_ngroups, n_cu, s);
    // (the regrouped layout holds at most nnz groups; its pointers bound the reads)
    seg_plan(h.n_minor(), h.nnz, L.t_ptr, L.t_vptr, 1, n_cu, kSegWaves, L.t_he, L.t_seg, n_cu, s);
}

// Pass 2 of a deterministic misaligned product: the aligned walk over the
// opposite layout in L.
vspmm_status walk_opposite(const vspmm_matrix_s &h, const OppositeWs &L, const void *B, void *out,
                           int w, int n_cu, hipStream_t s) {
    const bool vcs = h.layout != VSPMM_CSR;
    const int64_t nmin = h.n_minor(), nmaj = h.n_major();
    const Plan pl = make_plan(nmin, h.nnz, w, h.elt(), split_of(h), h.force_group, B, out, n_cu,
                              nmaj, vcs);
    if (h.dtype != VSPMM_F32) {
        launch_aligned<double>(false, pl, values_of(h, walk_args<double>(nmin, L.t_ptr, nullptr,
                                                                         L.t_vals, L.t_idx, B,
                                                                         out, w, nmaj)), s);
    } else {
        WalkArgs<float> a = walk_args<float>(nmin, L.t_ptr, L.t_vptr, L.t_vals, L.t_idx, B, out,
                                             w, nmaj);
        if (vcs) with_seg(a, L.t_he, L.t_seg, n_cu, kSegWaves);
        launch_aligned<float>(vcs, pl, a, s);
    }
    return hip_status();
}

// ---------------------------------------------------------------- checks

vspmm_status check_handle(const vspmm_matrix_s *h) { return h ? VSPMM_OK : VSPMM_ERR_NULL; }

vspmm_status check_product(const vspmm_matrix_s &h, const void *B, void *out, int64_t width,
                           int dir) {
    if (dir != VSPMM_AB && dir != VSPMM_BA) return VSPMM_ERR_ENUM;
    if (width < 0 || !fits_i32(width)) return VSPMM_ERR_DIM;
    const int64_t ni = n_in(h, dir), no = n_out(h, dir);
    (void)ni;
    (void)no;
    if (width > 0 && ni > 0 && !B) return VSPMM_ERR_NULL;
    if (width > 0 && no > 0 && !out) return VSPMM_ERR_NULL;
    if (width > 0 && (!aligned(B, h.elt()) || !aligned(out, h.elt()))) return VSPMM_ERR_DIM;
    return VSPMM_OK;
}

vspmm_status run_blocked(const vspmm_matrix_s &h, const void *B, void *out, int w, int dir,
                         int mode, void *ws, size_t ws_bytes, hipStream_t s,
                         const vspmm_schedule_s *sc = nullptr);

// One product. With `accumulate`, a misaligned atomic product adds into out
// instead of overwriting it (used for the row blocks of an int64 CSR).
vspmm_status run_product(const vspmm_matrix_s &h, const void *B, void *out, int64_t width,
                         int dir, int mode, void *ws, size_t ws_bytes, hipStream_t s,
                         bool accumulate = false) {
    vspmm_status st = check_product(h, B, out, width, dir);
    if (st) return st;
    if (mode != VSPMM_ATOMIC && mode != VSPMM_DETERMINISTIC) return VSPMM_ERR_ENUM;
    const int64_t no = n_out(h, dir);
    if (width == 0 || no == 0) return VSPMM_OK;
    const DeviceInfo di = device_info(h.device);
    const int n_cu = di.ok ? di.n_cu : 256;
    const bool vcs = h.layout != VSPMM_CSR;
    const bool split_matrix = split_of(h);
    const int w = int(width);
    if (h.nnz == 0) {
        if (!accumulate) launch_zero(out, size_t(no) * size_t(w) * h.elt(), s);
        return hip_status();
    }
    if (h.ptr64) return run_blocked(h, B, out, w, dir, mode, ws, ws_bytes, s);
    if (mode == VSPMM_DETERMINISTIC && ws && aligned(ws, 256)) {
        const TilePlan tp = tile_plan(h, dir, w, n_cu, split_matrix, B, ws);
        if (tp.ok && ws_bytes >= tiled_ws_bytes(h, tp, w)) {
            const OppositeWs L = carve_opposite(h, ws, tp.n_bins(), tp.n_bins() * w,
                                                tiled_waves(tp));
            build_tiled(h, L, tp, is_aligned(h, dir), n_cu, s);
            return walk_tiled(tp, L, B, out, w, n_cu, s);
        }
    }
    if (is_aligned(h, dir)) {
        const int64_t ni = h.n_minor();
        const Plan pl = make_plan(h.n_major(), h.nnz, w, h.elt(), split_matrix, h.force_group,
                                  B, out, n_cu, ni, vcs);
        if (h.dtype != VSPMM_F32)
            launch_csr_or_vcs<double>(h, vcs, pl, values_of(h, walk_args<double>(
                                                              h.n_major(), h.sptr, h.vptr,
                                                              h.vals, h.idx, B, out, w, ni)),
                                      n_cu, s);
        else {
            WalkArgs<float> a = walk_args<float>(h.n_major(), h.sptr, h.vptr, h.vals, h.idx, B,
                                                 out, w, ni);
            if (vcs) with_seg(a, h.seg_he, h.seg_desc, h.seg_grid, kSegWaves);
            launch_csr_or_vcs<float>(h, vcs, pl, a, n_cu, s);
        }
        return hip_status();
    }
    if (mode == VSPMM_ATOMIC) {
        const Plan pl = scatter_plan(h.nnz, w, no, h.elt(), n_cu, h.force_group);
        if (!accumulate) launch_zero(out, size_t(no) * size_t(w) * h.elt(), s);
        if (h.dtype != VSPMM_F32) launch_scatter_any<double>(vcs, pl, h, B, out, w, no, s);
        else launch_scatter_any<float>(vcs, pl, h, B, out, w, no, s);
        return hip_status();
    }
    // deterministic: build the opposite layout in ws, then walk it aligned
    const OppositeWs need = carve_opposite(h, nullptr);
    if (!ws || ws_bytes < need.bytes || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
    const OppositeWs L = carve_opposite(h, ws);
    build_opposite(h, L, n_cu, s);
    if (vspmm_status st2 = hip_status()) return st2;
    return walk_opposite(h, L, B, out, w, n_cu, s);
}

}  // namespace

// A deterministic product's pass-2 layout, built once and kept in device
// memory the schedule owns, sized to what the walks read.
struct vspmm_schedule_s {
    const vspmm_matrix_s *h = nullptr;
    int dir = 0;
    int64_t width = 0;
    int kind = 0;         // a SchedKind
    TilePlan tp;          // kSchedTiled: the tile plan the copy was built for
    OppositeWs L;         // the built arrays, inside mem
    void *mem = nullptr;  // owned device memory
    size_t bytes = 0;
    // kSchedBlocked (int64 CSR, B @ A): one schedule per non-empty row block
    // (null for empty ones), and, with more than one, the buffer each later
    // block's product lands in before it is added to out (inside mem)
    std::vector<vspmm_schedule_s *> subs;
    void *sum = nullptr;
};

namespace {

// Workspace of a deterministic B @ A over an int64 CSR: one region for a row
// block's exact transpose (built again for each block, in stream order, so
// one region serves them all), then, with more than one non-empty block, the
// n_cols x width buffer each later block's product lands in before it is
// added to out.
struct BlockedWs {
    void *sub = nullptr;
    size_t sub_bytes = 0;
    void *sum = nullptr;
    size_t bytes = 0;
};

BlockedWs carve_blocked(const vspmm_matrix_s &h, void *base, int64_t width) {
    BlockedWs L;
    int live = 0;
    for (const vspmm_matrix_s *b : h.blocks) {
        if (b->nnz <= 0) continue;
        L.sub_bytes = std::max(L.sub_bytes, align256(carve_opposite(*b, nullptr).bytes));
        ++live;
    }
    L.sub = base;
    size_t off = L.sub_bytes;
    if (live > 1 && width > 0) {
        L.sum = base ? static_cast<char *>(base) + off : nullptr;
        off += align256(size_t(h.n_cols) * size_t(width) * h.elt());
    }
    L.bytes = off;
    return L;
}

void launch_accumulate(void *out, const void *sum, size_t n_el, size_t e, int n_cu,
                       hipStream_t s) {
    const unsigned g = (unsigned)std::min<size_t>((n_el + 255) / 256, size_t(n_cu) * 8);
    if (e == 8)
        hipLaunchKernelGGL(k_accumulate<double>, dim3(g), dim3(256), 0, s,
                           static_cast<double *>(out), static_cast<const double *>(sum), n_el);
    else
        hipLaunchKernelGGL(k_accumulate<float>, dim3(g), dim3(256), 0, s,
                           static_cast<float *>(out), static_cast<const float *>(sum), n_el);
}

vspmm_status schedule_product(const vspmm_schedule_s &sc, const void *B, void *out,
                              hipStream_t s);

// A product over an int64 CSR, block by block. A @ B: each block writes its
// own rows of out. B @ A: each block meets its rows of B and adds into all of
// out, with atomics (out zeroed once), or, deterministically, block 0's
// product written to out and each later block's added to it in block order,
// so the sum repeats bit for bit (each block's transpose built in ws, or taken
// from the schedule sc).
vspmm_status run_blocked(const vspmm_matrix_s &h, const void *B, void *out, int w, int dir,
                         int mode, void *ws, size_t ws_bytes, hipStream_t s,
                         const vspmm_schedule_s *sc) {
    const size_t e = h.elt();
    const size_t nb = h.blocks.size();
    if (dir == VSPMM_AB) {
        for (size_t b = 0; b < nb; ++b) {
            void *o = static_cast<char *>(out) + size_t(h.block_row0[b]) * size_t(w) * e;
            if (vspmm_status st = run_product(*h.blocks[b], B, o, w, dir, mode, nullptr, 0, s))
                return st;
        }
        return VSPMM_OK;
    }
    const size_t n_el = size_t(h.n_cols) * size_t(w);
    auto b_rows = [&](size_t b) {
        return static_cast<const char *>(B) + size_t(h.block_row0[b]) * size_t(w) * e;
    };
    if (mode == VSPMM_ATOMIC) {
        launch_zero(out, n_el * e, s);
        for (size_t b = 0; b < nb; ++b) {
            if (h.blocks[b]->nnz == 0) continue;
            if (vspmm_status st = run_product(*h.blocks[b], b_rows(b), out, w, dir, mode, nullptr,
                                              0, s, true))
                return st;
        }
        return hip_status();
    }
    BlockedWs L;
    if (sc) {
        L.sum = sc->sum;
    } else {
        const BlockedWs need = carve_blocked(h, nullptr, w);
        if (!ws || ws_bytes < need.bytes || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
        L = carve_blocked(h, ws, w);
    }
    const DeviceInfo di = device_info(h.device);
    const int n_cu = di.ok ? di.n_cu : 256;
    bool first = true;
    for (size_t b = 0; b < nb; ++b) {
        if (h.blocks[b]->nnz == 0) continue;
        void *dst = first ? out : L.sum;
        const vspmm_status st =
            sc ? schedule_product(*sc->subs[b], b_rows(b), dst, s)
               : run_product(*h.blocks[b], b_rows(b), dst, w, dir, mode, L.sub, L.sub_bytes, s);
        if (st) return st;
        if (!first) launch_accumulate(out, L.sum, n_el, e, n_cu, s);
        first = false;
    }
    return hip_status();
}

// ------------------------------------------------------------ views

void launch_scale_rows(void *dst, const void *src, const void *stat, int64_t n_rows, int w,
                       size_t e, int n_cu, hipStream_t s) {
    const int64_t chunks = (w + 63) / 64;
    const int64_t waves = std::max<int64_t>(1, n_rows * chunks);
    const unsigned g = (unsigned)std::min<int64_t>((waves + 3) / 4, int64_t(n_cu) * 16);
    if (e == 8)
        hipLaunchKernelGGL(k_scale_rows<double>, dim3(g), dim3(256), 0, s,
                           static_cast<double *>(dst), static_cast<const double *>(src),
                           static_cast<const double *>(stat), (long long)n_rows, w);
    else
        hipLaunchKernelGGL(k_scale_rows<float>, dim3(g), dim3(256), 0, s,
                           static_cast<float *>(dst), static_cast<const float *>(src),
                           static_cast<const float *>(stat), (long long)n_rows, w);
}

// A product under the handle's normalized view. With VSPMM_VIEW_SCALE the
// product is diag(out_stat) A diag(in_stat) B: B's rows scaled by the
// statistic of their axis into the handle's buffer, the walk (`walk`, any of
// the product paths) over that, then out's rows scaled by the other axis's
// statistic.
template <typename F>
vspmm_status with_view(const vspmm_matrix_s &h, const void *B, void *out, int64_t width, int dir,
                       hipStream_t s, F walk) {
    if (h.view == VSPMM_VIEW_IDENTITY) return walk(B);
    if (width > h.view_width) return VSPMM_ERR_DIM;
    const int64_t ni = n_in(h, dir), no = n_out(h, dir);
    if (width == 0 || no == 0) return walk(B);
    const DeviceInfo di = device_info(h.device);
    const int n_cu = di.ok ? di.n_cu : 256;
    const void *in_stat = dir == VSPMM_AB ? h.col_stat : h.row_stat;
    const void *out_stat = dir == VSPMM_AB ? h.row_stat : h.col_stat;
    if (ni > 0) launch_scale_rows(h.view_buf, B, in_stat, ni, int(width), h.elt(), n_cu, s);
    if (vspmm_status st = walk(ni > 0 ? h.view_buf : B)) return st;
    launch_scale_rows(out, out, out_stat, no, int(width), h.elt(), n_cu, s);
    return hip_status();
}

// ------------------------------------------------------------- schedules

enum SchedKind { kSchedPlain = 0, kSchedOpposite = 1, kSchedTiled = 2, kSchedBlocked = 3 };

void schedule_free(vspmm_schedule_s *sc) {
    if (!sc) return;
    for (vspmm_schedule_s *sub : sc->subs) schedule_free(sub);
    if (sc->mem) (void)hipFree(sc->mem);
    delete sc;
}

// The resident arrays of a built layout: the pointers, the group values and
// pointers at the realized group count G (VCS), the indices, the k_vcs_seg
// plan, and (tiled) the product's partial rows.
OppositeWs carve_resident(const vspmm_matrix_s &h, void *base, int64_t n_bins, int64_t G,
                          int64_t partial_elems, int64_t seg_waves) {
    OppositeWs r;
    Bump b{static_cast<char *>(base)};
    const size_t nnz = size_t(h.nnz), nb = size_t(n_bins);
    const bool vcs = h.layout != VSPMM_CSR;
    r.t_ptr = b.take<int32_t>(nb + 1);
    r.t_vals = b.take<char>((vcs ? size_t(G) : nnz) * h.val_elt());
    if (vcs) r.t_vptr = b.take<int32_t>(size_t(G) + 1);
    r.t_idx = b.take<int32_t>(nnz);
    if (partial_elems > 0) r.partial = b.take<float>(size_t(partial_elems));
    if (vcs) {
        r.t_he = b.take<int32_t>(nb + 1);
        r.t_seg = b.take<SegDesc>(size_t(seg_waves));
    }
    r.bytes = align256(b.off);
    return r;
}

vspmm_status copy_d2d(void *dst, const void *src, size_t bytes, hipStream_t s) {
    if (!bytes) return VSPMM_OK;
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) == hipSuccess
               ? VSPMM_OK
               : VSPMM_ERR_HIP;
}

// Builds the layout of sc (kind, tp set) in scratch S, reads back its group
// count, and keeps an exact-size copy in memory the schedule owns. Waits for
// the stream.
vspmm_status schedule_fill(vspmm_schedule_s *sc, const OppositeWs &S, int n_cu, hipStream_t s) {
    const vspmm_matrix_s &h = *sc->h;
    const bool vcs = h.layout != VSPMM_CSR;
    const bool tiled = sc->kind == kSchedTiled;
    const int64_t nb = tiled ? sc->tp.n_bins() : h.n_minor();
    const int64_t seg_waves = tiled ? tiled_waves(sc->tp) : int64_t(n_cu) * kSegWaves;
    if (tiled)
        build_tiled(h, S, sc->tp, is_aligned(h, sc->dir), n_cu, s);
    else
        build_opposite(h, S, n_cu, s);
    if (vspmm_status st = hip_status()) return st;
    int32_t G = 0;
    if (vcs && hipMemcpyAsync(&G, S.t_ngroups, sizeof(G), hipMemcpyDeviceToHost, s) != hipSuccess)
        return VSPMM_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return VSPMM_ERR_HIP;
    if (G < 0 || G > h.nnz) return VSPMM_ERR_HIP;
    const int64_t partial = tiled ? nb * sc->width : 0;
    const OppositeWs need = carve_resident(h, nullptr, nb, G, partial, seg_waves);
    if (hipMalloc(&sc->mem, need.bytes) != hipSuccess) {
        sc->mem = nullptr;
        return VSPMM_ERR_HIP;
    }
    sc->bytes = need.bytes;
    OppositeWs &R = sc->L;
    R = carve_resident(h, sc->mem, nb, G, partial, seg_waves);
    const size_t nnz = size_t(h.nnz);
    vspmm_status st = copy_d2d(R.t_ptr, S.t_ptr, size_t(nb + 1) * 4, s);
    if (!st) st = copy_d2d(R.t_vals, S.t_vals, (vcs ? size_t(G) : nnz) * h.val_elt(), s);
    if (!st && vcs) st = copy_d2d(R.t_vptr, S.t_vptr, (size_t(G) + 1) * 4, s);
    if (!st) st = copy_d2d(R.t_idx, S.t_idx, nnz * 4, s);
    if (!st && vcs) st = copy_d2d(R.t_he, S.t_he, size_t(nb + 1) * 4, s);
    if (!st && vcs) st = copy_d2d(R.t_seg, S.t_seg, size_t(seg_waves) * sizeof(SegDesc), s);
    if (!st && hipStreamSynchronize(s) != hipSuccess) st = VSPMM_ERR_HIP;
    return st;
}

// Builds a schedule for (h, dir, width) in the build workspace build_ws of
// build_ws_bytes, or, when build_ws is null, in one of its own for the call.
vspmm_status schedule_build(vspmm_schedule_s *sc, void *build_ws, size_t build_ws_bytes,
                            hipStream_t s) {
    const vspmm_matrix_s &h = *sc->h;
    const DeviceInfo di = device_info(h.device);
    const int n_cu = di.ok ? di.n_cu : 256;
    size_t need = 0;
    if (h.ptr64) {
        if (sc->dir != VSPMM_BA || h.nnz == 0 || sc->width == 0) return VSPMM_OK;
        sc->kind = kSchedBlocked;
        const BlockedWs bw = carve_blocked(h, nullptr, sc->width);
        need = bw.sub_bytes;
    } else if (h.nnz > 0 && sc->width > 0) {
        alignas(256) static const float probe[64] = {};
        const TilePlan tp = tile_plan(h, sc->dir, sc->width, n_cu, split_of(h), probe, probe);
        if (tp.ok) {
            sc->kind = kSchedTiled;
            sc->tp = tp;
            need = tiled_ws_bytes(h, tp, sc->width);
        } else if (!is_aligned(h, sc->dir)) {
            sc->kind = kSchedOpposite;
            need = carve_opposite(h, nullptr).bytes;
        }
    }
    if (sc->kind == kSchedPlain) return VSPMM_OK;
    void *own = nullptr;
    if (build_ws) {
        if (build_ws_bytes < need || !aligned(build_ws, 256)) return VSPMM_ERR_WORKSPACE;
    } else {
        if (hipMalloc(&own, std::max<size_t>(need, 256)) != hipSuccess) return VSPMM_ERR_HIP;
        build_ws = own;
    }
    vspmm_status st = VSPMM_OK;
    if (sc->kind == kSchedBlocked) {
        sc->subs.assign(h.blocks.size(), nullptr);
        int live = 0;
        for (size_t b = 0; b < h.blocks.size() && !st; ++b) {
            if (h.blocks[b]->nnz == 0) continue;
            ++live;
            auto *sub = new (std::nothrow) vspmm_schedule_s{};
            if (!sub) {
                st = VSPMM_ERR_ALLOC;
                break;
            }
            sc->subs[b] = sub;
            sub->h = h.blocks[b];
            sub->dir = sc->dir;
            sub->width = sc->width;
            sub->kind = kSchedOpposite;
            st = schedule_fill(sub, carve_opposite(*sub->h, build_ws), n_cu, s);
        }
        if (!st && live > 1) {
            const size_t sum_bytes = size_t(h.n_cols) * size_t(sc->width) * h.elt();
            if (hipMalloc(&sc->mem, sum_bytes) != hipSuccess) {
                sc->mem = nullptr;
                st = VSPMM_ERR_HIP;
            } else {
                sc->sum = sc->mem;
                sc->bytes = sum_bytes;
            }
        }
    } else {
        const OppositeWs S =
            sc->kind == kSchedTiled
                ? carve_opposite(h, build_ws, sc->tp.n_bins(), sc->tp.n_bins() * sc->width,
                                 tiled_waves(sc->tp))
                : carve_opposite(h, build_ws);
        st = schedule_fill(sc, S, n_cu, s);
    }
    if (own) {
        if (hipStreamSynchronize(s) != hipSuccess && !st) st = VSPMM_ERR_HIP;
        (void)hipFree(own);
    }
    return st;
}

// One product through a built schedule.
vspmm_status schedule_product(const vspmm_schedule_s &sc, const void *B, void *out,
                              hipStream_t s) {
    const vspmm_matrix_s &h = *sc.h;
    const int w = int(sc.width);
    const DeviceInfo di = device_info(h.device);
    const int n_cu = di.ok ? di.n_cu : 256;
    switch (sc.kind) {
        case kSchedOpposite: return walk_opposite(h, sc.L, B, out, w, n_cu, s);
        case kSchedTiled: {
            // the launch's lane split follows B's alignment; the tiles, grid
            // and so the built copy and its plan do not
            const TilePlan tp = tile_plan(h, sc.dir, w, n_cu, split_of(h), B, sc.L.partial);
            if (!tp.ok || tp.tr != sc.tp.tr || tp.tiles != sc.tp.tiles ||
                tp.pl.grid != sc.tp.pl.grid || tp.pl.block != sc.tp.pl.block)
                return VSPMM_ERR_UNSUPPORTED;
            return walk_tiled(tp, sc.L, B, out, w, n_cu, s);
        }
        case kSchedBlocked:
            return run_blocked(h, B, out, w, sc.dir, VSPMM_DETERMINISTIC, nullptr, 0, s, &sc);
        default:
            return run_product(h, B, out, w, sc.dir, VSPMM_DETERMINISTIC, nullptr, 0, s);
    }
}

// Waves of the short CSR walk's grid (16 per CU), one entry-balanced row
// range each.
int csr_parts(int n_cu) { return 16 * std::max(n_cu, 1); }

// Rows the short walks leave to k_long: longer than one wave's share of the
// entries (nnz over the walk's waves, at least 64), and always those longer
// than one round of the short walk (64 * 24 entries for float32, 64 * 12 for
// float64). With entry-balanced row ranges a wave then walks about its share.
int csr_long_len(int dtype, int64_t nnz, int n_parts) {
    const int64_t round = csr_round_entries(dtype != VSPMM_F32 ? 8 : 4);
    const int64_t share = nnz / std::max(n_parts, 1);
    return int(std::min(round, std::max<int64_t>(64, share)));
}

// The handle's entry-balanced row ranges (no wait).
vspmm_status make_row_parts(vspmm_matrix_s *m, int n_cu, hipStream_t s) {
    if (m->n_rows <= 0) return VSPMM_OK;
    const int np = csr_parts(n_cu);
    if (hipMalloc(&m->parts, size_t(np + 1) * sizeof(int32_t)) != hipSuccess) {
        m->parts = nullptr;
        return VSPMM_ERR_HIP;
    }
    m->n_parts = np;
    hipLaunchKernelGGL(k_row_parts, dim3((np + 1 + 255) / 256), dim3(256), 0, s, int(m->n_rows),
                       m->sptr, (long long)m->nnz, np, m->parts);
    return hip_status();
}

// Lists a CSR handle's long rows on the device (count, read back, then fill
// an owned list). Waits for the stream once.
vspmm_status list_long_rows(vspmm_matrix_s *m, hipStream_t s) {
    const DeviceInfo di = device_info(m->device);
    m->long_len = csr_long_len(m->dtype, m->nnz, csr_parts(di.ok ? di.n_cu : 256));
    if (m->nnz <= 0 || m->n_rows <= 0) return VSPMM_OK;
    const int grid = grid_for(m->n_rows, di.ok ? di.n_cu : 256);
    int32_t *cnt = nullptr;
    if (hipMalloc(&cnt, sizeof(int32_t)) != hipSuccess) return VSPMM_ERR_HIP;
    int32_t host = 0;
    vspmm_status st = VSPMM_OK;
    launch_zero(cnt, sizeof(int32_t), s);
    hipLaunchKernelGGL(k_long_rows, dim3(grid), dim3(256), 0, s, int(m->n_rows), m->sptr,
                       m->long_len, cnt, (int32_t *)nullptr);
    if (hipMemcpyAsync(&host, cnt, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        st = VSPMM_ERR_HIP;
    } else if (host > 0) {
        if (hipMalloc(&m->long_rows, size_t(host) * sizeof(int32_t)) != hipSuccess) {
            st = VSPMM_ERR_HIP;
        } else {
            m->n_long = host;
            launch_zero(cnt, sizeof(int32_t), s);
            hipLaunchKernelGGL(k_long_rows, dim3(grid), dim3(256), 0, s, int(m->n_rows), m->sptr,
                               m->long_len, cnt, m->long_rows);
            if (hipStreamSynchronize(s) != hipSuccess) st = VSPMM_ERR_HIP;
        }
    }
    (void)hipFree(cnt);
    if (st == VSPMM_OK) st = hip_status();
    return st;
}

void free_handle(vspmm_matrix_s *m) {
    if (m->view_buf) (void)hipFree(m->view_buf);
    if (m->seg_he) (void)hipFree(m->seg_he);
    if (m->seg_desc) (void)hipFree(m->seg_desc);
    if (m->long_rows) (void)hipFree(m->long_rows);
    if (m->parts) (void)hipFree(m->parts);
    for (vspmm_matrix_s *b : m->blocks) vspmm_destroy(b);
    if (m->block_ptr) (void)hipFree(m->block_ptr);
    delete m;
}

vspmm_status finish_create(vspmm_matrix_s *m, vspmm_matrix *h, hipStream_t s) {
    if (hipGetDevice(&m->device) != hipSuccess) {
        delete m;
        return VSPMM_ERR_HIP;
    }
    // set-up of the no-alloc product on this device (a failure here is
    // reported by vspmm_spmm_noalloc, which tries again)
    void *unused = nullptr;
    (void)static_scratch(m->device, &unused);
    if (m->flags & VSPMM_VALIDATE) {
        const vspmm_status st = vspmm_validate(m, s);
        if (st) {
            delete m;
            return st;
        }
    }
    if (m->layout != VSPMM_CSR) {
        // the k_vcs_seg plan over the handle's own slices: n_cu blocks of
        // kSegWaves waves
        const DeviceInfo di = device_info(m->device);
        const int n_cu = di.ok ? di.n_cu : 256;
        const int64_t nmaj = m->n_major();
        if (hipMalloc(&m->seg_he, size_t(nmaj + 1) * sizeof(int32_t)) != hipSuccess ||
            hipMalloc(&m->seg_desc, size_t(n_cu) * kSegWaves * sizeof(SegDesc)) != hipSuccess) {
            free_handle(m);
            return VSPMM_ERR_HIP;
        }
        m->seg_grid = n_cu;
        seg_plan(nmaj, m->n_groups, m->sptr, m->vptr, 1, n_cu, kSegWaves, m->seg_he, m->seg_desc,
                 n_cu, s);
        if (vspmm_status st = hip_status()) {
            free_handle(m);
            return st;
        }
    }
    if (m->layout == VSPMM_CSR) {
        const DeviceInfo di = device_info(m->device);
        vspmm_status st = make_row_parts(m, di.ok ? di.n_cu : 256, s);
        if (!st) st = list_long_rows(m, s);
        if (st) {
            free_handle(m);
            return st;
        }
    }
    *h = m;
    return VSPMM_OK;
}

// Workspace of vspmm_assemble_csr: the element of each entry, the sort's key
// and payload pairs, its histograms and scan sums.
struct AssembleWs {
    int32_t *elem_of = nullptr;
    uint32_t *keys_a = nullptr, *keys_b = nullptr;
    int32_t *pay_a = nullptr, *pay_b = nullptr;
    int32_t *hist = nullptr, *bsums = nullptr;
    size_t bytes = 0;
};

AssembleWs carve_assemble(int64_t nnz, int64_t n_rows, void *base) {
    AssembleWs w;
    Bump b{static_cast<char *>(base)};
    const size_t n = size_t(std::max<int64_t>(nnz, 0));
    w.elem_of = b.take<int32_t>(n);
    w.keys_a = b.take<uint32_t>(n);
    w.keys_b = b.take<uint32_t>(n);
    w.pay_a = b.take<int32_t>(n);
    w.pay_b = b.take<int32_t>(n);
    const size_t nblocks = (n + kSortTile - 1) / kSortTile;
    w.hist = b.take<int32_t>(256 * std::max<size_t>(nblocks, 1));
    const size_t scan_len = std::max({n, size_t(n_rows) + 1, 256 * std::max<size_t>(nblocks, 1)});
    w.bsums = b.take<int32_t>((scan_len + kScanTile - 1) / kScanTile + 1);
    w.bytes = align256(b.off);
    return w;
}

// Rows and columns of an assembled operator (see vspmm_assemble_csr).
void role_dims(int role, int64_t n_elem, int64_t n_out, int64_t n_in, int64_t *rows,
               int64_t *cols) {
    *rows = role <= 1 ? n_elem * n_out : n_out;
    *cols = (role == 0 || role == 2) ? n_elem * n_in : n_in;
}

}  // namespace

// =================================================================== C ABI

extern "C" {

const char *vspmm_status_string(vspmm_status st) {
    switch (st) {
        case VSPMM_OK: return "ok";
        case VSPMM_ERR_NULL: return "a required pointer is null";
        case VSPMM_ERR_DIM: return "invalid or inconsistent extent";
        case VSPMM_ERR_ENUM: return "unknown layout, direction, dtype, mode or flag";
        case VSPMM_ERR_STRUCTURE: return "malformed sparse structure";
        case VSPMM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case VSPMM_ERR_UNSUPPORTED: return "unsupported request";
        case VSPMM_ERR_HIP: return "HIP call or kernel launch failed";
        case VSPMM_ERR_ALLOC: return "host allocation failed";
    }
    return "unknown status";
}

vspmm_status vspmm_create_vcs(vspmm_matrix *h, vspmm_layout layout, int64_t n_rows,
                              int64_t n_cols, int64_t n_groups, int64_t nnz,
                              const int32_t *major_ptr, const float *values,
                              const int32_t *value_ptr, const int32_t *indices, uint32_t flags,
                              int32_t force_group, hipStream_t stream) {
    if (!h) return VSPMM_ERR_NULL;
    if (layout != VSPMM_VCSR && layout != VSPMM_VCSC) return VSPMM_ERR_ENUM;
    if (flags & ~uint32_t(VSPMM_SPLIT_WIDTH | VSPMM_SPLIT_MATRIX | VSPMM_VALIDATE))
        return VSPMM_ERR_ENUM;
    if ((flags & VSPMM_SPLIT_WIDTH) && (flags & VSPMM_SPLIT_MATRIX)) return VSPMM_ERR_ENUM;
    if (!fits_i32(n_rows) || !fits_i32(n_cols) || !fits_i32(n_groups) || !fits_i32(nnz) ||
        n_rows + 1 > kI32Max || n_cols + 1 > kI32Max || n_groups + 1 > kI32Max)
        return VSPMM_ERR_DIM;
    if (force_group < 0 || force_group > 64 || (force_group & (force_group - 1)))
        return VSPMM_ERR_DIM;
    if (!major_ptr || !value_ptr) return VSPMM_ERR_NULL;
    if ((n_groups > 0 && !values) || (nnz > 0 && !indices)) return VSPMM_ERR_NULL;
    auto *m = new (std::nothrow) vspmm_matrix_s{};
    if (!m) return VSPMM_ERR_ALLOC;
    m->layout = layout;
    m->n_rows = n_rows;
    m->n_cols = n_cols;
    m->n_groups = n_groups;
    m->nnz = nnz;
    m->sptr = major_ptr;
    m->vals = values;
    m->vptr = value_ptr;
    m->idx = indices;
    m->dtype = VSPMM_F32;
    m->flags = flags;
    m->force_group = force_group;
    return finish_create(m, h, stream);
}

vspmm_status vspmm_create_csr(vspmm_matrix *h, int64_t n_rows, int64_t n_cols, int64_t nnz,
                              const int32_t *row_ptr, const int32_t *col, const void *val,
                              vspmm_dtype dtype, uint32_t flags, int32_t force_group,
                              hipStream_t stream) {
    if (!h) return VSPMM_ERR_NULL;
    if (dtype != VSPMM_F32 && dtype != VSPMM_F64 && dtype != VSPMM_F32_F64) return VSPMM_ERR_ENUM;
    if (flags & ~uint32_t(VSPMM_SPLIT_WIDTH | VSPMM_SPLIT_MATRIX | VSPMM_VALIDATE))
        return VSPMM_ERR_ENUM;
    if ((flags & VSPMM_SPLIT_WIDTH) && (flags & VSPMM_SPLIT_MATRIX)) return VSPMM_ERR_ENUM;
    if (!fits_i32(n_rows) || !fits_i32(n_cols) || !fits_i32(nnz) || n_rows + 1 > kI32Max ||
        n_cols + 1 > kI32Max)
        return VSPMM_ERR_DIM;
    if (force_group < 0 || force_group > 64 || (force_group & (force_group - 1)))
        return VSPMM_ERR_DIM;
    if (!row_ptr) return VSPMM_ERR_NULL;
    if (nnz > 0 && (!col || !val)) return VSPMM_ERR_NULL;
    auto *m = new (std::nothrow) vspmm_matrix_s{};
    if (!m) return VSPMM_ERR_ALLOC;
    m->layout = VSPMM_CSR;
    m->n_rows = n_rows;
    m->n_cols = n_cols;
    m->n_groups = 0;
    m->nnz = nnz;
    m->sptr = row_ptr;
    m->vals = val;
    m->vptr = nullptr;
    m->idx = col;
    m->dtype = dtype;
    m->flags = flags;
    m->force_group = force_group;
    return finish_create(m, h, stream);
}

vspmm_status vspmm_create_csr64(vspmm_matrix *h, int64_t n_rows, int64_t n_cols, int64_t nnz,
                                const int64_t *row_ptr, const int32_t *col, const void *val,
                                vspmm_dtype dtype, uint32_t flags, int32_t force_group,
                                int64_t block_nnz, hipStream_t stream) {
    if (!h) return VSPMM_ERR_NULL;
    if (dtype != VSPMM_F32 && dtype != VSPMM_F64 && dtype != VSPMM_F32_F64) return VSPMM_ERR_ENUM;
    if (flags & ~uint32_t(VSPMM_SPLIT_WIDTH | VSPMM_SPLIT_MATRIX | VSPMM_VALIDATE))
        return VSPMM_ERR_ENUM;
    if ((flags & VSPMM_SPLIT_WIDTH) && (flags & VSPMM_SPLIT_MATRIX)) return VSPMM_ERR_ENUM;
    if (!fits_i32(n_rows) || !fits_i32(n_cols) || n_rows + 1 > kI32Max || n_cols + 1 > kI32Max ||
        nnz < 0)
        return VSPMM_ERR_DIM;
    if (block_nnz == 0) block_nnz = kBlockMaxNnz;
    if (block_nnz < 1 || block_nnz > kBlockMaxNnz) return VSPMM_ERR_DIM;
    if (force_group < 0 || force_group > 64 || (force_group & (force_group - 1)))
        return VSPMM_ERR_DIM;
    if (!row_ptr) return VSPMM_ERR_NULL;
    if (nnz > 0 && (!col || !val)) return VSPMM_ERR_NULL;
    // the row pointers on the host: their checks and the block cuts
    std::vector<int64_t> rp;
    try {
        rp.resize(size_t(n_rows) + 1);
    } catch (...) {
        return VSPMM_ERR_ALLOC;
    }
    if (hipMemcpyAsync(rp.data(), row_ptr, rp.size() * sizeof(int64_t), hipMemcpyDeviceToHost,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return VSPMM_ERR_HIP;
    if (rp[0] != 0 || rp[size_t(n_rows)] != nnz) return VSPMM_ERR_STRUCTURE;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rp[size_t(r) + 1] < rp[size_t(r)]) return VSPMM_ERR_STRUCTURE;
    auto *m = new (std::nothrow) vspmm_matrix_s{};
    if (!m) return VSPMM_ERR_ALLOC;
    m->layout = VSPMM_CSR;
    m->n_rows = n_rows;
    m->n_cols = n_cols;
    m->nnz = nnz;
    m->sptr = nullptr;
    m->vals = val;
    m->idx = col;
    m->dtype = dtype;
    m->flags = flags;
    m->force_group = force_group;
    m->ptr64 = true;
    if (hipGetDevice(&m->device) != hipSuccess) {
        delete m;
        return VSPMM_ERR_HIP;
    }
    // blocks of whole rows, each of at most block_nnz entries unless one row
    // alone holds more (then at most 2^30)
    std::vector<int32_t> ptr32;
    try {
        for (int64_t r0 = 0; r0 < n_rows;) {
            int64_t r1 = r0 + 1;
            while (r1 < n_rows && rp[size_t(r1) + 1] - rp[size_t(r0)] <= block_nnz) ++r1;
            if (rp[size_t(r1)] - rp[size_t(r0)] > kBlockMaxNnz) {
                free_handle(m);
                return VSPMM_ERR_UNSUPPORTED;
            }
            m->block_row0.push_back(r0);
            for (int64_t r = r0; r <= r1; ++r)
                ptr32.push_back(int32_t(rp[size_t(r)] - rp[size_t(r0)]));
            r0 = r1;
        }
        m->block_row0.push_back(n_rows);
    } catch (...) {
        free_handle(m);
        return VSPMM_ERR_ALLOC;
    }
    if (!ptr32.empty()) {
        if (hipMalloc(&m->block_ptr, ptr32.size() * sizeof(int32_t)) != hipSuccess) {
            m->block_ptr = nullptr;
            free_handle(m);
            return VSPMM_ERR_HIP;
        }
        if (hipMemcpyAsync(m->block_ptr, ptr32.data(), ptr32.size() * sizeof(int32_t),
                           hipMemcpyHostToDevice, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess) {
            free_handle(m);
            return VSPMM_ERR_HIP;
        }
    }
    const size_t ve = m->val_elt();
    size_t off = 0;
    for (size_t b = 0; b + 1 < m->block_row0.size(); ++b) {
        const int64_t r0 = m->block_row0[b], r1 = m->block_row0[b + 1];
        const int64_t e0 = rp[size_t(r0)], nb = rp[size_t(r1)] - e0;
        vspmm_matrix sub = nullptr;
        const vspmm_status st = vspmm_create_csr(
            &sub, r1 - r0, n_cols, nb, m->block_ptr + off, nb > 0 ? col + e0 : nullptr,
            nb > 0 ? static_cast<const char *>(val) + size_t(e0) * ve : nullptr, dtype, flags,
            force_group, stream);
        if (st) {
            free_handle(m);
            return st;
        }
        m->blocks.push_back(sub);
        off += size_t(r1 - r0) + 1;
    }
    *h = m;
    return VSPMM_OK;
}

vspmm_status vspmm_destroy(vspmm_matrix h) {
    if (!h) return VSPMM_ERR_NULL;
    free_handle(h);
    return VSPMM_OK;
}

vspmm_status vspmm_spmm(vspmm_matrix h, const void *B, void *out, int64_t width,
                        vspmm_direction dir, hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (vspmm_status st = check_product(*h, B, out, width, dir)) return st;
    return with_view(*h, B, out, width, dir, stream, [&](const void *Bv) {
        return run_product(*h, Bv, out, width, dir, VSPMM_ATOMIC, nullptr, 0, stream);
    });
}

vspmm_status vspmm_workspace_size(vspmm_matrix h, vspmm_direction dir, vspmm_mode mode,
                                  size_t *bytes) {
    if (vspmm_status st = check_handle(h)) return st;
    if (!bytes) return VSPMM_ERR_NULL;
    if (dir != VSPMM_AB && dir != VSPMM_BA) return VSPMM_ERR_ENUM;
    if (mode != VSPMM_ATOMIC && mode != VSPMM_DETERMINISTIC) return VSPMM_ERR_ENUM;
    if (h->ptr64) {
        *bytes = mode == VSPMM_DETERMINISTIC && dir == VSPMM_BA ? carve_blocked(*h, nullptr, 0).bytes
                                                                : 0;
        return VSPMM_OK;
    }
    *bytes = (mode == VSPMM_DETERMINISTIC && !is_aligned(*h, dir))
                 ? carve_opposite(*h, nullptr).bytes
                 : 0;
    return VSPMM_OK;
}

vspmm_status vspmm_spmm_ex(vspmm_matrix h, const void *B, void *out, int64_t width,
                           vspmm_direction dir, vspmm_mode mode, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (vspmm_status st = check_product(*h, B, out, width, dir)) return st;
    if (mode != VSPMM_ATOMIC && mode != VSPMM_DETERMINISTIC) return VSPMM_ERR_ENUM;
    return with_view(*h, B, out, width, dir, stream, [&](const void *Bv) {
        return run_product(*h, Bv, out, width, dir, mode, ws, ws_bytes, stream);
    });
}

vspmm_status vspmm_schedule_create(vspmm_schedule *sc, vspmm_matrix h, vspmm_direction dir,
                                   int64_t width, void *build_ws, size_t build_ws_bytes,
                                   hipStream_t stream) {
    if (!sc) return VSPMM_ERR_NULL;
    *sc = nullptr;
    if (vspmm_status st = check_handle(h)) return st;
    if (dir != VSPMM_AB && dir != VSPMM_BA) return VSPMM_ERR_ENUM;
    if (width < 0 || !fits_i32(width)) return VSPMM_ERR_DIM;
    auto *s = new (std::nothrow) vspmm_schedule_s{};
    if (!s) return VSPMM_ERR_ALLOC;
    s->h = h;
    s->dir = dir;
    s->width = width;
    vspmm_status st;
    try {
        st = schedule_build(s, build_ws, build_ws_bytes, stream);
    } catch (...) {
        st = VSPMM_ERR_ALLOC;
    }
    if (st) {
        schedule_free(s);
        return st;
    }
    *sc = s;
    return VSPMM_OK;
}

vspmm_status vspmm_schedule_spmm(vspmm_schedule sc, const void *B, void *out, int64_t width,
                                 hipStream_t stream) {
    if (!sc) return VSPMM_ERR_NULL;
    if (vspmm_status st = check_product(*sc->h, B, out, width, sc->dir)) return st;
    if (width != sc->width) return VSPMM_ERR_DIM;
    if (width == 0 || n_out(*sc->h, sc->dir) == 0) return VSPMM_OK;
    return with_view(*sc->h, B, out, width, sc->dir, stream,
                     [&](const void *Bv) { return schedule_product(*sc, Bv, out, stream); });
}

vspmm_status vspmm_schedule_bytes(vspmm_schedule sc, size_t *bytes) {
    if (!sc || !bytes) return VSPMM_ERR_NULL;
    size_t n = sc->bytes;
    for (const vspmm_schedule_s *sub : sc->subs)
        if (sub) n += sub->bytes;
    *bytes = n;
    return VSPMM_OK;
}

vspmm_status vspmm_schedule_destroy(vspmm_schedule sc) {
    if (!sc) return VSPMM_ERR_NULL;
    schedule_free(sc);
    return VSPMM_OK;
}

vspmm_status vspmm_spmm_noalloc(vspmm_matrix h, const void *B, void *out, int64_t width,
                                vspmm_direction dir, vspmm_mode mode, hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (mode != VSPMM_ATOMIC && mode != VSPMM_DETERMINISTIC) return VSPMM_ERR_ENUM;
    if (dir != VSPMM_AB && dir != VSPMM_BA) return VSPMM_ERR_ENUM;
    if (width < 0 || !fits_i32(width)) return VSPMM_ERR_DIM;
    size_t need = 0;
    if (vspmm_status st = vspmm_workspace_size_width(h, dir, mode, width, &need)) return st;
    // a product that needs a workspace larger than the array, even without
    // the tiled copy, is refused before anything is enqueued
    size_t base_need = 0;
    if (vspmm_status st = vspmm_workspace_size(h, dir, mode, &base_need)) return st;
    if (h->ptr64 && mode == VSPMM_DETERMINISTIC && dir == VSPMM_BA) base_need = need;
    if (base_need > kStaticScratchBytes) return VSPMM_ERR_WORKSPACE;
    void *ws = nullptr;
    if (vspmm_status st = static_scratch(h->device, &ws)) return st;
    if (vspmm_status st = check_product(*h, B, out, width, dir)) return st;
    return with_view(*h, B, out, width, dir, stream, [&](const void *Bv) {
        return run_product(*h, Bv, out, width, dir, mode, ws, kStaticScratchBytes, stream);
    });
}

const char *vspmm_view_name(int32_t view) {
    switch (view) {
        case VSPMM_VIEW_IDENTITY: return "identity";
        case VSPMM_VIEW_SCALE: return "scale";
    }
    return nullptr;
}

vspmm_status vspmm_set_view(vspmm_matrix h, int32_t view, const void *row_stat,
                            const void *col_stat, int64_t max_width) {
    if (vspmm_status st = check_handle(h)) return st;
    if (!vspmm_view_name(view)) return VSPMM_ERR_ENUM;
    if (view == VSPMM_VIEW_SCALE) {
        if ((h->n_rows > 0 && !row_stat) || (h->n_cols > 0 && !col_stat)) return VSPMM_ERR_NULL;
        if (max_width < 1 || !fits_i32(max_width)) return VSPMM_ERR_DIM;
        if (!aligned(row_stat, h->elt()) || !aligned(col_stat, h->elt())) return VSPMM_ERR_DIM;
    }
    void *buf = nullptr;
    if (view == VSPMM_VIEW_SCALE) {
        const size_t rows = size_t(std::max(h->n_rows, h->n_cols));
        const size_t bytes = std::max<size_t>(rows * size_t(max_width) * h->elt(), 256);
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return VSPMM_ERR_HIP;
        if (cur != h->device && hipSetDevice(h->device) != hipSuccess) return VSPMM_ERR_HIP;
        const hipError_t e = hipMalloc(&buf, bytes);
        if (cur != h->device) (void)hipSetDevice(cur);
        if (e != hipSuccess) return VSPMM_ERR_HIP;
    }
    if (h->view_buf) (void)hipFree(h->view_buf);
    h->view = view;
    h->row_stat = view == VSPMM_VIEW_SCALE ? row_stat : nullptr;
    h->col_stat = view == VSPMM_VIEW_SCALE ? col_stat : nullptr;
    h->view_buf = buf;
    h->view_width = view == VSPMM_VIEW_SCALE ? max_width : 0;
    return VSPMM_OK;
}

vspmm_status vspmm_workspace_size_width(vspmm_matrix h, vspmm_direction dir, vspmm_mode mode,
                                        int64_t width, size_t *bytes) {
    if (vspmm_status st = vspmm_workspace_size(h, dir, mode, bytes)) return st;
    if (width < 0 || !fits_i32(width)) return VSPMM_ERR_DIM;
    if (mode != VSPMM_DETERMINISTIC) return VSPMM_OK;
    if (h->ptr64) {
        if (dir == VSPMM_BA) *bytes = carve_blocked(*h, nullptr, width).bytes;
        return VSPMM_OK;
    }
    const DeviceInfo di = device_info(h->device);
    const bool split_matrix = (h->flags & VSPMM_SPLIT_MATRIX) != 0;
    alignas(256) static const float probe[64] = {};
    const TilePlan tp = tile_plan(*h, dir, width, di.ok ? di.n_cu : 256, split_matrix, probe, probe);
    if (tp.ok) *bytes = tiled_ws_bytes(*h, tp, width);
    return VSPMM_OK;
}

vspmm_status vspmm_validate(vspmm_matrix h, hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (h->ptr64) {
        // the int64 row pointers were checked at creation; each block checks
        // its indices (and its rebased pointers)
        for (vspmm_matrix_s *b : h->blocks)
            if (vspmm_status st = vspmm_validate(b, stream)) return st;
        return VSPMM_OK;
    }
    const DeviceInfo di = device_info(h->device);
    const int n_cu = di.ok ? di.n_cu : 256;
    int *flag = nullptr;
    if (hipMalloc(&flag, sizeof(int)) != hipSuccess) return VSPMM_ERR_HIP;
    launch_zero(flag, 4, stream);
    const int64_t nmaj = h->n_major();
    hipLaunchKernelGGL(k_validate_ptr, dim3(grid_for(nmaj + 1, n_cu)), dim3(256), 0, stream,
                       h->sptr, int(nmaj), int(h->layout == VSPMM_CSR ? h->nnz : h->n_groups),
                       flag);
    if (h->layout != VSPMM_CSR)
        hipLaunchKernelGGL(k_validate_ptr, dim3(grid_for(h->n_groups + 1, n_cu)), dim3(256), 0,
                           stream, h->vptr, int(h->n_groups), int(h->nnz), flag);
    if (h->nnz > 0)
        hipLaunchKernelGGL(k_validate_idx, dim3(grid_for(h->nnz, n_cu)), dim3(256), 0, stream,
                           h->idx, int(h->nnz), int(h->n_minor()), flag);
    int host_flag = -1;
    vspmm_status st = hip_status();
    if (!st && hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, stream) !=
                   hipSuccess)
        st = VSPMM_ERR_HIP;
    if (!st && hipStreamSynchronize(stream) != hipSuccess) st = VSPMM_ERR_HIP;
    (void)hipFree(flag);
    if (st) return st;
    return host_flag == 0 ? VSPMM_OK : VSPMM_ERR_STRUCTURE;
}

vspmm_status vspmm_transpose_csr(vspmm_matrix h, int32_t *t_row_ptr, int32_t *t_col,
                                 void *t_val, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (h->layout != VSPMM_CSR) return VSPMM_ERR_ENUM;
    if (h->ptr64) return VSPMM_ERR_UNSUPPORTED;
    if (!t_row_ptr || (h->nnz > 0 && (!t_col || !t_val))) return VSPMM_ERR_NULL;
    const OppositeWs need = carve_opposite(*h, nullptr);
    if (!ws || ws_bytes < need.bytes || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
    const DeviceInfo di = device_info(h->device);
    build_transpose(*h, carve_opposite(*h, ws), t_row_ptr, t_col, t_val, di.ok ? di.n_cu : 256,
                    stream);
    return hip_status();
}

vspmm_status vspmm_transpose_csr_scaled(vspmm_matrix h, const void *factor, int32_t *t_row_ptr,
                                        int32_t *t_col, void *t_val, void *ws, size_t ws_bytes,
                                        hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (h->layout != VSPMM_CSR) return VSPMM_ERR_ENUM;
    if (h->ptr64) return VSPMM_ERR_UNSUPPORTED;
    if (!t_row_ptr || (h->nnz > 0 && (!t_col || !t_val || !factor))) return VSPMM_ERR_NULL;
    if (h->nnz > 0 && !aligned(factor, h->val_elt())) return VSPMM_ERR_DIM;
    const OppositeWs need = carve_opposite(*h, nullptr);
    if (!ws || ws_bytes < need.bytes || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
    const DeviceInfo di = device_info(h->device);
    build_transpose(*h, carve_opposite(*h, ws), t_row_ptr, t_col, t_val, di.ok ? di.n_cu : 256,
                    stream, factor);
    return hip_status();
}

vspmm_status vspmm_assemble_workspace_size(int32_t role, int64_t n_elem, int64_t n_out,
                                           int64_t n_in, int64_t nnz, size_t *bytes) {
    if (!bytes) return VSPMM_ERR_NULL;
    if (role < VSPMM_ROLE_OWN || role > VSPMM_ROLE_SUM_OF) return VSPMM_ERR_ENUM;
    if (n_elem < 0 || n_out < 0 || n_in < 0 || !fits_i32(nnz)) return VSPMM_ERR_DIM;
    int64_t rows, cols;
    role_dims(role, n_elem, n_out, n_in, &rows, &cols);
    if (!fits_i32(rows + 1) || !fits_i32(cols)) return VSPMM_ERR_DIM;
    *bytes = carve_assemble(nnz, rows, nullptr).bytes;
    return VSPMM_OK;
}

vspmm_status vspmm_assemble_csr(int32_t role, int64_t n_elem, int64_t n_out, int64_t n_in,
                                int64_t nnz, const int32_t *elem_ptr, const int32_t *out_idx,
                                const int32_t *in_idx, const void *weight, vspmm_dtype dtype,
                                int32_t *row_ptr, int32_t *col, void *val, void *ws,
                                size_t ws_bytes, hipStream_t stream) {
    size_t need = 0;
    if (vspmm_status st = vspmm_assemble_workspace_size(role, n_elem, n_out, n_in, nnz, &need))
        return st;
    if (dtype != VSPMM_F32 && dtype != VSPMM_F64) return VSPMM_ERR_ENUM;
    if (!fits_i32(n_elem) || !fits_i32(n_out) || !fits_i32(n_in)) return VSPMM_ERR_DIM;
    if (!elem_ptr || !row_ptr) return VSPMM_ERR_NULL;
    if (nnz > 0 && (!out_idx || !in_idx || !weight || !col || !val)) return VSPMM_ERR_NULL;
    if (!ws || ws_bytes < need || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
    int64_t rows, cols;
    role_dims(role, n_elem, n_out, n_in, &rows, &cols);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return VSPMM_ERR_HIP;
    const DeviceInfo di = device_info(dev);
    const int n_cu = di.ok ? di.n_cu : 256;
    const AssembleWs w = carve_assemble(nnz, rows, ws);
    if (nnz == 0) {
        bin_starts(nullptr, 0, rows, row_ptr, n_cu, stream);
        return hip_status();
    }
    // the counting sort by operator row: stable, so a row keeps its entries
    // in element order and, within an element, in the order given
    const int ge = int(std::max<int64_t>(1, std::min<int64_t>((n_elem + 3) / 4, n_cu * 16)));
    if (n_elem > 0)
        hipLaunchKernelGGL(k_elem_of, dim3(ge), dim3(256), 0, stream, int(n_elem), elem_ptr,
                           int(nnz), w.elem_of);
    const int grid = grid_for(nnz, n_cu);
    uint32_t *ka = w.keys_a, *kb = w.keys_b;
    int32_t *pa = w.pay_a, *pb = w.pay_b;
    hipLaunchKernelGGL(k_role_keys, dim3(grid), dim3(256), 0, stream, int(nnz), w.elem_of,
                       out_idx, int(role), int(n_out), ka, pa);
    radix_sort(&ka, &pa, &kb, &pb, nnz, key_bits(rows), w.hist, w.bsums, stream);
    bin_starts(ka, nnz, rows, row_ptr, n_cu, stream);
    if (dtype == VSPMM_F64)
        hipLaunchKernelGGL(k_role_emit<double>, dim3(grid), dim3(256), 0, stream, int(nnz), pa,
                           w.elem_of, in_idx, static_cast<const double *>(weight), int(role),
                           int(n_in), col, static_cast<double *>(val));
    else
        hipLaunchKernelGGL(k_role_emit<float>, dim3(grid), dim3(256), 0, stream, int(nnz), pa,
                           w.elem_of, in_idx, static_cast<const float *>(weight), int(role),
                           int(n_in), col, static_cast<float *>(val));
    return hip_status();
}


vspmm_status vspmm_regroup_vcs(vspmm_matrix h, int32_t *t_major_ptr, float *t_values,
                               int32_t *t_value_ptr, int32_t *t_indices, int32_t *t_n_groups,
                               void *ws, size_t ws_bytes, hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (h->layout == VSPMM_CSR) return VSPMM_ERR_ENUM;
    if (!t_major_ptr || !t_value_ptr || !t_n_groups) return VSPMM_ERR_NULL;
    if (h->nnz > 0 && (!t_values || !t_indices)) return VSPMM_ERR_NULL;
    const OppositeWs need = carve_opposite(*h, nullptr);
    if (!ws || ws_bytes < need.bytes || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
    const DeviceInfo di = device_info(h->device);
    build_regroup(*h, carve_opposite(*h, ws), t_major_ptr, t_values, t_value_ptr, t_indices,
                  t_n_groups, di.ok ? di.n_cu : 256, stream);
    return hip_status();
}

vspmm_status vspmm_expand_vcs(vspmm_matrix h, vspmm_format format, int32_t sort_indices,
                              int32_t *ptr, int32_t *idx, float *val, void *ws, size_t ws_bytes,
                              hipStream_t stream) {
    if (vspmm_status st = check_handle(h)) return st;
    if (h->layout == VSPMM_CSR) return VSPMM_ERR_ENUM;
    if (format != VSPMM_FORMAT_CSR && format != VSPMM_FORMAT_CSC) return VSPMM_ERR_ENUM;
    const bool own = (format == VSPMM_FORMAT_CSR) == (h->layout == VSPMM_VCSR);
    if (!ptr) return VSPMM_ERR_NULL;
    if (h->nnz > 0 && (!idx || !val)) return VSPMM_ERR_NULL;
    const bool needs_ws = !own || sort_indices;
    if (needs_ws) {
        const OppositeWs need = carve_opposite(*h, nullptr);
        if (!ws || ws_bytes < need.bytes || !aligned(ws, 256)) return VSPMM_ERR_WORKSPACE;
    }
    const DeviceInfo di = device_info(h->device);
    build_expand(*h, own, sort_indices != 0, needs_ws ? carve_opposite(*h, ws) : OppositeWs{}, ptr,
                 idx, val, di.ok ? di.n_cu : 256, stream);
    return hip_status();
}

vspmm_status vspmm_footprint(vspmm_matrix h, size_t *bytes, size_t *expanded_bytes) {
    if (vspmm_status st = check_handle(h)) return st;
    const size_t nmaj = size_t(h->n_major()), nnz = size_t(h->nnz), e = h->val_elt();
    const size_t pe = h->ptr64 ? 8 : 4;  // bytes of a row pointer
    size_t own;
    if (h->layout == VSPMM_CSR)
        own = pe * (nmaj + 1) + (4 + e) * nnz;
    else
        own = 4 * (nmaj + 1) + 4 * size_t(h->n_groups) + 4 * (size_t(h->n_groups) + 1) + 4 * nnz;
    if (bytes) *bytes = own;
    if (expanded_bytes) *expanded_bytes = pe * (nmaj + 1) + (4 + e) * nnz;
    return VSPMM_OK;
}

vspmm_status vspmm_plan_info(vspmm_matrix h, int64_t width, vspmm_direction dir,
                             vspmm_mode mode, int32_t *entry_lanes, int32_t *width_lanes,
                             int32_t *vec, int32_t *slices_per_wave, int32_t *lds_staged,
                             int32_t *kernel, int32_t *tiles) {
    if (vspmm_status st = check_handle(h)) return st;
    if (dir != VSPMM_AB && dir != VSPMM_BA) return VSPMM_ERR_ENUM;
    if (mode != VSPMM_ATOMIC && mode != VSPMM_DETERMINISTIC) return VSPMM_ERR_ENUM;
    if (width < 0 || !fits_i32(width)) return VSPMM_ERR_DIM;
    if (h->ptr64) {
        if (h->blocks.empty()) return VSPMM_ERR_UNSUPPORTED;
        if (tiles) *tiles = 0;
        return vspmm_plan_info(h->blocks[0], width, dir, mode, entry_lanes, width_lanes, vec,
                               slices_per_wave, lds_staged, kernel, nullptr);
    }
    const bool vcs = h->layout != VSPMM_CSR;
    const bool split_matrix = (h->flags & VSPMM_SPLIT_MATRIX) ||
                              (!vcs && !(h->flags & VSPMM_SPLIT_WIDTH));
    const bool al = is_aligned(*h, dir);
    const bool scatter = !al && mode == VSPMM_ATOMIC;
    const int64_t ns = al || scatter ? h->n_major() : h->n_minor();
    const int64_t ni = al || scatter ? h->n_minor() : h->n_major();
    // alignment of the caller's buffers is unknown here: assume 16-byte aligned
    alignas(256) static const float probe[64] = {};
    const DeviceInfo di = device_info(h->device);
    const int n_cu = di.ok ? di.n_cu : 256;
    const TilePlan tp = mode == VSPMM_DETERMINISTIC
                            ? tile_plan(*h, dir, width, n_cu, split_matrix, probe, probe)
                            : TilePlan{};
    const Plan pl = tp.ok ? tp.pl
                    : scatter ? scatter_plan(h->nnz, width, n_out(*h, dir), h->elt(), n_cu,
                                             h->force_group)
                              : make_plan(ns, h->nnz, width, h->elt(), split_matrix,
                                          h->force_group, probe, probe, n_cu, ni, vcs);
    if (tiles) *tiles = tp.ok ? tp.tiles : 0;
    if (entry_lanes) *entry_lanes = 1 << pl.sp.log_g;
    if (width_lanes) *width_lanes = 1 << pl.sp.log_ww;
    if (vec) *vec = pl.vec;
    if (slices_per_wave) *slices_per_wave = pl.R;
    if (lds_staged) *lds_staged = pl.lds ? 1 : 0;
    // the short VCS walk runs as k_vcs_seg at up to 4 width lanes per entry
    // (every VCS walk carries its per-wave plan)
    const bool seg = vcs && !scatter && pl.kind == kShort && pl.sp.log_ww <= 2;
    if (kernel)
        *kernel = scatter ? VSPMM_KERNEL_SCATTER
                  : seg   ? VSPMM_KERNEL_SEG
                  : pl.kind == kLong ? VSPMM_KERNEL_LONG
                  : pl.kind == kShort ? VSPMM_KERNEL_SHORT
                                      : VSPMM_KERNEL_PLAIN;
    return VSPMM_OK;
}

}  // extern "C"
