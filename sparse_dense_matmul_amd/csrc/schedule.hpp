// Building a matrix in the opposite layout on the device: the exact CSR
// transpose and the VCSR <-> VCSC regrouping. Both are a stable sort of the
// entries by their new slice (regridding page, section "How it is built":
// count per row, then place at the rows' cursors keeping each row's entries in
// source order). On the GPU the placement is an LSD radix sort whose scatter
// ranks equal digits in input order, so every result is unique and equals a
// sequential counting sort bit for bit, whatever the timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace vspmm {

constexpr int kSortThreads = 256;
constexpr int kSortRounds = 16;
constexpr int kSortTile = kSortThreads * kSortRounds;  // elements per block
constexpr int kScanTile = 4096;                         // elements per block

// ------------------------------------------------------------------- scan

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

// Exclusive scan of 256 per-thread values across a block; returns the prefix.
__device__ __forceinline__ int block_exclusive_scan(int x, int *sh_waves /*[4]*/, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_inclusive_scan(x, lane);
    if (lane == 63) sh_waves[wave] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int s = sh_waves[k];
        if (k < wave) before += s;
        total += s;
    }
    __syncthreads();
    return before + inc - x;
}

// Sum of each tile of kScanTile elements.
__global__ void __launch_bounds__(256) k_scan_reduce(const int *__restrict__ in, int n,
                                                     int *__restrict__ bsums) {
    __shared__ int sh[4];
    const int base = blockIdx.x * kScanTile;
    int s = 0;
    for (int r = 0; r < kScanTile / 256; ++r) {
        const int i = base + r * 256 + threadIdx.x;
        if (i < n) s += in[i];
    }
    int total;
    block_exclusive_scan(s, sh, total);
    if (threadIdx.x == 0) bsums[blockIdx.x] = total;
}

// Exclusive scan of the tile sums in place (one block); *total = their sum.
__global__ void __launch_bounds__(256) k_scan_bsums(int *__restrict__ bsums, int nb,
                                                    int *__restrict__ total) {
    __shared__ int sh[4];
    int carry = 0;
    for (int base = 0; base < nb; base += 256) {
        const int i = base + threadIdx.x;
        const int x = i < nb ? bsums[i] : 0;
        int t;
        const int ex = block_exclusive_scan(x, sh, t);
        if (i < nb) bsums[i] = carry + ex;
        carry += t;
    }
    if (threadIdx.x == 0 && total) *total = carry;
}

// Exclusive scan of each tile plus its offset; out may alias in.
__global__ void __launch_bounds__(256) k_scan_apply(const int *in, int n,
                                                    const int *__restrict__ bsums, int *out) {
    __shared__ int tile[kScanTile];
    __shared__ int sh[4];
    const int base = blockIdx.x * kScanTile;
    for (int r = 0; r < kScanTile / 256; ++r) {
        const int i = base + r * 256 + threadIdx.x;
        tile[r * 256 + threadIdx.x] = i < n ? in[i] : 0;
    }
    __syncthreads();
    constexpr int per = kScanTile / 256;
    int s = 0;
    for (int k = 0; k < per; ++k) s += tile[threadIdx.x * per + k];
    int total;
    int run = block_exclusive_scan(s, sh, total) + bsums[blockIdx.x];
    for (int k = 0; k < per; ++k) {
        const int x = tile[threadIdx.x * per + k];
        tile[threadIdx.x * per + k] = run;
        run += x;
    }
    __syncthreads();
    for (int r = 0; r < kScanTile / 256; ++r) {
        const int i = base + r * 256 + threadIdx.x;
        if (i < n) out[i] = tile[r * 256 + threadIdx.x];
    }
}

// ------------------------------------------------------------- radix sort

// Digit histogram of each tile: hist[d * nblocks + b].
__global__ void __launch_bounds__(kSortThreads)
k_radix_hist(const uint32_t *__restrict__ keys, int n, int shift, int nblocks,
             int *__restrict__ hist) {
    __shared__ int h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int base = blockIdx.x * kSortTile;
    for (int r = 0; r < kSortRounds; ++r) {
        const int i = base + r * kSortThreads + threadIdx.x;
        if (i < n) atomicAdd(&h[(keys[i] >> shift) & 255u], 1);
    }
    __syncthreads();
    hist[threadIdx.x * nblocks + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter: each element goes to offs[d * nblocks + b] plus the number of
// earlier elements of its tile with the same digit.
__global__ void __launch_bounds__(kSortThreads)
k_radix_scatter(const uint32_t *__restrict__ keys, const int *__restrict__ pay, int n, int shift,
                int nblocks, const int *__restrict__ offs, uint32_t *__restrict__ okeys,
                int *__restrict__ opay) {
    __shared__ int run[256];
    __shared__ int wc[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    run[threadIdx.x] = offs[threadIdx.x * nblocks + blockIdx.x];
#pragma unroll
    for (int k = 0; k < 4; ++k) wc[k][threadIdx.x] = 0;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int base = blockIdx.x * kSortTile;
    for (int r = 0; r < kSortRounds; ++r) {
        const int i = base + r * kSortThreads + threadIdx.x;
        const bool valid = i < n;
        const uint32_t k = valid ? keys[i] : 0u;
        const int d = (int)((k >> shift) & 255u);
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const int wrank = __popcll(m & lt);
        if (valid && wrank == 0) wc[wave][d] = __popcll(m);
        __syncthreads();
        if (valid) {
            int pos = run[d] + wrank;
            for (int w2 = 0; w2 < wave; ++w2) pos += wc[w2][d];
            okeys[pos] = k;
            opay[pos] = pay[i];
        }
        __syncthreads();
        run[threadIdx.x] += wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] +
                            wc[3][threadIdx.x];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) wc[k2][threadIdx.x] = 0;
        __syncthreads();
    }
}

// ------------------------------------------------------ entry bookkeeping

// For every entry p: the slice holding it (slice_of) and, for a VCS, its group
// (group_of). One wave per slice; each lane walks its entries with its own
// group cursor.
template <bool VCS>
__global__ void __launch_bounds__(256)
k_expand(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
         int *__restrict__ slice_of, int *__restrict__ group_of) {
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    for (int s = blockIdx.x * waves + (threadIdx.x >> 6); s < n_slices; s += gridDim.x * waves) {
        int e0, e1, kc = 0, kend = 0;
        if constexpr (VCS) {
            const int ka = sptr[s], kb = sptr[s + 1];
            e0 = vptr[ka];
            e1 = vptr[kb];
            kc = ka;
            kend = kb > ka ? vptr[ka + 1] : 0;
        } else {
            e0 = sptr[s];
            e1 = sptr[s + 1];
        }
        for (int p = e0 + lane; p < e1; p += 64) {
            slice_of[p] = s;
            if constexpr (VCS) {
                while (p >= kend) {
                    ++kc;
                    kend = vptr[kc + 1];
                }
                group_of[p] = kc;
            }
        }
    }
}

// ------------------------------------------------------------- expansion

// Pointers of a VCS expanded to one value per entry: ptr[s] = value_ptr of
// slice s's first group (s = 0 .. n_slices).
__global__ void __launch_bounds__(256)
k_expand_ptr(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
             int *__restrict__ ptr) {
    const int stride = gridDim.x * blockDim.x;
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s <= n_slices; s += stride)
        ptr[s] = vptr[sptr[s]];
}

// A VCS expanded in stored order: idx_out[p] = idx[p], val_out[p] = the
// value of p's group. One wave per slice, each lane with its own group cursor.
__global__ void __launch_bounds__(256)
k_expand_copy(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
              const float *__restrict__ values, const int *__restrict__ idx,
              int *__restrict__ idx_out, float *__restrict__ val_out) {
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    for (int s = blockIdx.x * waves + (threadIdx.x >> 6); s < n_slices; s += gridDim.x * waves) {
        const int ka = sptr[s], kb = sptr[s + 1];
        if (kb <= ka) continue;
        const int e0 = vptr[ka], e1 = vptr[kb];
        int kc = ka, kend = vptr[ka + 1];
        for (int p = e0 + lane; p < e1; p += 64) {
            while (p >= kend) {
                ++kc;
                kend = vptr[kc + 1];
            }
            idx_out[p] = idx[p];
            val_out[p] = values[kc];
        }
    }
}

// Entries in sorted order (pay[q] = the stored position of the q-th):
// idx_out[q] = src[pay[q]] (the entry's index, or its slice for the other
// format), val_out[q] = the value of its group.
__global__ void __launch_bounds__(256)
k_expand_emit(int nnz, const int *__restrict__ pay, const int *__restrict__ src,
              const int *__restrict__ group_of, const float *__restrict__ values,
              int *__restrict__ idx_out, float *__restrict__ val_out) {
    const int stride = gridDim.x * blockDim.x;
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < nnz; q += stride) {
        const int p = pay[q];
        idx_out[q] = src[p];
        val_out[q] = values[group_of[p]];
    }
}

// A VCS expanded with each slice's entries sorted by index (stable), one
// block of BLOCK threads per slice (grid-stride). A slice of at most CAP
// entries is sorted in LDS: keys (index << 32 | position in the slice) are
// unique, so a bitonic sort gives the stable order; each entry's value comes
// from its group through a per-thread cursor. A longer slice is sorted by the
// block alone with a stable LSD radix sort on the index (8 bits per pass,
// `bits` bits) through the workspace arrays ka/pa and kb/pb over the slice's
// own range, its values staged in vb; then emitted.
template <int BLOCK, int CAP>
__global__ void __launch_bounds__(BLOCK)
k_expand_sorted(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
                const float *__restrict__ values, const int *__restrict__ idx, int bits,
                uint32_t *__restrict__ ka, int *__restrict__ pa, uint32_t *__restrict__ kb,
                int *__restrict__ pb, float *__restrict__ vb, int *__restrict__ idx_out,
                float *__restrict__ val_out) {
    constexpr int WAVES = BLOCK / 64;
    __shared__ unsigned long long key[CAP];
    __shared__ float val[CAP];
    __shared__ int run[256];
    __shared__ int wc[WAVES][256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int s = blockIdx.x; s < n_slices; s += gridDim.x) {
        const int ka0 = sptr[s], kb0 = sptr[s + 1];
        const int e0 = kb0 > ka0 ? vptr[ka0] : 0, e1 = kb0 > ka0 ? vptr[kb0] : 0;
        const int n = e1 - e0;
        if (n <= 0) continue;  // uniform in the block
        if (n <= CAP) {
            int N = 1;
            while (N < n) N <<= 1;
            int kc = ka0, kend = vptr[ka0 + 1];
            for (int i = tid; i < N; i += BLOCK) {
                if (i < n) {
                    while (e0 + i >= kend) {
                        ++kc;
                        kend = vptr[kc + 1];
                    }
                    key[i] = ((unsigned long long)(uint32_t)idx[e0 + i] << 32) | (uint32_t)i;
                    val[i] = values[kc];
                } else {
                    key[i] = ~0ull;
                }
            }
            __syncthreads();
            for (int k = 2; k <= N; k <<= 1) {
                for (int j = k >> 1; j > 0; j >>= 1) {
                    for (int i = tid; i < N; i += BLOCK) {
                        const int ixj = i ^ j;
                        if (ixj > i) {
                            const unsigned long long a = key[i], b = key[ixj];
                            if ((a > b) == ((i & k) == 0)) {
                                key[i] = b;
                                key[ixj] = a;
                            }
                        }
                    }
                    __syncthreads();
                }
            }
            for (int r = tid; r < n; r += BLOCK) {
                const unsigned long long kk = key[r];
                idx_out[e0 + r] = (int)(kk >> 32);
                val_out[e0 + r] = val[(int)(kk & 0xffffffffu)];
            }
            __syncthreads();
            continue;
        }
        // long slice: stage keys, positions and values, then radix passes
        {
            int kc = ka0, kend = vptr[ka0 + 1];
            for (int i = tid; i < n; i += BLOCK) {
                while (e0 + i >= kend) {
                    ++kc;
                    kend = vptr[kc + 1];
                }
                ka[e0 + i] = (uint32_t)idx[e0 + i];
                pa[e0 + i] = i;
                vb[e0 + i] = values[kc];
            }
        }
        __syncthreads();
        uint32_t *ks = ka, *kd = kb;
        int *ps = pa, *pd = pb;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int shift = 0; shift < bits; shift += 8) {
            for (int d = tid; d < 256; d += BLOCK) run[d] = 0;
            __syncthreads();
            for (int i = tid; i < n; i += BLOCK) atomicAdd(&run[(ks[e0 + i] >> shift) & 255u], 1);
            __syncthreads();
            {  // exclusive scan of the 256 digit counts: BPT per thread, then
               // the threads' sums scanned across lanes and waves
                constexpr int BPT = 256 / BLOCK;
                int c[BPT], sum = 0;
#pragma unroll
                for (int q = 0; q < BPT; ++q) {
                    c[q] = run[tid * BPT + q];
                    sum += c[q];
                }
                int incl = sum;  // inclusive scan of sum over the wave's lanes
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
                if (lane == 63) wc[0][wave] = incl;  // wave totals (wc is free here)
                __syncthreads();
                int before = incl - sum;
                for (int w2 = 0; w2 < wave; ++w2) before += wc[0][w2];
#pragma unroll
                for (int q = 0; q < BPT; ++q) {
                    run[tid * BPT + q] = before;
                    before += c[q];
                }
            }
            __syncthreads();
            for (int d = tid; d < 256 * WAVES; d += BLOCK) wc[d / 256][d % 256] = 0;
            __syncthreads();
            for (int base = 0; base < n; base += BLOCK) {  // tiles in order: stable
                const int i = base + tid;
                const bool valid = i < n;
                const uint32_t kk = valid ? ks[e0 + i] : 0u;
                const int d = (int)((kk >> shift) & 255u);
                uint64_t m = __ballot(valid);
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const bool bit = (d >> b) & 1;
                    const uint64_t bb = __ballot(bit);
                    m &= bit ? bb : ~bb;
                }
                const int wrank = __popcll(m & lt);
                if (valid && wrank == 0) wc[wave][d] = __popcll(m);
                __syncthreads();
                if (valid) {
                    int pos = run[d] + wrank;
                    for (int w2 = 0; w2 < wave; ++w2) pos += wc[w2][d];
                    kd[e0 + pos] = kk;
                    pd[e0 + pos] = ps[e0 + i];
                }
                __syncthreads();
                for (int dd = tid; dd < 256; dd += BLOCK) {
                    int t = 0;
                    for (int w2 = 0; w2 < WAVES; ++w2) {
                        t += wc[w2][dd];
                        wc[w2][dd] = 0;
                    }
                    run[dd] += t;
                }
                __syncthreads();
            }
            uint32_t *tk = ks;
            ks = kd;
            kd = tk;
            int *tp = ps;
            ps = pd;
            pd = tp;
        }
        for (int r = tid; r < n; r += BLOCK) {
            idx_out[e0 + r] = (int)ks[e0 + r];
            val_out[e0 + r] = vb[e0 + ps[e0 + r]];
        }
        __syncthreads();
    }
}

// Order key of a float32 bit pattern: ascending value, -0 before +0, NaNs
// beyond the infinities by payload. Equal keys iff equal bits.
__device__ __forceinline__ uint32_t value_order(uint32_t bits) {
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

__global__ void __launch_bounds__(256)
k_value_keys(int nnz, const int *__restrict__ group_of, const float *__restrict__ values,
             uint32_t *__restrict__ keys, int *__restrict__ pay) {
    const int stride = gridDim.x * blockDim.x;
    for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += stride) {
        keys[p] = value_order(__float_as_uint(values[group_of[p]]));
        pay[p] = p;
    }
}

__global__ void __launch_bounds__(256)
k_index_keys(int nnz, const int *__restrict__ idx, uint32_t *__restrict__ keys,
             int *__restrict__ pay) {
    const int stride = gridDim.x * blockDim.x;
    for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += stride) {
        keys[p] = (uint32_t)idx[p];
        pay[p] = p;
    }
}

// keys[e] = idx[pay[e]] (the new slice of the e-th entry in current order).
__global__ void __launch_bounds__(256)
k_gather_index(int nnz, const int *__restrict__ pay, const int *__restrict__ idx,
               uint32_t *__restrict__ keys) {
    const int stride = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += stride)
        keys[e] = (uint32_t)idx[pay[e]];
}

// ------------------------------------------------------------- transpose

// The transpose's e-th entry is the source's entry pay[e]; with factor, its
// value is scaled by that entry's own factor (one rounding, as a product).
template <typename T>
__global__ void __launch_bounds__(256)
k_transpose_emit(int nnz, const int *__restrict__ pay, const int *__restrict__ slice_of,
                 const T *__restrict__ val, const T *__restrict__ factor, int *__restrict__ t_idx,
                 T *__restrict__ t_val) {
    const int stride = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += stride) {
        const int p = pay[e];
        t_idx[e] = slice_of[p];
        t_val[e] = factor ? val[p] * factor[p] : val[p];
    }
}

// ------------------------------------------------------------- assembly

// The operator of a regridder's elements: element e's entries are
// [elem_ptr[e], elem_ptr[e + 1]); the orthogonal axis's role places entry
// (e, o, i) at row e * n_out + o (each element its own output: roles 0 and
// 1) or o (outputs summed: 2 and 3), column e * n_in + i (each element its
// own input: 0 and 2) or i (one shared input: 1 and 3).
__device__ __forceinline__ int role_row(int role, int e, int o, int n_out) {
    return role <= 1 ? e * n_out + o : o;
}
__device__ __forceinline__ int role_col(int role, int e, int i, int n_in) {
    return (role == 0 || role == 2) ? e * n_in + i : i;
}

// elem_of[p] = the element holding entry p (pointers clamped to [0, nnz], so
// a malformed list writes nothing out of range).
__global__ void __launch_bounds__(256)
k_elem_of(int n_elem, const int *__restrict__ elem_ptr, int nnz, int *__restrict__ elem_of) {
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    for (int e = blockIdx.x * waves + (threadIdx.x >> 6); e < n_elem; e += gridDim.x * waves) {
        const int p0 = min(max(elem_ptr[e], 0), nnz), p1 = min(max(elem_ptr[e + 1], 0), nnz);
        for (int p = p0 + lane; p < p1; p += 64) elem_of[p] = e;
    }
}

// Row keys of the entries (the counting sort's keys), payload = position.
__global__ void __launch_bounds__(256)
k_role_keys(int nnz, const int *__restrict__ elem_of, const int *__restrict__ out_idx, int role,
            int n_out, uint32_t *__restrict__ keys, int *__restrict__ pay) {
    const int stride = gridDim.x * blockDim.x;
    for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += stride) {
        keys[p] = (uint32_t)role_row(role, elem_of[p], out_idx[p], n_out);
        pay[p] = p;
    }
}

// The q-th entry of the operator is source entry pay[q]: its column and value.
template <typename T>
__global__ void __launch_bounds__(256)
k_role_emit(int nnz, const int *__restrict__ pay, const int *__restrict__ elem_of,
            const int *__restrict__ in_idx, const T *__restrict__ w, int role, int n_in,
            int *__restrict__ col, T *__restrict__ val) {
    const int stride = gridDim.x * blockDim.x;
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < nnz; q += stride) {
        const int p = pay[q];
        col[q] = role_col(role, elem_of[p], in_idx[p], n_in);
        val[q] = w[p];
    }
}

// ------------------------------------------------------------- regrouping

// flag[e] = 1 where a new group starts in the sorted order: a new slice, or a
// value whose bits differ from the previous entry's.
__global__ void __launch_bounds__(256)
k_group_flags(int nnz, const int *__restrict__ pay, const uint32_t *__restrict__ slice_key,
              const int *__restrict__ group_of, const float *__restrict__ values,
              int *__restrict__ flag) {
    const int stride = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += stride) {
        int f = 1;
        if (e > 0) {
            const uint32_t a = __float_as_uint(values[group_of[pay[e]]]);
            const uint32_t b = __float_as_uint(values[group_of[pay[e - 1]]]);
            f = (slice_key[e] != slice_key[e - 1]) || (a != b);
        }
        flag[e] = f;
    }
}

// Writes the regrouped entries; gid holds the exclusive scan of the flags.
__global__ void __launch_bounds__(256)
k_group_emit(int nnz, const int *__restrict__ pay, const int *__restrict__ slice_of,
             const int *__restrict__ group_of, const float *__restrict__ values,
             const int *__restrict__ flag, const int *__restrict__ gid,
             float *__restrict__ t_values, int *__restrict__ t_value_ptr,
             int *__restrict__ t_indices) {
    const int stride = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += stride) {
        const int p = pay[e];
        t_indices[e] = slice_of[p];
        if (flag[e]) {
            const int g = gid[e];
            t_values[g] = values[group_of[p]];
            t_value_ptr[g] = e;
        }
    }
}

// t_major_ptr[j] = first group of new slice j = gid at the slice's first
// entry (entry offsets tptr), or the group count at the end.
__global__ void __launch_bounds__(256)
k_group_major_ptr(int n_minor, int nnz, const int *__restrict__ tptr, const int *__restrict__ gid,
                  const int *__restrict__ n_groups, int *__restrict__ t_major_ptr,
                  int *__restrict__ t_value_ptr, int *__restrict__ t_n_groups) {
    const int stride = gridDim.x * blockDim.x;
    const int G = *n_groups;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j <= n_minor; j += stride) {
        const int t = j < n_minor ? tptr[j] : nnz;
        t_major_ptr[j] = t < nnz ? gid[t] : G;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        t_value_ptr[G] = nnz;
        if (t_n_groups) *t_n_groups = G;
    }
}

// ------------------------------------------------------------- long rows

// Rows longer than min_len: counted into *count, or, with list, appended to
// list at an atomic cursor (*count zeroed first; the order is arbitrary,
// which does not matter: each listed row is walked on its own).
__global__ void __launch_bounds__(256)
k_long_rows(int n_rows, const int *__restrict__ row_ptr, int min_len, int *__restrict__ count,
            int *__restrict__ list) {
    const int stride = gridDim.x * blockDim.x;
    for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < n_rows; r += stride) {
        if (row_ptr[r + 1] - row_ptr[r] > min_len) {
            const int c = atomicAdd(count, 1);
            if (list) list[c] = r;
        }
    }
}

// Entry-balanced row ranges: parts[p] is the first row whose entries start at
// or after p * nnz / n_parts (parts[n_parts] = n_rows), a binary search over
// row_ptr per part.
__global__ void __launch_bounds__(256)
k_row_parts(int n_rows, const int *__restrict__ row_ptr, long long nnz, int n_parts,
            int *__restrict__ parts) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p > n_parts) return;
    const long long target = nnz * p / n_parts;
    int lo = 0, hi = n_rows;  // first r in [0, n_rows] with row_ptr[r] >= target
    while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        if (row_ptr[mid] >= target) hi = mid;
        else lo = mid + 1;
    }
    parts[p] = p == n_parts ? n_rows : lo;
}

// ------------------------------------------------------------ tiled layout

// Keys of the tiled layout: entry e sits at output row m and input row n of
// the product (m = its slice and n = its index when the walked layout already
// runs along the output (MAJOR_IS_OUT), the other way round otherwise). Input
// rows are cut into tiles of tr rows: the entry's virtual slice is
// (n / tr) * n_out + m and its index the row inside the tile, n % tr.
// minor_of (the entry's slice on input) is overwritten with that index.
template <bool MAJOR_IS_OUT>
__global__ void __launch_bounds__(256)
k_tile_keys(int nnz, const int *__restrict__ idx, int *__restrict__ minor_of, int tr, int n_out,
            int *__restrict__ vkey) {
    const int stride = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += stride) {
        const int m = MAJOR_IS_OUT ? minor_of[e] : idx[e];
        const int n = MAJOR_IS_OUT ? idx[e] : minor_of[e];
        const int t = n / tr;
        vkey[e] = t * n_out + m;
        minor_of[e] = n - t * tr;
    }
}

// tptr[b] = the first position of key b in the sorted keys, or the position
// of the next larger key (nnz past the last): the bins in (keys[e-1], keys[e]]
// all start at e.
__global__ void __launch_bounds__(256)
k_bin_starts(int nnz, const uint32_t *__restrict__ keys, int n_bins, int *__restrict__ tptr) {
    const int stride = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e <= nnz; e += stride) {
        const int lo = e == 0 ? 0 : (int)keys[e - 1] + 1;
        const int hi = e == nnz ? n_bins : (int)keys[e];
        for (int b = lo; b <= hi; ++b) tptr[b] = e;
    }
}

// out[k] = the sum over t = 0 .. tiles-1 of part[t * n + k]: the tiles'
// partial rows of a tiled walk, added in a fixed order. A block of 256 threads
// takes 64 consecutive elements; its four thread quarters each add a run of
// consecutive tiles in order (all of a run's loads issued before its adds),
// then quarter 0 adds the four runs in order. Spreading an element over four
// threads keeps the short kernel from being one long chain of load latencies.
// With few tiles per run over many outputs, a pass takes four chunks of 64
// elements; each element's order of adds is the same either way.
__global__ void __launch_bounds__(256)
k_tile_sum(const float *__restrict__ part, float *__restrict__ out, int tiles, size_t n) {
    __shared__ float run[4][64];
    const int e = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int per = (tiles + 3) >> 2;  // tiles per run
    const int t0 = q * per, t1 = min(tiles, t0 + per);
    if (per <= 4 && n >= (size_t)gridDim.x * 256) {
        // few tiles per run over many outputs (the grid loops): four chunks
        // of 64 elements per pass, so a thread has up to 16 loads in flight
        // (1M x 20k at width 8, 5 tiles: 0.78 ms against 0.81)
        __shared__ float run4[4][4][64];
        for (size_t base = (size_t)blockIdx.x * 256; base < n; base += (size_t)gridDim.x * 256) {
            float x[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const size_t k = base + 64 * u + e;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    x[u][j] = k < n && t0 + j < t1 ? __builtin_nontemporal_load(part + (size_t)(t0 + j) * n + k) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float a = x[u][0];
#pragma unroll
                for (int j = 1; j < 4; ++j)
                    if (t0 + j < t1) a = a + x[u][j];
                run4[u][q][e] = a;
            }
            __syncthreads();
            if (q == 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const size_t k = base + 64 * u + e;
                    if (k < n) {
                        float s = run4[u][0][e];
                        for (int r = 1; r < 4; ++r)
                            if (r * per < tiles) s += run4[u][r][e];
                        out[k] = s;
                    }
                }
            }
            __syncthreads();
        }
        return;
    }
    for (size_t base = (size_t)blockIdx.x * 64; base < n; base += (size_t)gridDim.x * 64) {
        const size_t k = base + e;
        float a = 0.f;
        if (k < n) {
            for (int tb = t0; tb < t1; tb += 16) {
                float x[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    x[j] = tb + j < t1 ? __builtin_nontemporal_load(part + (size_t)(tb + j) * n + k) : 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (tb + j < t1) a = (tb + j == t0) ? x[j] : a + x[j];
                }
            }
        }
        run[q][e] = a;
        __syncthreads();
        if (q == 0 && k < n) {
            float s = run[0][e];
            for (int r = 1; r < 4; ++r)
                if (r * per < tiles) s += run[r][e];
            out[k] = s;
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------- utilities

// Fill n bytes (a multiple of 4) at p with zeros; p is 4-byte aligned.
// he[s] = value_ptr[major_ptr[s]] for s = 0 .. n_slices: the first entry of
// each VCS slice (and the entry count at the end). Group numbers are clamped
// to [0, n_groups], so a malformed structure reads nothing out of bounds.
__global__ void __launch_bounds__(256)
k_slice_starts(int n_slices, int n_groups, const int *__restrict__ sptr,
               const int *__restrict__ vptr, int *__restrict__ he) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s <= n_slices; s += gridDim.x * blockDim.x)
        he[s] = vptr[min(max(sptr[s], 0), n_groups)];
}

// The starts of the waves of a k_vcs_seg launch of `grid` blocks of `wpb`
// waves over a VCS of n_slices slices (as `tiles` runs): block b owns the
// slices seg_block_range gives it; its waves cut the block's entries into
// wpb shares, and wave k takes the slices that start in its share (the last
// wave also every empty slice at the end). One thread per wave. Reads stay in
// bounds for any structure (group numbers clamped to [0, n_groups]); a
// malformed one gets a meaningless plan, as its products are undefined.
//
// The shares of a 16-wave block are not equal. Its waves go to the CU's four
// SIMDs in turn, so wave k is the (k / 4)-th wave on its SIMD, and a SIMD
// issues from its oldest wave first: with equal shares the block's first
// four waves end well before its last four, whose SIMDs then run with fewer
// waves than they can overlap. Shares weighted 20 : 17 : 15 : 12 by that
// place (with k_vcs_seg's issue priorities) let a block's waves end nearly
// together. Blocks of 4 waves (one per SIMD) take equal shares. The weights
// change only which wave walks a slice, never the slice's result.
__global__ void __launch_bounds__(256)
k_seg_plan(int n_slices, int n_groups, const int *__restrict__ sptr,
           const int *__restrict__ vptr, const int *__restrict__ he, int tiles, int grid, int wpb,
           SegDesc *__restrict__ desc) {
    const int gw = blockIdx.x * blockDim.x + threadIdx.x;
    if (gw >= grid * wpb) return;
    const int b = gw / wpb, w = gw - b * wpb;
    int bb, be, tile;
    seg_block_range(b, grid, tiles, n_slices, bb, be, tile);
    const int EB = he[bb], EE = he[be];
    // share weights by a wave's place on its SIMD (blocks of 16 waves, four
    // per SIMD; smaller blocks put one wave per SIMD and take equal shares)
    auto weight = [&](int k) {
        const int place = k >> 2;
        return wpb != 16 ? 1 : place == 0 ? 20 : place == 1 ? 17 : place == 2 ? 15 : 12;
    };
    long long w_all = 0;
    for (int k = 0; k < wpb; ++k) w_all += weight(k);
    auto first_at = [&](int k) {  // the first slice in [bb, be] starting at or after cut k
        if (k >= wpb) return be;
        long long w_before = 0;
        for (int j = 0; j < k; ++j) w_before += weight(j);
        const int cut = EB + (int)((long long)(EE - EB) * w_before / w_all);
        int lo = bb, hi = be;  // he[be] = EE >= cut
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (he[mid] >= cut) hi = mid;
            else lo = mid + 1;
        }
        return lo;
    };
    SegDesc d;
    d.s_a = first_at(w);
    d.s_b = first_at(w + 1);
    d.E_a = he[d.s_a];
    d.E_b = he[d.s_b];
    d.K_b = min(max(sptr[d.s_b], 0), n_groups);
    // the last group of the run starting at or before E_a (groups before it
    // are empty: slice s_a's first group starts at E_a)
    int lo = min(max(sptr[d.s_a], 0), d.K_b), hi = d.K_b - 1;
    if (d.E_a < d.E_b) {
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (vptr[mid] <= d.E_a) lo = mid;
            else hi = mid - 1;
        }
    }
    d.K_a = lo;
    d.pad0 = d.pad1 = 0;
    desc[gw] = d;
}

__global__ void __launch_bounds__(256) k_zero(uint32_t *__restrict__ p, size_t n_words) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uintptr_t mis = ((uintptr_t)p >> 2) & 3;  // words before 16-byte alignment
    const size_t head = mis ? (4 - mis) : 0;
    if (head >= n_words) {
        if (t < n_words) p[t] = 0;
        return;
    }
    if (t < head) p[t] = 0;
    uint4 *q = reinterpret_cast<uint4 *>(p + head);
    const size_t n4 = (n_words - head) >> 2;
    for (size_t k = t; k < n4; k += stride) q[k] = make_uint4(0, 0, 0, 0);
    const size_t tail0 = head + (n4 << 2);
    if (t < n_words - tail0) p[tail0 + t] = 0;
}

// out[i] += src[i] for i < n (the fixed-order sum of row-block products).
template <typename T>
__global__ void __launch_bounds__(256) k_accumulate(T *__restrict__ out, const T *__restrict__ src,
                                                    size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] += src[i];
}

// dst[r][c] = src[r][c] * stat[r] for an n_rows x w row-major block (dst may
// be src): one thread per row chunk of 64 elements, so the row's factor is
// read once.
template <typename T>
__global__ void __launch_bounds__(256)
k_scale_rows(T *dst, const T *src, const T *__restrict__ stat, long long n_rows, int w) {
    const long long chunks = (w + 63) / 64;
    const long long n = n_rows * chunks;
    const long long stride = (long long)gridDim.x * (blockDim.x >> 6);
    const int lane = threadIdx.x & 63;
    for (long long q = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); q < n;
         q += stride) {
        const long long r = q / chunks;
        const int c = (int)(q - r * chunks) * 64 + lane;
        if (c < w) {
            const size_t e = (size_t)r * w + c;
            dst[e] = src[e] * stat[r];
        }
    }
}

// Structure checks: flag bit 1 = pointer array does not start at 0, bit 2 =
// decreasing, bit 4 = last pointer differs from count, bit 8 = index out of
// range.
__global__ void __launch_bounds__(256)
k_validate_ptr(const int *__restrict__ ptr, int n, int count, int *__restrict__ flag) {
    const int stride = gridDim.x * blockDim.x;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i <= n; i += stride) {
        const int a = ptr[i];
        int f = 0;
        if (i == 0 && a != 0) f |= 1;
        if (i < n && ptr[i + 1] < a) f |= 2;
        if (i == n && a != count) f |= 4;
        if (f) atomicOr(flag, f);
    }
}

__global__ void __launch_bounds__(256)
k_validate_idx(const int *__restrict__ idx, int nnz, int n_minor, int *__restrict__ flag) {
    const int stride = gridDim.x * blockDim.x;
    int f = 0;
    for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += stride) {
        const int i = idx[p];
        if (i < 0 || i >= n_minor) f = 8;
    }
    if (f) atomicOr(flag, f);
}

}  // namespace vspmm
