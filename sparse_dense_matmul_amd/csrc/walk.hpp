// Slice walks for gfx950 (wave64): the plain aligned walk (output rows are
// the layout's major slices) and the helpers the walk families share. It
// follows the lane split of the vsparse page, section "The
// kernels", widened to a 64-lane wave: a slice is walked by G "entry lanes"
// that take its entries in stride, and each entry lane is WW "width lanes"
// wide, each covering VEC consecutive elements of the dense width. With
// G * WW < 64, a wave walks R = 64 / (G * WW) slices side by side (the
// regridding page's row groups, section "How it is built").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace vspmm {



template <typename T, int N>
struct vec_of {
    typedef T type __attribute__((ext_vector_type(N)));
};
template <typename T>
struct vec_of<T, 1> {
    typedef T type;
};

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T *p, T (&r)[N]) {
    if constexpr (N == 1) {
        r[0] = *p;
    } else {
        const auto x = *reinterpret_cast<const typename vec_of<T, N>::type *>(p);
#pragma unroll
        for (int e = 0; e < N; ++e) r[e] = x[e];
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_vec(T *p, const T (&r)[N]) {
    if constexpr (N == 1) {
        *p = r[0];
    } else {
        typename vec_of<T, N>::type x;
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = r[e];
        *reinterpret_cast<typename vec_of<T, N>::type *>(p) = x;
    }
}

__device__ __forceinline__ float fma_t(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_t(double a, double b, double c) { return __builtin_fma(a, b, c); }

__device__ __forceinline__ int readlane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float readlane(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ void atomic_add_t(float *p, float v) { unsafeAtomicAdd(p, v); }
__device__ __forceinline__ void atomic_add_t(double *p, double v) { unsafeAtomicAdd(p, v); }

// The G entry lanes of a slice are summed by a fixed butterfly over the slot
// bits of the lane id (bits log_ww .. log_ww + log_g - 1), highest bit first:
// at each level a lane adds the partial of the lane whose id differs in that
// bit. The pairing and order depend only on G, never on the width lanes, so
// a column gets the same bits in any batch. slot_reduce_dpp does it with
// cross-lane VALU ops for a full wave (G * WW == 64), slot_reduce_sub for
// sub-waves.

// One butterfly level on a 32-bit value: partner differs in lane bit `bit`.
__device__ __forceinline__ float level_f(float v, int bit) {
    const uint32_t u = __float_as_uint(v);
    switch (bit) {
        case 5: {
            const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            return __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
        case 4: {
            const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            return __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
        // within a row of 16 the rotations pair lanes like xor because the
        // higher in-row bit was already summed (partials are equal there)
        case 3: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xf, 0xf, false));
        case 2: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xf, 0xf, false));
        case 1: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xf, 0xf, false));
        default: return v + __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xf, 0xf, false));
    }
}

__device__ __forceinline__ double partner_d(double v, int bit) {
    const unsigned long long u = __double_as_longlong(v);
    uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    uint32_t plo, phi;
    switch (bit) {
        case 5: {
            const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
            const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
            // lanes in the low half get the partner from the second result
            const bool low = (__lane_id() & 32) == 0;
            plo = low ? a[1] : a[0];
            phi = low ? b[1] : b[0];
            break;
        }
        case 4: {
            const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
            const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
            const bool even = (__lane_id() & 16) == 0;
            plo = even ? a[1] : a[0];
            phi = even ? b[1] : b[0];
            break;
        }
        default: {
            const int ctrl = bit == 3 ? 0x128 : bit == 2 ? 0x124 : bit == 1 ? 0x4E : 0xB1;
            switch (ctrl) {
                case 0x128:
                    plo = __builtin_amdgcn_update_dpp(0, (int)lo, 0x128, 0xf, 0xf, false);
                    phi = __builtin_amdgcn_update_dpp(0, (int)hi, 0x128, 0xf, 0xf, false);
                    break;
                case 0x124:
                    plo = __builtin_amdgcn_update_dpp(0, (int)lo, 0x124, 0xf, 0xf, false);
                    phi = __builtin_amdgcn_update_dpp(0, (int)hi, 0x124, 0xf, 0xf, false);
                    break;
                case 0x4E:
                    plo = __builtin_amdgcn_update_dpp(0, (int)lo, 0x4E, 0xf, 0xf, false);
                    phi = __builtin_amdgcn_update_dpp(0, (int)hi, 0x4E, 0xf, 0xf, false);
                    break;
                default:
                    plo = __builtin_amdgcn_update_dpp(0, (int)lo, 0xB1, 0xf, 0xf, false);
                    phi = __builtin_amdgcn_update_dpp(0, (int)hi, 0xB1, 0xf, 0xf, false);
                    break;
            }
        }
    }
    return __longlong_as_double((long long)(((unsigned long long)phi << 32) | plo));
}

// The levels are unrolled so each one's lane pattern is an immediate; a
// level below the width lanes is skipped by one uniform branch.
template <typename T, int VEC>
__device__ __forceinline__ void slot_reduce_dpp(T (&acc)[VEC], int log_ww) {
#pragma unroll
    for (int bit = 5; bit >= 0; --bit) {
        if (bit < log_ww) break;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (sizeof(T) == 4) acc[e] = level_f(acc[e], bit);
            else acc[e] = acc[e] + partner_d(acc[e], bit);
        }
    }
}

// The same tree for sub-waves of 2^log_sub lanes, with the full-wave
// patterns where they pair lanes exactly like xor: the swaps at bits 5 and 4
// and the in-row rotations at bits 3, 1 and 0 always do; the rotation at bit
// 2 does once bit 3 is summed (log_sub > 3), else a lane shuffle is used.
template <typename T, int VEC>
__device__ __forceinline__ void slot_reduce_sub(T (&acc)[VEC], int log_ww, int log_sub) {
#pragma unroll
    for (int bit = 5; bit >= 0; --bit) {
        if (bit >= log_sub) continue;
        if (bit < log_ww) break;
        if (bit == 2 && log_sub == 3) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], 4);
            continue;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (sizeof(T) == 4) acc[e] = level_f(acc[e], bit);
            else acc[e] = acc[e] + partner_d(acc[e], bit);
        }
    }
}

// Walks the entries [e0, e1) of one slice in steps of G. For a VCS slice the
// value of each entry is its group's: with UNIFORM (one slice per wave) the
// wave keeps up to 64 group starts and values in lanes and advances a
// wave-uniform group cursor with readlane; otherwise each lane keeps its own
// cursor. Calls body(p, index, value) for the lane's entry p of each step
// (p >= e1 marks an idle lane).
template <bool VCS, bool UNIFORM, typename T, typename VP, typename Body>
__device__ __forceinline__ void walk_slice(int lane, int slot, int G, int ka, int kb, int e0,
                                           int e1, const int *__restrict__ vptr, VP vals,
                                           const int *__restrict__ idx, Body &&body) {
    if constexpr (!VCS) {
        // the next step's index and value are loaded (clamped to the slice)
        // before this step's body, so they are in flight with its gathers
        if (e0 >= e1) return;
        int pn = min(e0 + slot, e1 - 1);
        int i_n = idx[pn];
        T v_n = vals[pn];
        for (int q = e0; q < e1; q += G) {
            const bool valid = q + slot < e1;
            const int i = i_n;
            const T v = v_n;
            pn = min(q + G + slot, e1 - 1);
            i_n = idx[pn];
            v_n = vals[pn];
            body(valid, i, v);
        }
    } else if constexpr (UNIFORM) {
        if (kb <= ka) return;
        int gb = ka;  // group held by lane 0
        int u = 0;    // current group, as a lane of the window (wave-uniform)
        int gs = vptr[min(gb + lane, kb)];        // start of group gb + lane
        T gv = vals[min(gb + lane, kb - 1)];      // value of group gb + lane
        for (int q = e0; q < e1; q += G) {
            const int p = q + slot;
            const bool valid = p < e1;
            const int i = valid ? idx[p] : 0;
            const int qend = min(q + G, e1);
            T v = readlane(gv, u);
            for (;;) {
                if (u == 63) {  // slide the window of group starts
                    gb += 63;
                    u = 0;
                    gs = vptr[min(gb + lane, kb)];
                    gv = vals[min(gb + lane, kb - 1)];
                }
                const int ns = readlane(gs, u + 1);
                if (ns >= qend) break;
                ++u;
                const T nv = readlane(gv, u);
                v = (p >= ns) ? nv : v;
            }
            body(valid, i, v);
        }
    } else {
        int kc = ka;
        int kend = (kb > ka) ? vptr[ka + 1] : 0;
        for (int q = e0; q < e1; q += G) {
            const int p = q + slot;
            const bool valid = p < e1;
            const int i = valid ? idx[p] : 0;
            T v = T(0);
            if (valid) {
                while (p >= kend) {
                    ++kc;
                    kend = vptr[kc + 1];
                }
                v = vals[kc];
            }
            body(valid, i, v);
        }
    }
}

// Aligned walk: out[s][:] = sum over the entries (s, i, v) of slice s of
// v * B[i][:]. Each lane accumulates its own entries in order with fused
// multiply-adds, then the G entry lanes are summed by a fixed xor tree, so the
// result depends only on the matrix and G, never on timing.
//   sptr: CSR row pointers or VCS major_ptr; vptr: VCS value_ptr (unused for
//   CSR); vals: CSR values or VCS group values; idx: minor indices;
//   B: n_minor x w; out: n_slices x w.
template <bool VCS, typename T, int VEC, bool UNIFORM, typename VP = const T *>
__global__ void __launch_bounds__(256)
k_aligned(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
          VP vals, const int *__restrict__ idx,
          const T *__restrict__ B, T *__restrict__ out, int w, Split sp, int long_len) {
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int log_sub = sp.log_ww + sp.log_g;
    const int G = 1 << sp.log_g;
    const int sub = lane >> log_sub;
    const int slot = (lane >> sp.log_ww) & (G - 1);
    const int cl = lane & ((1 << sp.log_ww) - 1);
    const int R = 64 >> log_sub;
    const int chunk = VEC << sp.log_ww;
    const int stride = gridDim.x * waves * R;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int s = (blockIdx.x * waves + wave) * R + (UNIFORM ? 0 : sub); s < n_slices;
         s += stride) {
        int e0, e1, ka = 0, kb = 0;
        if constexpr (VCS) {
            ka = sptr[s];
            kb = sptr[s + 1];
            e0 = vptr[ka];
            e1 = vptr[kb];
        } else {
            e0 = sptr[s];
            e1 = sptr[s + 1];
        }
        // a slice longer than long_len is left to the long walk (k_long over
        // the handle's list of long slices): walked here as empty, not written
        const bool skip = e1 - e0 > long_len;
        if (skip) e1 = e0;
        for (int c0 = 0; c0 < w; c0 += chunk) {
            const int col = c0 + cl * VEC;
            const bool act = col < w && !skip;
            T acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = T(0);
            walk_slice<VCS, UNIFORM, T>(lane, slot, G, ka, kb, e0, e1, vptr, vals, idx,
                                        [&](bool valid, int i, T v) {
                                            // the gather is issued by every
                                            // lane (row 0 / column 0 when
                                            // idle); only the FMA is masked
                                            T b[VEC];
                                            load_vec<T, VEC>(B + (size_t)(valid ? i : 0) * w +
                                                                 (act ? col : 0), b);
                                            if (valid && act) {
#pragma unroll
                                                for (int e = 0; e < VEC; ++e)
                                                    acc[e] = fma_t(v, b[e], acc[e]);
                                            }
                                        });
            slot_reduce_sub<T, VEC>(acc, sp.log_ww, log_sub);
            if (slot == 0 && act) store_vec<T, VEC>(out + (size_t)s * w + col, acc);
        }
    }
}

}  // namespace vspmm
