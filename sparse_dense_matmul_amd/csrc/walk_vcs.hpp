// Aligned walk over short VCS slices with the work in vector instructions.
//
// One wave walks a contiguous block of slices in rounds (see Round in
// walk_fast.hpp): a round's entry windows (lane t of window k holds entry
// E0 + 64k + t), group windows and slice pointers are loaded at once. The
// round is then walked window by window, and everything per entry is done by
// vector instructions, because a CU has one scalar unit shared by all its
// waves and per-step scalar decisions would bound the kernel:
//
//  - the value of each entry of a window is found without a loop: every group
//    starting inside the window marks its start position in a per-wave LDS
//    row (LDS max keeps the last of several empty groups), a max-scan across
//    the lanes gives each position the last group started at or before it,
//    and the group's value is shuffled in from the group windows;
//  - steps are aligned to the window, not to the slice: step j of window k
//    gives entry lane `slot` the entry E0 + 64k + jG + slot, with its index
//    and value shuffled from the window registers;
//  - a slice that ends inside a step is closed there: the lanes holding its
//    entries add them, the G entry lanes are summed by the fixed butterfly and
//    the row is written, and the remaining lanes start the next slice.
//
// Each entry lane accumulates its entries of a slice in increasing position
// order with fused multiply-adds; the summation order depends only on the
// matrix and the launch shape, so results repeat bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "walk.hpp"
#include "walk_fast.hpp"

namespace vspmm {

// Inclusive max-scan of a per-lane int across the wave (DPP row shifts within
// rows of 16, then the row broadcasts).
__device__ __forceinline__ int wave_max_scan(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}

// Sum of the G entry lanes, compile-time width-lane count.
template <int LOG_WW, typename T, int VEC>
__device__ __forceinline__ void slot_sum(T (&acc)[VEC]) {
#pragma unroll
    for (int bit = 5; bit >= LOG_WW; --bit) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (sizeof(T) == 4) acc[e] = level_f(acc[e], bit);
            else acc[e] = acc[e] + partner_d(acc[e], bit);
        }
    }
}

template <int LOG_WW, bool LDS_B, int VEC>
__global__ void __launch_bounds__(1024)
k_vcs_rows(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
           const float *__restrict__ vals, const int *__restrict__ idx,
           const float *__restrict__ B, float *__restrict__ out, int w, int n_in) {
    using T = float;
    constexpr int NWR = 24;
    constexpr int GWR = 4;
    constexpr int G = 64 >> LOG_WW;
    constexpr int NSTEP = 64 / G;  // steps per window
    // steps per sub-batch: gathers of one sub-batch are in flight together
    constexpr int SBV = NSTEP < (VEC >= 4 ? 4 : 8) ? NSTEP : (VEC >= 4 ? 4 : 8);
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int slot = lane >> LOG_WW;
    const int cl = lane & ((1 << LOG_WW) - 1);
    const int chunk = VEC << LOG_WW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t b_bytes = LDS_B ? (((size_t)n_in * w * sizeof(T) + 15) & ~size_t(15)) : 0;
    int *mark = reinterpret_cast<int *>(smem + b_bytes) + wave * 64;
    const long long tw = (long long)gridDim.x * waves;
    const long long gw = (long long)blockIdx.x * waves + wave;
    const int s_beg = (int)(gw * n_slices / tw);
    const int s_end = (int)((gw + 1) * n_slices / tw);

    Round r;
    int W[NWR], GS[GWR];
    T V[NWR], GV[GWR];
    if (s_beg < s_end) {
        round_plan<true, NWR, GWR>(r, s_beg, s_end, n_slices, lane, sptr, vptr);
        if (r.nsl > 0) round_load<true, T, NWR, GWR>(r, W, V, GS, GV, lane, vptr, vals, idx);
    }

    const T *Bs = B;
    if constexpr (LDS_B) {
        T *lb = reinterpret_cast<T *>(smem);
        const size_t n_el = (size_t)n_in * w;
        if ((n_el * sizeof(T)) % 16 == 0 && ((uintptr_t)B % 16) == 0) {
            const uint4 *src = reinterpret_cast<const uint4 *>(B);
            uint4 *dst = reinterpret_cast<uint4 *>(lb);
            for (size_t k = threadIdx.x; k < n_el * sizeof(T) / 16; k += blockDim.x)
                dst[k] = src[k];
        } else {
            for (size_t k = threadIdx.x; k < n_el; k += blockDim.x) lb[k] = B[k];
        }
        __syncthreads();
        Bs = lb;
    }

    int sa = s_beg;
    while (sa < s_end) {
        if (r.nsl < 0) {  // one slice larger than a round
            big_slice<true, T, VEC, 4>(sa, lane, slot, cl, Split{LOG_WW, 6 - LOG_WW}, sptr, vptr,
                                       vals, idx, Bs, out, w);
            sa += 1;
        } else {
            for (int c0 = 0; c0 < w; c0 += chunk) {
                const int col = c0 + cl * VEC;
                const bool act = col < w;
                int i = 0;                    // slice of the round being accumulated
                int e1 = readlane(r.he, 1);   // its end
                int carry = 0;                // group (round-relative) of the previous position
                T acc[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = T(0);
                // empty slices before the first entry
                while (i < r.nsl && e1 <= r.E0) {
                    slot_sum<LOG_WW, T, VEC>(acc);
                    if (slot == 0 && act)
                        store_vec<T, VEC>(out + (size_t)(r.sa + i) * w + col, acc);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = T(0);
                    ++i;
                    if (i < r.nsl) e1 = readlane(r.he, i + 1);
                }
                const int nwin = (r.E1 - r.E0 + 63) >> 6;
                for (int k = 0; k < nwin; ++k) {
                    const int wbase = r.E0 + 64 * k;
                    const int wi = W[k];
                    // value of each position of the window
                    mark[lane] = INT_MIN;
#pragma unroll
                    for (int j = 0; j < GWR; ++j) {
                        const int gidx = 64 * j + lane;  // round-relative group
                        const int st = GS[j] - wbase;
                        if (gidx < r.K1 - r.K0 && st >= 0 && st < 64) atomicMax(&mark[st], gidx);
                    }
                    const int g = max(wave_max_scan(mark[lane]), carry);
                    carry = readlane(g, 63);
                    T vk = T(0);
#pragma unroll
                    for (int j = 0; j < GWR; ++j) {
                        const T t = __shfl(GV[j], g & 63);
                        vk = (g >> 6) == j ? t : vk;
                    }
                    // the window's steps in sub-batches: gathers first, then the sums
#pragma unroll 1
                    for (int j0 = 0; j0 < NSTEP; j0 += SBV) {
                        int pj[SBV];
                        T vj[SBV];
                        T bv[SBV][VEC];
#pragma unroll
                        for (int t = 0; t < SBV; ++t) {
                            const int src = (j0 + t) * G + slot;
                            const int ix = __shfl(wi, src);
                            vj[t] = __shfl(vk, src);
                            pj[t] = wbase + src;
                            if (act && pj[t] < r.E1) {
                                load_vec<T, VEC>(Bs + (size_t)ix * w + col, bv[t]);
                            } else {
#pragma unroll
                                for (int e = 0; e < VEC; ++e) bv[t][e] = T(0);
                            }
                        }
#pragma unroll
                        for (int t = 0; t < SBV; ++t) {
                            const int step_end = min(wbase + (j0 + t + 1) * G, r.E1);
                            // close every slice that ends inside this step
                            while (i < r.nsl && e1 < step_end) {
                                if (pj[t] < e1) {
#pragma unroll
                                    for (int e = 0; e < VEC; ++e)
                                        acc[e] = fma_t(vj[t], bv[t][e], acc[e]);
                                }
                                slot_sum<LOG_WW, T, VEC>(acc);
                                if (slot == 0 && act)
                                    store_vec<T, VEC>(out + (size_t)(r.sa + i) * w + col, acc);
#pragma unroll
                                for (int e = 0; e < VEC; ++e) acc[e] = T(0);
                                ++i;
                                const int e0n = e1;
                                if (i < r.nsl) e1 = readlane(r.he, i + 1);
                                // entries before the new slice's start are done
                                if (pj[t] < e0n) {
#pragma unroll
                                    for (int e = 0; e < VEC; ++e) bv[t][e] = T(0);
                                }
                            }
                            if (pj[t] < e1) {
#pragma unroll
                                for (int e = 0; e < VEC; ++e)
                                    acc[e] = fma_t(vj[t], bv[t][e], acc[e]);
                            }
                        }
                    }
                }
                // slices ending at the round's last entry, and empty ones after
                while (i < r.nsl) {
                    slot_sum<LOG_WW, T, VEC>(acc);
                    if (slot == 0 && act)
                        store_vec<T, VEC>(out + (size_t)(r.sa + i) * w + col, acc);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = T(0);
                    ++i;
                }
            }
            sa += r.nsl;
        }
        if (sa < s_end) {
            round_plan<true, NWR, GWR>(r, sa, s_end, n_slices, lane, sptr, vptr);
            if (r.nsl > 0) round_load<true, T, NWR, GWR>(r, W, V, GS, GV, lane, vptr, vals, idx);
        }
    }
}

}  // namespace vspmm
