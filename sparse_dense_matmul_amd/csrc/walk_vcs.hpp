// Aligned walk over short VCS slices with the work in vector instructions.
//
// One wave walks a contiguous block of slices in rounds (see Round in
// walk_fast.hpp): a round's entry windows (lane t of window k holds entry
// E0 + 64k + t), group windows and slice pointers are loaded at once. The
// round is then walked window by window with as few instructions per entry as
// the lane split allows, since a wave's vector and scalar issue slots, not
// memory, bound this walk once the dense operand sits in LDS:
//
//  - group values without a search: at the start of a round every non-empty
//    group writes its round-relative number (plus one) as a byte at its first
//    position in a per-wave LDS row, and its value into a per-wave table. A
//    window reads its 64 bytes, a DPP max-scan carries each group number over
//    the positions that follow it, and one LDS read fetches the value;
//  - steps are aligned to the window: step j gives entry lane `slot` the entry
//    E0 + 64k + jG + slot, its index and value shuffled from the window
//    registers. Gathers never need a mask: positions past the round's end hold
//    a clamped (valid) index;
//  - a step inside one slice accumulates without masks. A step in which a
//    slice ends closes it there: the lanes holding its entries add them, the G
//    entry lanes are summed (the two top butterfly levels split the lane's
//    elements between the partners instead of both keeping all of them), and
//    the row is written; the remaining lanes go on with the next slice.
//
// Each entry lane accumulates its entries of a slice in increasing position
// order with fused multiply-adds and the tree is fixed, so the summation order
// depends only on the matrix and the launch shape: results repeat bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "walk.hpp"
#include "walk_fast.hpp"

namespace vspmm {

// Inclusive max-scan of a per-lane int across the wave (DPP row shifts within
// rows of 16, then the row broadcasts). Lanes with no source keep their own
// value (the DPP result is then the lane's `old` operand, here 0).
__device__ __forceinline__ int wave_max_scan(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}

// Sum over the G = 64 >> LOG_WW entry lanes of each width lane's VEC
// elements. At lane bit 5 (and then 4), when a lane holds two or more
// elements, partners swap halves (permlane32/16 swap) so each keeps the total
// of half of them; the remaining levels add the partner's value (DPP).
// Afterwards a lane holds VO elements starting at element base(lane), and the
// lanes whose plainly summed slot bits are zero hold every element once.
template <int LOG_WW, int VEC>
struct SlotSum {
    static constexpr bool H5 = LOG_WW <= 5 && VEC >= 2;
    static constexpr int V5 = H5 ? VEC / 2 : VEC;
    static constexpr bool H4 = LOG_WW <= 4 && V5 >= 2;
    static constexpr int VO = H4 ? V5 / 2 : V5;
    // slot bits summed by adding the partner (their lanes hold copies)
    static constexpr int PLAIN = (0x3f & ~((1 << LOG_WW) - 1)) & ~(H5 ? 32 : 0) & ~(H4 ? 16 : 0);

    __device__ static __forceinline__ int base(int lane) {
        return (H5 ? ((lane >> 5) & 1) * V5 : 0) + (H4 ? ((lane >> 4) & 1) * VO : 0);
    }
    __device__ static __forceinline__ bool writer(int lane) { return (lane & PLAIN) == 0; }

    __device__ static __forceinline__ void run(const float (&acc)[VEC], float (&res)[VO]) {
        float a5[V5];
        if constexpr (H5) {
#pragma unroll
            for (int e = 0; e < V5; ++e) {
                const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]),
                                                                __float_as_uint(acc[e + V5]),
                                                                false, false);
                a5[e] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < V5; ++e) a5[e] = LOG_WW <= 5 ? level_f(acc[e], 5) : acc[e];
        }
        if constexpr (H4) {
#pragma unroll
            for (int e = 0; e < VO; ++e) {
                const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a5[e]),
                                                                __float_as_uint(a5[e + VO]),
                                                                false, false);
                res[e] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < VO; ++e) res[e] = LOG_WW <= 4 ? level_f(a5[e], 4) : a5[e];
        }
#pragma unroll
        for (int bit = 3; bit >= LOG_WW; --bit) {
#pragma unroll
            for (int e = 0; e < VO; ++e) res[e] = level_f(res[e], bit);
        }
    }
};

template <int LOG_WW, bool LDS_B, int VEC>
__global__ void __launch_bounds__(1024)
k_vcs_rows(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
           const float *__restrict__ vals, const int *__restrict__ idx,
           const float *__restrict__ B, float *__restrict__ out, int w, int n_in) {
    using T = float;
    using Sum = SlotSum<LOG_WW, VEC>;
    constexpr int NWR = kRowsNWR;
    constexpr int GWR = kRowsGWR;
    static_assert(NWR == 16, "one 16-byte mark word per lane");
    static_assert(64 * NWR + 256 * GWR == kRowsWaveLds, "per-wave LDS layout");
    constexpr int G = 64 >> LOG_WW;
    constexpr int NSTEP = 64 / G;  // steps per window
    // steps per sub-batch: the gathers of one sub-batch are in flight together
    constexpr int SBV = NSTEP < (VEC >= 4 ? 4 : 8) ? NSTEP : (VEC >= 4 ? 4 : 8);
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int slot = lane >> LOG_WW;
    const int cl = lane & ((1 << LOG_WW) - 1);
    const int chunk = VEC << LOG_WW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t b_bytes = LDS_B ? (((size_t)n_in * w * sizeof(T) + 15) & ~size_t(15)) : 0;
    // per wave: [64*NWR mark bytes][64*GWR group values]
    unsigned char *mark = smem + b_bytes + (size_t)wave * kRowsWaveLds;
    T *gvt = reinterpret_cast<T *>(mark + 64 * NWR);
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
            // the round's group starts (bytes) and values (table)
            reinterpret_cast<uint4 *>(mark)[lane] = make_uint4(0, 0, 0, 0);
            const int n_grp = r.K1 - r.K0;
#pragma unroll
            for (int j = 0; j < GWR; ++j) {
                gvt[64 * j + lane] = GV[j];
                int nxt = __shfl_down(GS[j], 1);
                if (j + 1 < GWR) {
                    const int first_next = readlane(GS[j + 1 < GWR ? j + 1 : j], 0);
                    nxt = lane == 63 ? first_next : nxt;
                }
                const int gidx = 64 * j + lane;
                if (gidx < n_grp && nxt > GS[j]) mark[GS[j] - r.E0] = (unsigned char)(gidx + 1);
            }
            __builtin_amdgcn_wave_barrier();
            const int nwin = (r.E1 - r.E0 + 63) >> 6;
            for (int c0 = 0; c0 < w; c0 += chunk) {
                const int col = c0 + cl * VEC;
                const bool act = col < w;
                const int coff = act ? col : 0;  // gathers stay inside B's rows
                int i = 0;                       // slice of the round being accumulated
                int e0 = r.E0;                   // its first entry
                int e1 = readlane(r.he, 1);      // its end
                int carry = 0;                   // group number reaching the window start
                T acc[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = T(0);

                // sums slice i over the entry lanes, writes its row, moves on
                auto close = [&]() {
                    T res[Sum::VO];
                    Sum::run(acc, res);
                    if (Sum::writer(lane) && act) {
                        T *o = out + (size_t)(r.sa + i) * w + col + Sum::base(lane);
                        store_vec<T, Sum::VO>(o, res);
                    }
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = T(0);
                    ++i;
                    e0 = e1;
                    if (i < r.nsl) e1 = readlane(r.he, i + 1);
                };

                // empty slices before the first entry
                while (i < r.nsl && e1 <= r.E0) close();
                for (int k = 0; k < nwin; ++k) {
                    const int wbase = r.E0 + 64 * k;
                    const int wi = W[k];
                    const int g = max(wave_max_scan((int)mark[64 * k + lane]), carry);
                    carry = readlane(g, 63);
                    const T vk = gvt[g - 1];
#pragma unroll 1
                    for (int j0 = 0; j0 < NSTEP; j0 += SBV) {
                        T vj[SBV];
                        T bv[SBV][VEC];
#pragma unroll
                        for (int t = 0; t < SBV; ++t) {
                            const int src = (j0 + t) * G + slot;
                            const int ix = __shfl(wi, src);
                            vj[t] = __shfl(vk, src);
                            // LDS rows: n_in * w < 2^24 (a 24-bit multiply is full rate)
                            const size_t at = LDS_B ? size_t(__umul24(ix, w) + coff)
                                                    : size_t(ix) * size_t(w) + size_t(coff);
                            load_vec<T, VEC>(Bs + at, bv[t]);
                        }
#pragma unroll
                        for (int t = 0; t < SBV; ++t) {
                            const int step_end = wbase + (j0 + t + 1) * G;
                            if (i < r.nsl && e1 >= step_end) {
                                // every lane of the step is in slice i
#pragma unroll
                                for (int e = 0; e < VEC; ++e)
                                    acc[e] = fma_t(vj[t], bv[t][e], acc[e]);
                            } else {
                                const int pj = wbase + (j0 + t) * G + slot;
                                while (i < r.nsl && e1 < step_end) {
                                    if (pj >= e0 && pj < e1) {
#pragma unroll
                                        for (int e = 0; e < VEC; ++e)
                                            acc[e] = fma_t(vj[t], bv[t][e], acc[e]);
                                    }
                                    close();
                                }
                                if (i < r.nsl && pj >= e0) {
#pragma unroll
                                    for (int e = 0; e < VEC; ++e)
                                        acc[e] = fma_t(vj[t], bv[t][e], acc[e]);
                                }
                            }
                        }
                    }
                }
                // slices ending at the round's last entry, and empty ones after
                while (i < r.nsl) close();
            }
            sa += r.nsl;
            __builtin_amdgcn_wave_barrier();
        }
        if (sa < s_end) {
            round_plan<true, NWR, GWR>(r, sa, s_end, n_slices, lane, sptr, vptr);
            if (r.nsl > 0) round_load<true, T, NWR, GWR>(r, W, V, GS, GV, lane, vptr, vals, idx);
        }
    }
}

}  // namespace vspmm
