// Aligned walk over VCS slices: each wave walks one contiguous run of entries,
// windows packed across slice boundaries.
//
// A block (one per CU when B is staged in LDS) owns a contiguous range of
// slices; its 16 waves cut the range's entries into runs (cut at slice
// starts) sized by each wave's place on its SIMD (k_seg_plan), so the waves
// of a SIMD end about together whatever the slice lengths. A run is
// taken in rounds of at most 64 * kRowsNWR entries and 64 * kRowsGWR - 1
// groups, whose index windows, group starts and group values are loaded one
// round ahead. Inside a round:
//
//  - group of each entry without a search: every group starting in the round
//    writes its round-relative number (plus one) as a byte at its first
//    position in a per-wave LDS row; a window of 64 entries reads its bytes,
//    and a DPP max-scan carries each number over the positions after it;
//  - lane split (vsparse page, section "The kernels", widened to wave64): WW
//    lanes cover the width (VEC elements each) and G = 64 / WW entry slots
//    walk the entries; step t of a window gives slot q entry 64k + G t + q, so
//    a step covers G consecutive entries and a slice end splits at most one
//    step. Each window is loaded permuted (lane q WW + t holds entry G t + q)
//    so that a step hands every slot its entry by a broadcast inside its own
//    WW lanes (DPP quad_perm / row_newbcast, or ds_swizzle);
//  - a step entirely inside one slice is a gather and VEC fused multiply-adds
//    per lane, with no masks. A step holding a slice end adds the lanes before
//    the end, sums the G slots (SlotSum: two permlane swap levels, then DPP),
//    writes the row, and goes on with the lanes after it;
//  - each round notes, for every slice that closes in it, the window holding
//    its last entry; a window's ballot of that number picks its path: no end
//    (plain steps), one end (a straight-line copy of the window for the step
//    that holds it), or several ends, empty slices or the round's partial last
//    window (step by step).
//
// A wave's issue priority falls as it gets through its run (3 in the first
// quarter, 0 in the last): a SIMD otherwise issues from its oldest wave
// first, its waves drift apart, and the last one ends alone. With the plan's
// weighted shares a block's waves end nearly together.
//
// Each slot accumulates its entries of a slice in increasing position order
// with fused multiply-adds. A slice starting at slot r gives its entry j to
// slot (r + j) mod G, and the tree adds slots that differ in the highest slot
// bit first: slot s and s + G/2 (mod G), then within each half likewise, so
// every level pairs the same residue classes of j whatever r is. A slice's
// result thus depends only on its entries in stored order, not on where runs,
// rounds or windows start: results repeat bit for bit, whatever the plan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "launch.hpp"
#include "walk.hpp"
#include "walk_vcs.hpp"

namespace vspmm {

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order.
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Every lane L gets x from lane (L & ~(WW - 1)) + T: element T of its group of
// WW = 1 << LOG_WW lanes. (Every lane has a source, so the DPP forms' bound
// control changes nothing; set, it lets the compiler fold the move into the
// instruction that uses it.)
template <int LOG_WW, int T>
__device__ __forceinline__ int group_bcast(int x) {
    if constexpr (LOG_WW == 0) {
        return x;
    } else if constexpr (LOG_WW == 1) {
        return __builtin_amdgcn_update_dpp(0, x, T == 0 ? 0xA0 : 0xF5, 0xf, 0xf, true);  // [T,T,2+T,2+T]
    } else if constexpr (LOG_WW == 2) {
        return __builtin_amdgcn_update_dpp(0, x, T * 0x55, 0xf, 0xf, true);  // quad_perm [T,T,T,T]
    } else if constexpr (LOG_WW == 3) {
        // swizzle, bit mask mode within 32 lanes: keep lane bits 3-4, set T
        return __builtin_amdgcn_ds_swizzle(x, 0x18 | (T << 5));
    } else if constexpr (LOG_WW == 4) {
        return __builtin_amdgcn_update_dpp(0, x, 0x150 + T, 0xf, 0xf, true);  // row_newbcast:T
    } else if constexpr (LOG_WW == 5) {
        return __builtin_amdgcn_ds_swizzle(x, T << 5);  // lane T of each 32
    } else {
        return __builtin_amdgcn_readlane(x, T);
    }
}
template <int LOG_WW, int T>
__device__ __forceinline__ float group_bcast(float x) {
    return __int_as_float(group_bcast<LOG_WW, T>(__float_as_int(x)));
}

// One lane's VEC elements of a row of B at byte offset off: from LDS (B
// staged at the start of the kernel's dynamic LDS) or from global memory.
template <bool LDS_B, int VEC>
__device__ __forceinline__ void gather(const char *Bg, uint32_t off, float (&r)[VEC]) {
    if constexpr (LDS_B) {
        typedef __attribute__((address_space(3))) const typename vec_of<float, VEC>::type *lds_ptr;
        const auto x = *reinterpret_cast<lds_ptr>((uintptr_t)off);
        if constexpr (VEC == 1) {
            r[0] = x;
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) r[e] = x[e];
        }
    } else {
        load_vec<float, VEC>(reinterpret_cast<const float *>(Bg + off), r);
    }
}

// a * b + c, fused, into a register of its own (the three-address form; the
// compiler keeps a chain of fused adds in one register, and where a window's
// paths merge it then copies the sums to where the other paths left theirs)
__device__ __forceinline__ float fma_to(float a, float b, float c) {
    float d;
    asm("v_fma_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// The value of the first active lane (for values every lane holds alike,
// e.g. read from one LDS address: the compiler then keeps them in scalar
// registers and branches on them without masks).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Inclusive max-scan over the wave of a non-negative int: DPP row shifts
// within rows of 16, then the row broadcasts. Lanes without a source read 0
// (bound control), which a max ignores; so does a row that also takes a
// partial prefix (row_bcast:15 into row 2 brings row 1's maximum, which the
// next level's full prefix covers), so every step runs on all rows.
__device__ __forceinline__ int scan_max(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));  // row_shr:1
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));  // row_shr:2
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));  // row_shr:4
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));  // row_shr:8
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xf, 0xf, true));  // row_bcast:15
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xf, 0xf, true));  // row_bcast:31
    return x;
}

// The G = 64 >> LOG_WW slots' partial sums of a slice, added by a fixed tree
// over the slot bits of the lane id (as SlotSum: halving permlane32/16 swaps
// at bits 5 and 4 when a lane holds two or more elements, then the partner's
// value added by DPP within rows of 16; bound control set on DPP steps whose
// every lane has a source, so the moves fold into the adds). Afterwards lane
// L holds Sum::VO elements from element Sum::base(L), and Sum::writer(L)
// lanes hold every element once.
template <int LOG_WW, int VEC>
__device__ __forceinline__ void slot_sum(const float (&acc)[VEC], float (&res)[SlotSum<LOG_WW, VEC>::VO]) {
    using Sum = SlotSum<LOG_WW, VEC>;
    constexpr int V5 = Sum::V5, VO = Sum::VO;
    auto dpp_add = [](float v, auto ctrl_c) {
        constexpr int C = decltype(ctrl_c)::value;
        return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), C, 0xf, 0xf, true));
    };
    float a5[V5];
    if constexpr (Sum::H5) {
#pragma unroll
        for (int e = 0; e < V5; ++e) {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]),
                                                            __float_as_uint(acc[e + V5]), false, false);
            a5[e] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < V5; ++e) a5[e] = LOG_WW <= 5 ? level_f(acc[e], 5) : acc[e];
    }
    if constexpr (Sum::H4) {
#pragma unroll
        for (int e = 0; e < VO; ++e) {
            const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a5[e]),
                                                            __float_as_uint(a5[e + VO]), false, false);
            res[e] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < VO; ++e) res[e] = LOG_WW <= 4 ? level_f(a5[e], 4) : a5[e];
    }
    // rotations within a row pair lanes like xor once the higher in-row bits
    // are summed (their partials are equal)
#pragma unroll
    for (int e = 0; e < VO; ++e) {
        if constexpr (LOG_WW <= 3) res[e] = dpp_add(res[e], std::integral_constant<int, 0x128>{});  // row_ror:8
        if constexpr (LOG_WW <= 2) res[e] = dpp_add(res[e], std::integral_constant<int, 0x124>{});  // row_ror:4
        if constexpr (LOG_WW <= 1) res[e] = dpp_add(res[e], std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
        if constexpr (LOG_WW <= 0) res[e] = dpp_add(res[e], std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    }
}

// A wave's place in its run: the slice being summed (i), where it ends (e1,
// or a position past every entry once the run's slices are done) and the
// run's last slice (exclusive).
struct SegCursor {
    int i, e1, s_end;
};

template <int LOG_WW, bool LDS_B, int VEC>
__global__ void __launch_bounds__(1024)
k_vcs_seg(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
          const float *__restrict__ vals, const int *__restrict__ idx,
          const float *__restrict__ B, float *__restrict__ out, int w, int n_in, int tiles,
          int n_b_rows, const int *__restrict__ he, const SegDesc *__restrict__ desc) {
    using T = float;
    using Sum = SlotSum<LOG_WW, VEC>;
    constexpr int WW = 1 << LOG_WW;
    constexpr int G = 64 >> LOG_WW;
    constexpr int NSTEP = WW;  // steps per window
    constexpr int SBV = NSTEP < (VEC >= 4 ? 4 : 8) ? NSTEP : (VEC >= 4 ? 4 : 8);
    constexpr int NSB = NSTEP / SBV;  // stages of SBV steps per window
    constexpr int NWR = kRowsNWR;
    constexpr int GWR = kRowsGWR;
    constexpr int kFar = 0x7fffffff;
    static_assert(64 * NWR + 256 * GWR == kRowsWaveLds, "per-wave LDS layout");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int slot = lane >> LOG_WW;
    const int cl = lane & (WW - 1);
    const int chunk_w = VEC << LOG_WW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t b_bytes = LDS_B ? (((size_t)n_in * w * sizeof(T) + 15) & ~size_t(15)) : 0;
    unsigned char *mark = smem + b_bytes + (size_t)wave * kRowsWaveLds;
    T *gvt = reinterpret_cast<T *>(mark + 64 * NWR);
    int bb, be, tile;
    seg_block_range(blockIdx.x, gridDim.x, tiles, n_slices, bb, be, tile);
    B += (size_t)tile * n_in * w;  // this tile's rows of B
    const int b_rows = min(n_in, n_b_rows - tile * n_in);
    const uint32_t w4 = (uint32_t)w * 4u;
    // LDS address of the staged B (the start of the dynamic LDS)
    const uint32_t b_lds0 =
        LDS_B ? (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem : 0u;

    const size_t b_el = (size_t)b_rows * w;
    const bool b_dma = LDS_B && (b_el * sizeof(T)) % 16 == 0 && ((uintptr_t)B % 16) == 0;
    // this wave's run, planned ahead (k_seg_plan); its first round's loads go
    // out before B's copies, which would otherwise delay the plan's own load
    // and so the whole chain
    const SegDesc d = desc[blockIdx.x * waves + wave];
    const int s_a = d.s_a, s_b = d.s_b, E_a = d.E_a, E_b = d.E_b, K_b = d.K_b;
    // lane L = q WW + t holds entry G t + q of a window; it reads its group
    // number from lane G t + q of the window's max-scan
    const int perm = G * cl + slot;
    const int perm4 = perm * 4;

    // the group holding entry E (at or after K): groups before it end at or
    // before E
    auto seek = [&](int K, int E) {
        for (;;) {
            const int k = K + 1 + lane;
            const int n = __popcll(__ballot(k < K_b && vptr[min(k, K_b)] <= E));
            K += n;
            if (n < 64) return K;
        }
    };
    // round state: entries [E, ...) with groups from K; windows W and group
    // starts/values GS, GV (group K + 64 j + lane), loaded a round ahead.
    // The loads go through raw buffers based at the round's first entry and
    // group: a load past a buffer's end (past the run) returns 0 and reads no
    // memory, so no lane clamps its address, and the offsets of the windows
    // and group rows are immediates. An index read as 0 gathers row 0 of B,
    // which no slice adds; group starts past the run are set at the round's
    // start (fix_starts).
    auto buf = [](const void *p, int n) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 4 * n, 0x00020000);
    };
    auto load_round = [&](int E0, int K0, int (&Wd)[NWR], int (&GSd)[GWR], T (&GVd)[GWR]) {
        const auto ri = buf(idx + E0, min(E_b - E0, 64 * NWR));
#pragma unroll
        for (int k = 0; k < NWR; ++k) Wd[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, perm4 + 256 * k, 0, 0);
        const auto rg = buf(vptr + K0, min(K_b - K0 + 1, 64 * GWR));
        const auto rv = buf(vals + K0, min(K_b - K0, 64 * GWR));
#pragma unroll
        for (int j = 0; j < GWR; ++j) {
            GSd[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rg, 4 * lane + 256 * j, 0, 0);
            GVd[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, 4 * lane + 256 * j, 0, 0));
        }
    };
    // group starts past the run's last group (read as 0) lie past every entry
    auto fix_starts = [&](int K0, int (&GSd)[GWR]) {
#pragma unroll
        for (int j = 0; j < GWR; ++j) GSd[j] = K0 + 64 * j + lane <= K_b ? GSd[j] : kFar;
    };
    int E = E_a, K = d.K_a;
    int W[NWR], GS[GWR];
    T GV[GWR];
    // ends of slices: lane j of RE holds the end of slice row0 + j, loaded
    // with the round's other data (a round never closes a slice past lane 63;
    // nothing is reloaded inside a round, so no load is pending across the
    // window walk's branches)
    int RE = 0, row0 = s_a;
    auto load_ends = [&]() { RE = he[min(s_a + 1 + lane, s_b)]; };
    if (E_a < E_b) {
        load_round(E, K, W, GS, GV);
        load_ends();
    }
    // B into LDS as direct global->LDS copies (16 bytes per lane, 1 KB per
    // wave instruction; no registers)
    if constexpr (LDS_B) {
        if (b_dma) {
            const int nq = (int)(b_el * sizeof(T) / 16);
            const uint4 *src = reinterpret_cast<const uint4 *>(B);
            for (int c = wave; c * 64 < nq; c += waves) {
                if (c * 64 + lane < nq)
                    __builtin_amdgcn_global_load_lds(
                        src + c * 64 + lane,
                        (__attribute__((address_space(3))) void *)(smem + (size_t)c * 1024), 16, 0, 0);
            }
        }
    }
    const char *Bb = reinterpret_cast<const char *>(B);
    if constexpr (LDS_B) {
        T *lb = reinterpret_cast<T *>(smem);
        if (!b_dma) {
            for (size_t k = threadIdx.x; k < b_el; k += blockDim.x) lb[k] = B[k];
        }
        Bb = reinterpret_cast<const char *>(lb);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies and loads
    __syncthreads();                     // and every other wave's copies
    if (s_a >= s_b) return;

    for (int c0 = 0; c0 < w; c0 += chunk_w) {
        const int col = c0 + cl * VEC;
        const bool act = col < w;
        // byte offset of the lane's elements in a row (gathers stay inside B's
        // rows), plus, for B in LDS, the LDS address where B starts
        const uint32_t coff4 = (act ? 4u * col : 0u) + b_lds0;
        if (c0 > 0) {  // a later width pass walks the run again
            // (the run's start is hidden from the compiler here, so the first
            // round's addresses are not kept live across the whole pass for
            // this reload)
            int ea = E_a, ka = d.K_a;
            asm volatile("" : "+s"(ea), "+s"(ka));
            E = ea;
            K = ka;
            if (ea < E_b) {
                load_round(E, K, W, GS, GV);
                load_ends();
            }
        }
        row0 = s_a;
        SegCursor cur{s_a, E_a < E_b ? readlane(RE, 0) : E_a, s_b};
        T acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = T(0);

        // issue priority by progress through the run, checked every other
        // window: one less each time the wave passes a quarter of its entries
        const int quarter = (E_b - E_a) >> 2;
        int p_next = E_a + quarter, p_lev = 3;
        __builtin_amdgcn_s_setprio(3);
        auto pace = [&](int at) {
            if (at >= p_next) {
                --p_lev;
                p_next = p_lev > 0 ? p_next + quarter : kFar;
                if (p_lev == 2) __builtin_amdgcn_s_setprio(2);
                else if (p_lev == 1) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
        };

        // the end of slice i: lane i - row0 of RE, or past every entry when RE
        // does not hold it (no branch: the lane is read modulo 64, then the
        // result selected on i < s_end and i - row0 < 64 as one sign test)
        auto end_at = [&](int i) {
            const int j = i - row0;
            const int r = readlane(RE, j & 63);
            return ((i - cur.s_end) & (j - 64)) < 0 ? r : kFar;
        };
        // sums slice cur.i over the slots, writes its row, moves on (close
        // leaves cur.e1 as it was; close_track looks up the next end)
        auto close = [&]() {
            T res[Sum::VO];
            slot_sum<LOG_WW, VEC>(acc, res);
            if (Sum::writer(lane) && act) {
                T *o = out + (size_t)cur.i * w + col + Sum::base(lane);
                store_vec<T, Sum::VO>(o, res);
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = T(0);
            ++cur.i;
        };
        auto close_track = [&]() {
            close();
            cur.e1 = end_at(cur.i);
        };
        // closes slice cur.i and starts the next one with v * b in the lanes
        // that `keep` (zero elsewhere; the sum's tree and the next slice's
        // products are independent, so they overlap)
        auto close_into = [&](const T (&b)[VEC], T v, bool keep) {
            T res[Sum::VO];
            slot_sum<LOG_WW, VEC>(acc, res);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = keep ? fma_t(v, b[e], T(0)) : T(0);
            if (Sum::writer(lane) && act) {
                T *o = out + (size_t)cur.i * w + col + Sum::base(lane);
                store_vec<T, Sum::VO>(o, res);
            }
            ++cur.i;
        };

        while (E < E_b) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this round's loads
            fix_starts(K, GS);
            // the current slice is the first one RE holds (row0): its end
            // (a round that closed all 64 slices it held left kFar in e1)
            cur.e1 = cur.i < cur.s_end ? readlane(RE, 0) : kFar;
            // the round ends at the run's end, after NWR windows, or where the
            // groups held in GS end (group K + 64 GWR - 1 starts there)
            int gs_last = readlane(GS[GWR - 1], 63);
            if (gs_last <= E) {
                // every held group starts at or before E (a run of empty
                // groups at E): move K past them and load the groups again
                K = seek(K, E);
#pragma unroll
                for (int j = 0; j < GWR; ++j) {
                    GS[j] = vptr[min(K + 64 * j + lane, K_b)];
                    GV[j] = vals[max(min(K + 64 * j + lane, K_b - 1), 0)];
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);
                gs_last = readlane(GS[GWR - 1], 63);
            }
            // 64 or more empty slices at E (every slice RE holds ends at or
            // before E): close them and load the ends from the next slice
            while (readlane(RE, 63) <= E && cur.i < cur.s_end) {
                while (cur.e1 <= E) close_track();
                row0 = cur.i;
                RE = he[min(row0 + 1 + lane, s_b)];
                __builtin_amdgcn_s_waitcnt(0x0F70);
                cur.e1 = cur.i < cur.s_end ? readlane(RE, 0) : kFar;
            }
            // ... nor past the end of the last slice RE holds
            const int rend = min(min(min(E_b, E + 64 * NWR), gs_last), readlane(RE, 63));
            int n_le = 0;
#pragma unroll
            for (int j = 0; j < GWR; ++j) n_le += __popcll(__ballot(GS[j] <= rend));
            const int K_next = K + n_le - 1;  // the group holding entry rend
            // the slices this round closes (every one ending at or before
            // rend), so the next round's first slice
            const int row0_next = row0 + (int)__popcll(__ballot(RE <= rend));
            int W2[NWR], GS2[GWR], RE2 = 0;
            T GV2[GWR];
            const bool more = rend < E_b;
            if (more) {
                load_round(rend, K_next, W2, GS2, GV2);
                RE2 = he[min(row0_next + 1 + lane, s_b)];
            }
            write_marks<NWR, GWR>(GS, GV, min(K_b - K, 64 * GWR - 1), E, rend, true, lane, mark,
                                  gvt);

            const int nwin = (rend - E + 63) >> 6;
            // where the slices closing in this round end: lane j of wv holds
            // the window of slice row0 + j's last entry (NWR when the slice
            // does not close in this round, or ends at or before E: an empty
            // slice at the round's start). Bit k of `whole` says that window
            // k lies inside the round and no slice ends in it at or before
            // its start (only window 0 can hold such an end).
            const bool closes = lane < cur.s_end - row0 && RE <= rend;
            const int wv = closes && RE > E ? (RE - 1 - E) >> 6 : NWR;
            const int nfull = (rend - E) >> 6;
            int whole = nfull >= NWR ? (1 << NWR) - 1 : (1 << nfull) - 1;
            if (__ballot(closes && RE <= E) != 0) whole &= ~1;
            // the value of every window's entries, for the whole round at
            // once (independent chains): each window's group numbers by a
            // max-scan of its marks, raised to the last number of the windows
            // before it, then the lane's own (permuted) entry's number and
            // its value
            // (every window of the round's mark row is scanned, also past
            // its end: marks there are zero and the numbers stay valid, and
            // with no branches the reads and scans overlap)
            T V[NWR];
            {
                int gs[NWR];
                static_for<NWR>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    gs[k] = (int)mark[64 * k + lane];
                });
                static_for<NWR>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    gs[k] = scan_max(gs[k]);
                });
                int carry = 0;
                static_for<NWR>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    const int g = max(gs[k], carry);
                    carry = max(carry, readlane(gs[k], 63));
                    const int gp = G == 64 ? g : __builtin_amdgcn_ds_bpermute(perm4, g);
                    V[k] = gvt[gp - 1];
                });
            }
            // windows are software-pipelined: the gathers of window k + 1
            // go out before window k's are consumed
            static_assert(NSB == 1, "a window's steps form one stage");
            T bvs[2][NSTEP][VEC];
            auto issue = [&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                const uint32_t a = __umul24((uint32_t)W[k], w4);  // row offset of each entry
                static_for<NSTEP>([&](auto t_c) {
                    constexpr int TT = decltype(t_c)::value;
                    gather<LDS_B, VEC>(Bb, (uint32_t)group_bcast<LOG_WW, TT>((int)a) + coff4,
                                       bvs[k & 1][TT]);
                });
            };
            issue(std::integral_constant<int, 0>{});
            static_for<NWR>([&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                if (k >= nwin) return;
                if constexpr (k + 1 < NWR) issue(std::integral_constant<int, k + 1>{});
                const int wbase = E + 64 * k;
                if constexpr ((k & 1) == 0) pace(wbase);
                // (the cursor is the same in every lane; saying so keeps the
                // branches below scalar)
                cur.i = uni(cur.i);
                const T v = V[k];
                auto full = [&](const T(&b)[VEC], T vt) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = fma_t(vt, b[e], acc[e]);
                };
                // the slices (lanes of RE) whose last entry is in this window
                const uint64_t em = (whole >> k) & 1 ? __ballot(wv == k) : ~0ull;
                if (em == 0) {
                    // every step inside the current slice and round (the
                    // last one into fresh registers)
                    static_for<NSTEP>([&](auto t_c) {
                        constexpr int TT = decltype(t_c)::value;
                        const T vt = group_bcast<LOG_WW, TT>(v);
                        if constexpr (TT + 1 < NSTEP) {
                            full(bvs[k & 1][TT], vt);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) acc[e] = fma_to(vt, bvs[k & 1][TT][e], acc[e]);
                        }
                    });
                    return;
                }
                if ((em & (em - 1)) == 0) {
                    // exactly one slice (cur.i) ends in the window, after
                    // entry b - 1: the step holding that entry adds its first
                    // qb slots, closes the slice, then adds the rest; every
                    // other step adds all its slots
                    const int b = readlane(RE, (int)__builtin_ctzll(em)) - wbase;  // 1 .. 64
                    const int tb = (int)((unsigned)(b - 1) >> (6 - LOG_WW)), qb = b - G * tb;
                    // the step holding the end: slots below qb add their
                    // entry to the closing slice, the others start the next
                    // one (selects instead of masked lanes: a lane holding
                    // the other slice's entry keeps its sum as is, so a
                    // non-finite B element or value never reaches a slice
                    // it is not stored in; qb = G needs no case of its own)
                    auto split = [&](const T(&bv)[VEC], T vt) {
                        const bool mine = slot < qb;
                        if (mine) {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) acc[e] = fma_t(vt, bv[e], acc[e]);
                        }
                        close_into(bv, vt, !mine);
                    };
                    // one straight run of steps per split step (few steps
                    // per window: no merges between the steps)
                    auto run = [&](auto tb_c) {
                        constexpr int TB = decltype(tb_c)::value;
                        static_for<NSTEP>([&](auto t_c) {
                            constexpr int TT = decltype(t_c)::value;
                            if constexpr (TT == TB) split(bvs[k & 1][TT], group_bcast<LOG_WW, TT>(v));
                            else full(bvs[k & 1][TT], group_bcast<LOG_WW, TT>(v));
                        });
                    };
                    if constexpr (NSTEP <= 8) {
                        bool done = false;
                        static_for<NSTEP>([&](auto tb_c) {
                            constexpr int TB = decltype(tb_c)::value;
                            if (!done && (TB + 1 == NSTEP || tb == TB)) {
                                run(tb_c);
                                done = true;
                            }
                        });
                    } else {
                        static_for<NSTEP>([&](auto t_c) {
                            constexpr int TT = decltype(t_c)::value;
                            if (TT != tb) full(bvs[k & 1][TT], group_bcast<LOG_WW, TT>(v));
                            else split(bvs[k & 1][TT], group_bcast<LOG_WW, TT>(v));
                        });
                    }
                    return;
                }
                // several slice ends, empty slices, or the round's end: step
                // by step
                cur.e1 = end_at(cur.i);
                static_for<NSTEP>([&](auto t_c) {
                    constexpr int TT = decltype(t_c)::value;
                    const T (&b)[VEC] = bvs[k & 1][TT];
                    const T vt = group_bcast<LOG_WW, TT>(v);
                    // step [s, s + G): slot q holds entry s + q; slices
                    // ending in it close there
                    const int s = wbase + TT * G;
                    const int stop = min(rend, s + G);
                    if (s >= stop) return;  // past the round's end
                    auto add = [&](int lo, int hi) {  // slots holding entries [lo, hi)
                        if (hi > lo) {
                            const bool in = slot >= lo - s && slot < hi - s;
#pragma unroll
                            for (int e = 0; e < VEC; ++e) acc[e] = in ? fma_t(vt, b[e], acc[e]) : acc[e];
                        }
                    };
                    int lo = s;
                    while (cur.e1 <= stop) {
                        add(lo, cur.e1);
                        lo = max(lo, cur.e1);
                        close_track();
                    }
                    add(lo, stop);
                });
            });
            E = rend;
            K = K_next;
            if (!more) break;
            RE = RE2;
            row0 = row0_next;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < NWR; ++k) W[k] = W2[k];
#pragma unroll
            for (int j = 0; j < GWR; ++j) {
                GS[j] = GS2[j];
                GV[j] = GV2[j];
            }
        }
        // slices ending at the run's last entry, and empty ones after
        while (cur.i < cur.s_end) close();
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace vspmm
