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

// Lane geometry of the VCS walks: G entry lanes per step, NSTEP steps per
// 64-entry window, taken in stages of SBV steps whose gathers are in flight
// together (NSB stages per window).
template <int LOG_WW, int VEC>
struct Geo {
    static constexpr int G = 64 >> LOG_WW;
    static constexpr int NSTEP = 64 / G;
    static constexpr int SBV = NSTEP < (VEC >= 4 ? 4 : 8) ? NSTEP : (VEC >= 4 ? 4 : 8);
    static constexpr int NSB = NSTEP / SBV;
};

// The gathered operands of one stage: the entry values and B's row pieces.
template <int SBV, int VEC>
struct Stage {
    float vj[SBV];
    float bv[SBV][VEC];
};

// The window walk shared by both VCS walks. Positions base + 64k + lane of
// windows k < nwin hold W[k] (indices); `mark` holds the round's group-start
// bytes at the same offsets and `gvt` the group values. Stages run as a
// two-deep pipeline: the next stage's gathers are issued before the current
// stage is consumed, so their latency overlaps the current stage's work.
// consume(k, j0, stage) does the arithmetic of stage (k, j0). Returns the
// group number (round-relative plus one) of the last window's last lane.
// B rows are read at byte offset ix * w4 + coff4 from Bb (32-bit offsets:
// every row index is below 2^24 and B is under 4 GiB).
template <int LOG_WW, int VEC, int NWR, bool ROTATE, typename Consume>
__device__ __forceinline__ int window_stream(const int (&W)[NWR], int nwin, int lane, int slot,
                                              const unsigned char *mark, const float *gvt,
                                              const char *Bb, uint32_t w4, uint32_t coff4,
                                              Consume &&consume) {
    using Gm = Geo<LOG_WW, VEC>;
    using St = Stage<Gm::SBV, VEC>;
    const int ns = nwin * Gm::NSB;
    int carry = 0;  // group number reaching the next window's start
    int wi = 0;     // the current window's indices
    float vk = 0;   // and values
    // ROTATE: the windows still to come move down one register per window
    // (short arrays are otherwise indexed through a select chain per window)
    int Wq[ROTATE ? NWR : 1];
    if constexpr (ROTATE) {
#pragma unroll
        for (int k = 0; k < NWR; ++k) Wq[k] = W[k];
    }
    auto issue = [&](int q, St &st) {
        const int k = q / Gm::NSB;
        const int j0 = (q - k * Gm::NSB) * Gm::SBV;
        if (j0 == 0) {
            if constexpr (ROTATE) {
                wi = Wq[0];
#pragma unroll
                for (int m = 0; m + 1 < NWR; ++m) Wq[m] = Wq[m + 1];
            } else {
                wi = W[k];
            }
            const int g = max(wave_max_scan((int)mark[64 * k + lane]), carry);
            carry = readlane(g, 63);
            vk = gvt[g - 1];
        }
#pragma unroll
        for (int t = 0; t < Gm::SBV; ++t) {
            // with 64 entry lanes a lane's entry is its own (no shuffle)
            const int src = (j0 + t) * Gm::G + slot;
            const int ix = Gm::G == 64 ? wi : __shfl(wi, src);
            st.vj[t] = Gm::G == 64 ? vk : __shfl(vk, src);
            const uint32_t off = __umul24((uint32_t)ix, w4) + coff4;
            load_vec<float, VEC>(reinterpret_cast<const float *>(Bb + off), st.bv[t]);
        }
    };
    auto eat = [&](int q, const St &st) {
        const int k = q / Gm::NSB;
        consume(k, (q - k * Gm::NSB) * Gm::SBV, st);
    };
    if (ns <= 0) return carry;
    St a, b;
    issue(0, a);
    for (int q = 0;;) {
        if (q + 1 < ns) issue(q + 1, b);
        eat(q, a);
        if (++q >= ns) break;
        if (q + 1 < ns) issue(q + 1, a);
        eat(q, b);
        if (++q >= ns) break;
    }
    return carry;
}

// Writes the round's (or pass's) group marks and value table: group numbers
// are round-relative plus one. Non-empty groups starting in [base, pe) mark
// their first position (relative to base); with mark_first, group 0 holds
// position base (it may start before it) and marks position 0.
template <int NWR, int GWR>
__device__ __forceinline__ void write_marks(const int (&GS)[GWR], const float (&GV)[GWR],
                                            int n_grp, int base, int pe, bool mark_first,
                                            int lane, unsigned char *mark, float *gvt) {
    static_assert(NWR == 8 || NWR == 16, "a mark row of 512 or 1024 bytes");
    if constexpr (NWR == 16) reinterpret_cast<uint4 *>(mark)[lane] = make_uint4(0, 0, 0, 0);
    else reinterpret_cast<uint2 *>(mark)[lane] = make_uint2(0, 0);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < GWR; ++j) {
        gvt[64 * j + lane] = GV[j];
        int nxt = __shfl_down(GS[j], 1);
        if (j + 1 < GWR) {
            const int first_next = readlane(GS[j + 1 < GWR ? j + 1 : j], 0);
            nxt = lane == 63 ? first_next : nxt;
        }
        const int li = 64 * j + lane;
        // group 0 may start before base; an empty group 0 (base at its
        // slice's end) holds nothing, and the group starting at base marks it
        if (mark_first && li == 0) {
            if (nxt > GS[j]) mark[0] = 1;
        } else if (li < n_grp && nxt > GS[j] && GS[j] < pe) {
            mark[GS[j] - base] = (unsigned char)(li + 1);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Accumulates entries [P0, P1) of one VCS slice, whose groups are [ka, kb),
// into acc: entry lane `slot` takes positions P0 + 64k + jG + slot in order.
// The entries are walked in passes of up to 64 * kPieceNWR positions and
// 64 * kPieceGWR - 1 groups with per-wave LDS marks and a value table. The
// group holding a pass's first position is found 64 group starts at a time
// with a ballot. Indices are read non-temporally so the stream does not push
// B's rows out of L2.
template <int LOG_WW, int VEC>
__device__ __forceinline__ void vcs_piece(int ka, int kb, int P0, int P1, int lane, int slot,
                                          uint32_t coff4, const int *__restrict__ vptr,
                                          const float *__restrict__ vals,
                                          const int *__restrict__ idx, const char *Bb,
                                          uint32_t w4, unsigned char *mark, float *gvt,
                                          float (&acc)[VEC]) {
    using Gm = Geo<LOG_WW, VEC>;
    constexpr int NWR = kPieceNWR;
    constexpr int GWR = kPieceGWR;
    int kf = ka;  // the group holding position P0
    while (P0 < P1) {
        // the pass's indices do not depend on its groups: issue them first
        int PE = min(P1, P0 + 64 * NWR);
        int W[NWR], GS[GWR];
        float GV[GWR];
#pragma unroll
        for (int k = 0; k < NWR; ++k) {
            if (P0 + 64 * k < PE) W[k] = __builtin_nontemporal_load(idx + min(P0 + 64 * k + lane, PE - 1));
        }
        for (;;) {  // count the groups after kf that start at or before P0
            const int k = kf + 1 + lane;
            const int gs = vptr[min(k, kb)];
            const int n = __popcll(__ballot(k < kb && gs <= P0));
            kf += n;
            if (n < 64) break;
        }
        // at most 64 * GWR - 1 groups per pass (the windows loaded past PE are not used)
        if (kb - kf > 64 * GWR - 1) PE = min(PE, vptr[kf + 64 * GWR - 1]);
#pragma unroll
        for (int j = 0; j < GWR; ++j) {
            GS[j] = vptr[min(kf + 64 * j + lane, kb)];
            GV[j] = vals[min(kf + 64 * j + lane, kb - 1)];
        }
        write_marks<NWR, GWR>(GS, GV, min(kb - kf, 64 * GWR - 1), P0, PE, true, lane, mark, gvt);
        const int nwin = (PE - P0 + 63) >> 6;
        const int last_g = window_stream<LOG_WW, VEC, NWR, false>(
            W, nwin, lane, slot, mark, gvt, Bb, w4, coff4,
            [&](int k, int j0, const Stage<Gm::SBV, VEC> &st) {
                const int step0 = P0 + 64 * k + j0 * Gm::G;
                if (step0 + Gm::SBV * Gm::G <= PE) {
#pragma unroll
                    for (int t = 0; t < Gm::SBV; ++t) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) acc[e] = fma_t(st.vj[t], st.bv[t][e], acc[e]);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < Gm::SBV; ++t) {
                        if (step0 + t * Gm::G + slot < PE) {
#pragma unroll
                            for (int e = 0; e < VEC; ++e)
                                acc[e] = fma_t(st.vj[t], st.bv[t][e], acc[e]);
                        }
                    }
                }
            });
        kf += last_g - 1;  // the group of the pass's last position
        P0 = PE;
        __builtin_amdgcn_wave_barrier();
    }
}

// Where a wave's walk stands: the next slice, and (mid) whether the walk is
// inside that slice at entry p, whose group is at or after kf.
struct RowCursor {
    int sa, p, kf;
    bool mid;
};

// A round of k_vcs_rows: entries [E0, E1) and groups [K0, K1). nsl slices end
// inside it; with open_end the slice after them continues past E1 (a slice
// too large for one round is walked as a run of such rounds, its sum carried
// over). With mid, the round starts inside slice sa at E0, and group K0 holds
// E0. hp / he: lanes hold the first group / first entry of slice sa + lane
// (lanes below nhl hold headers).
struct RowRound {
    int sa, nsl, E0, E1, K0, K1, hp, he, nhl;
    bool open_end, mid;
};

// Loads the headers of slices sa .. sa + 63 into the lanes.
__device__ __forceinline__ void rows_headers(RowRound &r, int sa, int n_slices, int lane,
                                             const int *__restrict__ sptr,
                                             const int *__restrict__ vptr) {
    r.hp = sptr[min(sa + lane, n_slices)];
    r.he = vptr[r.hp];
    r.nhl = 64;
}

// The same from the block's header table in LDS (slice bb + t in entry t,
// entries up to be - bb).
__device__ __forceinline__ void rows_headers_lds(RowRound &r, int sa, int bb, int be, int lane,
                                                 const int *hp_l, const int *he_l) {
    const int t = min(sa - bb + lane, be - bb);
    r.hp = hp_l[t];
    r.he = he_l[t];
    r.nhl = 64;
}

// Plans the round that starts at cursor c from the headers in r (slice c.sa in
// lane 0): the longest run of whole slices that fits (at least one), or, when
// the first slice alone does not fit, the part of it that does.
template <int NWR, int GWR>
__device__ __forceinline__ void rows_fit(RowRound &r, const RowCursor &c, int s_end, int lane,
                                         const int *__restrict__ vptr) {
    r.sa = c.sa;
    r.mid = c.mid;
    // the last group of slice sa starting at or before P0 (past empty groups)
    auto seek = [&](int K0, int P0) {
        const int kb = readlane(r.hp, 1);
        for (;;) {
            const int k = K0 + 1 + lane;
            const int n = __popcll(__ballot(k < kb && vptr[min(k, kb)] <= P0));
            K0 += n;
            if (n < 64) return K0;
        }
    };
    int P0, K0;
    if (c.mid) {
        P0 = c.p;
        K0 = seek(c.kf, P0);
    } else {
        P0 = readlane(r.he, 0);
        K0 = readlane(r.hp, 0);
    }
    const bool fits = lane < r.nhl && (c.sa + lane <= s_end) && (r.he - P0 <= 64 * NWR) &&
                      (r.hp - K0 <= 64 * GWR - 1);
    const int last = __popcll(__ballot(fits)) - 1;  // fits is a prefix; lane 0 always fits
    r.E0 = P0;
    r.K0 = K0;
    if (last >= 1) {
        r.nsl = last;
        r.open_end = false;
        r.E1 = readlane(r.he, last);
        r.K1 = readlane(r.hp, last);
    } else {  // the next slice alone does not fit: take the part that does
        if (!c.mid) r.K0 = K0 = seek(K0, P0);  // so that group K0 + 64 GWR - 1 starts after P0
        r.nsl = 0;
        r.open_end = true;
        const int kb = readlane(r.hp, 1);
        int e1 = min(readlane(r.he, 1), P0 + 64 * NWR);
        if (kb - K0 > 64 * GWR - 1) e1 = min(e1, vptr[K0 + 64 * GWR - 1]);
        r.E1 = e1;
        r.K1 = min(kb, K0 + 64 * GWR - 1);
        if (e1 == readlane(r.he, 1)) {  // the rest of the slice fits after all
            r.nsl = 1;                   // (groups past K1 are empty)
            r.open_end = false;
        }
    }
}

// Loads a round's entry windows W[k] = idx[E0 + 64k + lane] and group windows
// GS[j] = vptr[K0 + 64j + lane], GV[j] = values[K0 + 64j + lane], every one
// of them (clamped to the round), so the number of loads in flight is fixed.
template <int NWR, int GWR>
__device__ __forceinline__ void rows_load(const RowRound &r, int (&W)[NWR], int (&GS)[GWR],
                                          float (&GV)[GWR], int lane,
                                          const int *__restrict__ vptr,
                                          const float *__restrict__ vals,
                                          const int *__restrict__ idx) {
#pragma unroll
    for (int k = 0; k < NWR; ++k) W[k] = idx[max(min(r.E0 + 64 * k + lane, r.E1 - 1), 0)];
#pragma unroll
    for (int j = 0; j < GWR; ++j) {
        GS[j] = vptr[min(r.K0 + 64 * j + lane, r.K1)];
        GV[j] = vals[max(min(r.K0 + 64 * j + lane, r.K1 - 1), 0)];
    }
}

// Short VCS slices. A block (one per CU with LDS_B) takes a contiguous range
// of slices, cut into chunks of kRowsChunk slices; a (width pass, chunk) pair
// is a unit of work. Each wave starts with unit `wave` and then claims the
// next free unit from a counter in LDS, so waves that the CU serves faster
// take more units. A unit is walked in rounds of up to 64 * kRowsNWR entries
// and 64 * kRowsGWR - 1 groups that start at the chunk's first slice (a
// longer slice takes several rounds), so a slice's arithmetic does not depend
// on which wave walks it. Two rounds are held in registers: while one is
// walked, the next one's windows are in flight, planned from the block's
// slice headers in LDS. With LDS_B the dense operand B (n_in x w) is copied
// into the CU's LDS first and gathered from there. Dynamic LDS: [B, 16-byte
// aligned][per wave: kRowsWaveLds bytes of marks and group values][header
// table: 2 x hcap ints][unit counter].
//
// Tiled (tiles > 1): the slices are `tiles` runs of n_slices / tiles, run t
// reading B's rows [t * n_in, t * n_in + n_in) (n_in rows per tile, the last
// tile cut at n_b_rows) with tile-local indices. The grid is tiles x bpt
// blocks, each taking one of the bpt parts of one run and staging its tile;
// with a multiple of 8 tiles the blocks of a tile share an XCD.
template <int LOG_WW, bool LDS_B, int VEC>
__global__ void __launch_bounds__(1024)
k_vcs_rows(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
           const float *__restrict__ vals, const int *__restrict__ idx,
           const float *__restrict__ B, float *__restrict__ out, int w, int n_in, int tiles,
           int n_b_rows) {
    using T = float;
    using Sum = SlotSum<LOG_WW, VEC>;
    using Gm = Geo<LOG_WW, VEC>;
    constexpr int NWR = kRowsNWR;
    constexpr int GWR = kRowsGWR;
    constexpr int CH = kRowsChunk;
    static_assert(64 * NWR + 256 * GWR == kRowsWaveLds, "per-wave LDS layout");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int slot = lane >> LOG_WW;
    const int cl = lane & ((1 << LOG_WW) - 1);
    const int chunk_w = VEC << LOG_WW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t b_bytes = LDS_B ? (((size_t)n_in * w * sizeof(T) + 15) & ~size_t(15)) : 0;
    unsigned char *mark = smem + b_bytes + (size_t)wave * kRowsWaveLds;
    T *gvt = reinterpret_cast<T *>(mark + 64 * NWR);
    const int hcap = rows_header_cap(n_slices, gridDim.x);
    int *hp_l = reinterpret_cast<int *>(smem + b_bytes + (size_t)waves * kRowsWaveLds);
    int *he_l = hp_l + hcap;
    int *unit_ctr = he_l + hcap;
    const int bpt = gridDim.x / tiles;  // blocks per tile
    int tile = blockIdx.x / bpt, part = blockIdx.x - tile * bpt;
    if (tiles % 8 == 0) {
        // blocks go to the 8 XCDs round robin (block b to XCD b % 8): give
        // each XCD whole tiles, so a tile of B is fetched into one L2 only
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        tile = x * (tiles >> 3) + j / bpt;
        part = j - (j / bpt) * bpt;
    }
    const int n_run = n_slices / tiles;  // slices per tile
    const int bb = tile * n_run + (int)((long long)part * n_run / bpt);
    const int be = tile * n_run + (int)((long long)(part + 1) * n_run / bpt);
    B += (size_t)tile * n_in * w;  // this tile's rows of B
    const int b_rows = min(n_in, n_b_rows - tile * n_in);
    const int nch = (be - bb + CH - 1) / CH;
    const int npass = (w + chunk_w - 1) / chunk_w;
    const int nunits = nch * npass;
    const uint32_t w4 = (uint32_t)w * 4u;

    // B into LDS first, as direct global->LDS copies (16 bytes per lane, 1 KB
    // per wave instruction; no registers).
    const size_t b_el = (size_t)b_rows * w;
    const bool b_dma = LDS_B && (b_el * sizeof(T)) % 16 == 0 && ((uintptr_t)B % 16) == 0;
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
    // the block's slice headers into LDS
    for (int t = threadIdx.x; t <= be - bb; t += blockDim.x) {
        const int hp = sptr[bb + t];
        hp_l[t] = hp;
        he_l[t] = vptr[hp];
    }
    if (threadIdx.x == 0) *unit_ctr = waves;  // units 0 .. waves-1 are taken below

    // the first unit's first round, planned from global headers meanwhile
    int u = wave;
    int cs = 0, ce = 0, c0 = 0;
    auto unit_bounds = [&](int unit) {
        const int c = unit % nch;
        c0 = (unit / nch) * chunk_w;
        cs = bb + c * CH;
        ce = min(cs + CH, be);
    };
    RowRound r;
    int W[NWR], GS[GWR];
    T GV[GWR];
    if (u < nunits) {
        unit_bounds(u);
        rows_headers(r, cs, n_slices, lane, sptr, vptr);
        rows_fit<NWR, GWR>(r, RowCursor{cs, 0, 0, false}, ce, lane, vptr);
        rows_load<NWR, GWR>(r, W, GS, GV, lane, vptr, vals, idx);
    }

    const char *Bb = reinterpret_cast<const char *>(B);
    if constexpr (LDS_B) {
        T *lb = reinterpret_cast<T *>(smem);
        if (!b_dma) {
            for (size_t k = threadIdx.x; k < b_el; k += blockDim.x) lb[k] = B[k];
        }
        Bb = reinterpret_cast<const char *>(lb);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
    __syncthreads();                     // and every other wave's, and the headers
    if (u >= nunits) return;

    int u_next = -1;  // the unit claimed for after this one
    T acc[VEC];       // carried over the rounds of a slice
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = T(0);
    for (;;) {
        // this round's windows have landed (they were in flight during the
        // previous round); after this wait only the next round's loads are
        // pending, and nothing in this round's walk waits for them
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        if (u_next < 0) {
            int t = 0;
            if (lane == 0) t = atomicAdd(unit_ctr, 1);
            u_next = readlane(t, 0);
        }
        const int col = c0 + cl * VEC;
        const bool act = col < w;
        const uint32_t coff4 = act ? 4u * col : 0u;  // gathers stay inside B's rows

        // plan the next round and put its windows in flight (not after a
        // partial round: where it stops is known only once it is walked)
        RowRound rn;
        int W2[NWR], GS2[GWR];
        T GV2[GWR];
        bool pre = false, switch_unit = false;
        if (!r.open_end) {
            const int s_next = r.sa + r.nsl;
            if (s_next < ce) {
                rows_headers_lds(rn, s_next, bb, be, lane, hp_l, he_l);
                rows_fit<NWR, GWR>(rn, RowCursor{s_next, 0, 0, false}, ce, lane, vptr);
                pre = true;
            } else if (u_next < nunits) {
                const int c = u_next % nch;
                const int ncs = bb + c * CH, nce = min(ncs + CH, be);
                rows_headers_lds(rn, ncs, bb, be, lane, hp_l, he_l);
                rows_fit<NWR, GWR>(rn, RowCursor{ncs, 0, 0, false}, nce, lane, vptr);
                pre = switch_unit = true;
            }
            if (pre) rows_load<NWR, GWR>(rn, W2, GS2, GV2, lane, vptr, vals, idx);
        }

        write_marks<NWR, GWR>(GS, GV, r.K1 - r.K0, r.E0, r.E1, r.mid || r.open_end, lane,
                              mark, gvt);
        const int nwin = (r.E1 - r.E0 + 63) >> 6;
        int i = 0;        // slice of the round being accumulated
        int e0 = r.E0;    // its first entry in the round
        int e1 = r.nsl > 0 ? readlane(r.he, 1) : r.E1;  // its end (round end if open)

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
            e1 = i < r.nsl ? readlane(r.he, i + 1) : (r.open_end ? r.E1 : e1);
        };

        // empty slices before the first entry
        while (i < r.nsl && e1 <= r.E0) close();
        const int g_last = window_stream<LOG_WW, VEC, NWR, true>(
            W, nwin, lane, slot, mark, gvt, Bb, w4, coff4,
            [&](int k, int j0, const Stage<Gm::SBV, VEC> &st) {
                const int step0 = r.E0 + 64 * k + j0 * Gm::G;
                if (e1 >= step0 + Gm::SBV * Gm::G) {
                    // every lane of the stage is in the current slice
#pragma unroll
                    for (int t = 0; t < Gm::SBV; ++t) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[e] = fma_t(st.vj[t], st.bv[t][e], acc[e]);
                    }
                    return;
                }
#pragma unroll
                for (int t = 0; t < Gm::SBV; ++t) {
                    const int step_end = step0 + (t + 1) * Gm::G;
                    if (e0 <= step_end - Gm::G && e1 >= step_end) {
                        // this step lies inside the current slice
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[e] = fma_t(st.vj[t], st.bv[t][e], acc[e]);
                        continue;
                    }
                    const int pj = step_end - Gm::G + slot;
                    // close every slice that ends inside this step
                    while (i < r.nsl && e1 < step_end) {
                        if (pj >= e0 && pj < e1) {
#pragma unroll
                            for (int e = 0; e < VEC; ++e)
                                acc[e] = fma_t(st.vj[t], st.bv[t][e], acc[e]);
                        }
                        close();
                    }
                    if (pj >= e0 && pj < e1) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[e] = fma_t(st.vj[t], st.bv[t][e], acc[e]);
                    }
                }
            });
        // slices ending at the round's last entry, and empty ones after
        while (i < r.nsl) close();
        __builtin_amdgcn_wave_barrier();
        if (r.open_end) {  // the open slice goes on from E1
            const RowCursor c{r.sa, r.E1, r.K0 + g_last - 1, true};
            rows_headers_lds(r, c.sa, bb, be, lane, hp_l, he_l);
            rows_fit<NWR, GWR>(r, c, ce, lane, vptr);
            rows_load<NWR, GWR>(r, W, GS, GV, lane, vptr, vals, idx);
            continue;
        }
        if (!pre) break;
        if (switch_unit) {
            u = u_next;
            u_next = -1;
            unit_bounds(u);
        }
        r = rn;
#pragma unroll
        for (int k = 0; k < NWR; ++k) W[k] = W2[k];
#pragma unroll
        for (int j = 0; j < GWR; ++j) {
            GS[j] = GS2[j];
            GV[j] = GV2[j];
        }
    }
}

// Long VCS slices: each slice is walked by `wps` waves (1, 2, 4 or 8) of a
// block of 8 waves, so a block takes 8 / wps slices at a time (grid-stride
// over slice groups). Wave k of a slice takes the k-th of wps contiguous
// pieces of its entries (vcs_piece); the pieces' sums are added in wave order.
// The host picks wps so the grid's waves fill the chip about once: each wave
// then pays its chain of dependent header loads once. B stays in global
// memory (it is gathered through L2).
template <int LOG_WW, int VEC>
__global__ void __launch_bounds__(512)
k_vcs_long(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
           const float *__restrict__ vals, const int *__restrict__ idx,
           const float *__restrict__ B, float *__restrict__ out, int w, int wps) {
    using T = float;
    using Sum = SlotSum<LOG_WW, VEC>;
    __shared__ T part[8][64 * VEC];
    __shared__ __attribute__((aligned(16))) unsigned char lds[8][kPieceWaveLds];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int spb = waves / wps;     // slices per block
    const int sub = wave / wps;      // this wave's slice within the block
    const int piece = wave - sub * wps;
    const int slot = lane >> LOG_WW;
    const int cl = lane & ((1 << LOG_WW) - 1);
    const int chunk = VEC << LOG_WW;
    unsigned char *mark = lds[wave];
    T *gvt = reinterpret_cast<T *>(lds[wave] + 64 * kPieceNWR);
    const uint32_t w4 = (uint32_t)w * 4u;
    const char *Bb = reinterpret_cast<const char *>(B);
    for (int s0 = blockIdx.x * spb; s0 < n_slices; s0 += gridDim.x * spb) {
        const int s = s0 + sub;  // wave-uniform
        const bool live = s < n_slices;
        int ka = 0, kb = 0, ps = 0, pe = 0;
        if (live) {
            ka = sptr[s];
            kb = sptr[s + 1];
            const int e0 = vptr[ka], e1 = vptr[kb];
            const long long len = e1 - e0;
            ps = e0 + (int)(len * piece / wps);
            pe = e0 + (int)(len * (piece + 1) / wps);
        }
        for (int c0 = 0; c0 < w; c0 += chunk) {
            const int col = c0 + cl * VEC;
            const bool act = col < w;
            T acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = T(0);
            if (live)
                vcs_piece<LOG_WW, VEC>(ka, kb, ps, pe, lane, slot, act ? 4u * col : 0u, vptr,
                                       vals, idx, Bb, w4, mark, gvt, acc);
            T res[Sum::VO];
            Sum::run(acc, res);
            if (Sum::writer(lane)) {
#pragma unroll
                for (int e = 0; e < Sum::VO; ++e) part[wave][cl * VEC + Sum::base(lane) + e] = res[e];
            }
            __syncthreads();
            for (int t = threadIdx.x; t < spb * chunk; t += blockDim.x) {
                const int ss = t / chunk, c = t - ss * chunk;
                if (s0 + ss < n_slices && c0 + c < w) {
                    T tot = part[ss * wps][c];
                    for (int k = 1; k < wps; ++k) tot += part[ss * wps + k][c];
                    out[(size_t)(s0 + ss) * w + c0 + c] = tot;
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace vspmm
