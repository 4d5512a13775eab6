// Latency-hiding forms of the aligned walk (output rows = major slices).
//
// The plain walk issues one dependent chain per step (index load, then the
// gather of B's row, then the fma), so a wave keeps ~64 bytes in flight and
// the product runs far below the chip's bandwidth. These forms load many
// entries at once and keep several steps' gathers in flight:
//
//  - k_short: one wave walks a contiguous range of slices (for a CSR handle,
//    its entry-balanced range) in rounds: a round's entry windows are loaded
//    together, turned into (index, value) pairs in a per-wave LDS ring, and
//    walked step by step, NC width chunks at a time. With LDS_B the gathered
//    operand is first copied into the CU's LDS (one 1024-thread block per
//    CU), so gathers use the LDS pipe. Slices longer than long_len are left to
//    the long walk; with long blocks, the first blocks of the same launch run
//    it beside the short slices.
//  - long_walk (k_long, and the long blocks of k_short): a group of waves
//    walks one slice (kLongWaves for a handle's long-row list; for a matrix
//    walked by k_long alone, as many as its mean row fills passes), wave k
//    taking the k-th of the group's contiguous pieces of its entries; the
//    pieces' partial sums are added in wave order.
//
// Gathers are issued by every lane without branches (an idle lane reads a
// valid row), so a step's loads go out together; only the FMAs are masked.
//
// Arithmetic order: entry lane `slot` adds v * B[i] with one fma per element
// over its entries slot, slot + G, slot + 2G, ... of the slice (of the wave's
// piece, for the long walk) in order; the G entry lanes are combined by a
// fixed xor tree, and the long walk adds the waves' partials in wave order.
// Results repeat bit for bit and depend on the width only through the
// chunking of columns, never in a column's own arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "walk.hpp"

namespace vspmm {

template <typename T>
struct BatchSteps {
    static constexpr int value = sizeof(T) == 8 ? 4 : 8;
};

// Group bookkeeping for a VCS walk. Lanes hold the starts and values of 64
// consecutive groups (gb + lane); u is the wave-uniform cursor of the group
// holding the current position.
template <typename T>
struct Groups {
    int gb, u, kb, gs;
    T gv;
};

template <typename T>
__device__ __forceinline__ void groups_load(Groups<T> &g, int gb, int kb, int lane,
                                            const int *__restrict__ vptr,
                                            const T *__restrict__ vals) {
    g.gb = gb;
    g.u = 0;
    g.kb = kb;
    g.gs = vptr[min(gb + lane, kb)];
    g.gv = vals[min(gb + lane, max(kb - 1, 0))];
}

// Value of position p for a step covering [q, qend) (positions only move
// forward). Groups that start inside the step are applied in order, so an
// empty group is overridden by the next one.
template <typename T>
__device__ __forceinline__ T groups_value(Groups<T> &g, int p, int qend, int lane,
                                          const int *__restrict__ vptr,
                                          const T *__restrict__ vals) {
    T v = readlane(g.gv, g.u);
    for (;;) {
        if (g.u == 63) {
            g.gb += 63;
            g.u = 0;
            g.gs = vptr[min(g.gb + lane, g.kb)];
            g.gv = vals[min(g.gb + lane, g.kb - 1)];
        }
        const int ns = readlane(g.gs, g.u + 1);
        if (ns >= qend) break;
        ++g.u;
        const T nv = readlane(g.gv, g.u);
        v = (p >= ns) ? nv : v;
    }
    return v;
}

// groups_value for a slice whose groups all fit one window with its end
// sentinel (kb - gb <= 63): no reload, so the cursor never issues a load.
template <typename T>
__device__ __forceinline__ T groups_value_fast(const Groups<T> &gc, int &u, int p, int qend) {
    T v = readlane(gc.gv, u);
    for (;;) {
        const int ns = readlane(gc.gs, u + 1);
        if (ns >= qend) break;
        ++u;
        const T nv = readlane(gc.gv, u);
        v = (p >= ns) ? nv : v;
    }
    return v;
}

// Moves the cursor to the group holding entry c (the last group whose start
// is <= c), for a slice with groups [ka, kb). g0 is the slice's first window.
template <typename T>
__device__ __forceinline__ void groups_seek(Groups<T> &g, const Groups<T> &g0, int ka, int kb,
                                            int c, int lane, const int *__restrict__ vptr,
                                            const T *__restrict__ vals) {
    if (kb - ka <= 64) {
        g = g0;
    } else {  // binary search over the slice's group starts
        int lo = ka, hi = kb - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (vptr[mid] <= c) lo = mid;
            else hi = mid - 1;
        }
        groups_load(g, lo, kb, lane, vptr, vals);
    }
    const bool le = (g.gb + lane < kb) && (g.gs <= c);
    g.u = max(__popcll(__ballot(le)) - 1, 0);
}

// Header of slice s from a batch of pointers held in lanes: hp = sptr[hb +
// lane], he = first entry of slice hb + lane.
struct Headers {
    int hb, hp, he;
};

// Waits for every outstanding vector-memory access of the wave (vmcnt 0,
// other counters left alone). Used inside rarely taken branches whose loads
// are consumed right away, so the compiler does not carry them as pending into
// the common path (where a conservative wait would drain the prefetches).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <bool VCS>
__device__ __forceinline__ void headers_load(Headers &h, int hb, int n_slices, int lane,
                                             const int *__restrict__ sptr,
                                             const int *__restrict__ vptr) {
    h.hb = hb;
    h.hp = sptr[min(hb + lane, n_slices)];
    if constexpr (VCS) {
        wait_vm_all();
        h.he = vptr[h.hp];
    } else {
        h.he = h.hp;
    }
    wait_vm_all();
}

// A batch: NS steps of a run of entries starting at c (lane's entry of step j
// is c + j*G + slot; idle lanes hold index 0 and value 0).
template <typename T, int NS>
struct Batch {
    int ix[NS];
    T vv[NS];
};

template <bool VCS, typename T, int NS, typename VP>
__device__ __forceinline__ void batch_load(Batch<T, NS> &b, int c, int e1, int G, int slot,
                                           VP vals, const int *__restrict__ idx) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int p = c + j * G + slot;
        const bool valid = p < e1;
        b.ix[j] = valid ? idx[p] : 0;
        if constexpr (!VCS) b.vv[j] = valid ? vals[p] : T(0);
    }
}

// Gathers issued for a batch, not yet accumulated.
template <typename T, int VEC, int NS>
struct Pending {
    T v[NS];
    T b[NS][VEC];
};

template <bool VCS, typename T, int VEC, int NS, typename VP>
__device__ __forceinline__ void batch_issue(Pending<T, VEC, NS> &pd, const Batch<T, NS> &b, int c,
                                            int e1, int G, int slot, int col, bool act,
                                            Groups<T> &g, int lane, const int *__restrict__ vptr,
                                            VP vals, const T *Bs, int w) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int q = c + j * G;
        if constexpr (VCS) {
            pd.v[j] = (q < e1) ? groups_value(g, q + slot, min(q + G, e1), lane, vptr, vals) : T(0);
        } else {
            pd.v[j] = b.vv[j];
        }
        if (act && q + slot < e1) {
            load_vec<T, VEC>(Bs + (size_t)b.ix[j] * w + col, pd.b[j]);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) pd.b[j][e] = T(0);
        }
    }
}

template <typename T, int VEC, int NS>
__device__ __forceinline__ void batch_consume(const Pending<T, VEC, NS> &pd, T (&acc)[VEC]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fma_t(pd.v[j], pd.b[j][e], acc[e]);
    }
}

// Sum of the slice's G entry lanes for a full-wave split (G * WW == 64).
template <typename T, int VEC>
__device__ __forceinline__ void xor_reduce(T (&acc)[VEC], int from, int to) {
    (void)to;
    slot_reduce_dpp<T, VEC>(acc, __builtin_ctz(from));
}

// Accumulates the batches starting at c, c + stride, ... below e1 into acc,
// loading each next batch while the current one's gathers are in flight.
// stride must be NS * G (a contiguous run), so the group cursor g, which must
// sit at or before entry c, only moves forward.
template <bool VCS, typename T, int VEC, int NS, typename VP>
__device__ __forceinline__ void run_batches(int c, int e1, int stride, int G, int slot, int col,
                                            bool act, Groups<T> &g, int lane,
                                            const int *__restrict__ vptr, VP vals,
                                            const int *__restrict__ idx, const T *Bs, int w,
                                            T (&acc)[VEC]) {
    if (c >= e1) return;
    Batch<T, NS> ba, bb;
    Pending<T, VEC, NS> pd;
    batch_load<VCS, T, NS>(ba, c, e1, G, slot, vals, idx);
    for (;;) {
        batch_issue<VCS, T, VEC, NS>(pd, ba, c, e1, G, slot, col, act, g, lane, vptr, vals, Bs, w);
        const int cn = c + stride;
        if (cn < e1) batch_load<VCS, T, NS>(bb, cn, e1, G, slot, vals, idx);
        batch_consume<T, VEC, NS>(pd, acc);
        if (cn >= e1) return;
        batch_issue<VCS, T, VEC, NS>(pd, bb, cn, e1, G, slot, col, act, g, lane, vptr, vals, Bs,
                                     w);
        c = cn + stride;
        if (c < e1) batch_load<VCS, T, NS>(ba, c, e1, G, slot, vals, idx);
        batch_consume<T, VEC, NS>(pd, acc);
        if (c >= e1) return;
    }
}

// ------------------------------------------------------------------ short

// Short slices are walked in rounds. A round is a run of whole consecutive
// slices of the wave's block holding at most 64*NWR entries and 64*GWR groups:
// all its loads (slice pointers, entry windows, group windows) are issued
// together and awaited once, then the round is computed from registers. All
// of a round's bytes are in flight at the same time, which is what keeps HBM
// busy; nothing is carried in flight across a wait, so the schedule does not
// depend on the compiler keeping partial wait counts.
//
// The lane-held windows are separate local arrays (not struct members): a
// struct whose arrays are indexed at run time cannot be split into registers
// and would live in scratch memory.
struct Round {
    int sa, nsl;      // first slice, number of slices
    int E0, E1;       // entries [E0, E1)
    int K0, K1;       // groups [K0, K1) (VCS)
    int hp, he;       // lanes: slice pointer / first entry of slice sa + lane
};
// Windows of a round, held by lanes:
//   W[k]  = idx[E0 + 64k + lane]       V[k]  = CSR value of the same entry
//   GS[k] = vptr[K0 + 64k + lane] (clamped to K1)   GV[k] = values[K0 + 64k + lane]

// Loads the slice pointers of slices sa .. sa+63 and picks the longest run
// of whole slices that fits the round's windows (at least one slice; a single
// slice too big for the round is reported with nsl = -1).
template <bool VCS, int NWR, int GWR>
__device__ __forceinline__ void round_plan(Round &r, int sa, int s_end, int n_slices,
                                           int lane, const int *__restrict__ sptr,
                                           const int *__restrict__ vptr,
                                           int long_len = 0x7fffffff) {
    r.sa = sa;
    r.hp = sptr[min(sa + lane, n_slices)];
    if constexpr (VCS) r.he = vptr[r.hp];
    else r.he = r.hp;
    const int e_first = readlane(r.he, 0);
    const int k_first = readlane(r.hp, 0);
    // the round stops before the first slice longer than long_len (a round
    // starting at one is empty: the caller skips that slice)
    const int len = __shfl_down(r.he, 1) - r.he;  // slice sa + lane (lanes 0..62)
    const unsigned long long lng = __ballot(lane < 63 && sa + lane < s_end && len > long_len);
    const int first_long = lng ? __builtin_ctzll(lng) : 64;
    const bool fits = (sa + lane <= s_end) && (r.he - e_first <= 64 * NWR) &&
                      lane <= first_long && (!VCS || r.hp - k_first <= 64 * GWR - 1);
    const int last = __popcll(__ballot(fits)) - 1;  // fits is a prefix of the lanes
    r.nsl = last > 0 ? last : -1;
    r.E0 = e_first;
    r.K0 = k_first;
    r.E1 = readlane(r.he, last > 0 ? last : 1);
    r.K1 = readlane(r.hp, last > 0 ? last : 1);
}

template <bool VCS, typename T, int NWR, int GWR, typename VP>
__device__ __forceinline__ void round_load(const Round &r, int (&W)[NWR], T (&V)[NWR],
                                           int (&GS)[GWR], T (&GV)[GWR], int lane,
                                           const int *__restrict__ vptr, VP vals,
                                           const int *__restrict__ idx) {
#pragma unroll
    for (int k = 0; k < NWR; ++k) {
        if (r.E0 + 64 * k < r.E1) {
            const int p = min(r.E0 + 64 * k + lane, r.E1 - 1);
            W[k] = idx[p];
            if constexpr (!VCS) V[k] = vals[p];
        }
    }
    if constexpr (VCS) {
#pragma unroll
        for (int k = 0; k < GWR; ++k) {
            if (r.K0 + 64 * k <= r.K1) {
                GS[k] = vptr[min(r.K0 + 64 * k + lane, r.K1)];
                GV[k] = vals[max(min(r.K0 + 64 * k + lane, r.K1 - 1), 0)];
            }
        }
    }
}

// Element o (round-relative) of a lane-held window array, as seen by this
// lane's entry lane: the windows hold entry o at lane o & 63 of W[o >> 6].
template <typename T, int N>
__device__ __forceinline__ T window_pick(const T (&W)[N], int o_step, int slot, int G) {
    const int k = o_step >> 6;      // wave-uniform
    const int l0 = o_step & 63;
    const int src = l0 + slot;
    T a = __shfl(W[k], src & 63);
    if (l0 + G > 64) {  // the step runs into the next window
        const T b = __shfl(W[min(k + 1, N - 1)], src & 63);
        a = src >= 64 ? b : a;
    }
    return a;
}

template <typename T, int N>
__device__ __forceinline__ T lanes_at(const T (&X)[N], int g) {
    return readlane(X[g >> 6], g & 63);
}

// Per-wave LDS ring of (index, value) pairs: positions of the round are
// written 64 at a time (one window) and read back by the entry lanes, so each
// step costs two LDS reads instead of shuffles and scalar loops.

template <typename T>
struct RingEntry {
    int ix;
    T v;
};

// out[s] for each slice of a loaded round, width chunks c0 .. c0 + NC - 1
// (a chunk is the VEC << log_ww columns the width lanes cover at once).
// Windows are turned into (index, value) pairs one at a time; every step
// whose entries are already in the ring is then walked, finishing slices as
// they end. Taking NC chunks in one walk reads each step's (index, value) pair
// once for all of them; a column's arithmetic is the same for any NC.
template <bool VCS, typename T, int VEC, int NWR, int GWR, int SB, int NC>
__device__ __forceinline__ void round_compute(const Round &r, const int (&W)[NWR],
                                              const T (&V)[NWR], const int (&GS)[GWR],
                                              const T (&GV)[GWR], int c0, int lane, int slot,
                                              int cl, const Split &sp, const T *Bs,
                                              RingEntry<T> *ring, int ring_n, T *__restrict__ out,
                                              int w) {
    // steps whose gathers are in flight together (float64 keeps two at any
    // NC; float32 at NC = 4 has no registers left for a second)
    constexpr int SBN = sizeof(T) == 8 ? 2 : (SB / NC > 0 ? SB / NC : 1);
    const int G = 1 << sp.log_g;
    const int chunk = VEC << sp.log_ww;
    int col[NC];
    bool act[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        col[j] = c0 + j * chunk + cl * VEC;
        act[j] = col[j] < w;
    }
    int i = 0;                       // slice of the round being accumulated
    int q = r.E0;                    // its next step
    int e1 = readlane(r.he, 1);      // its end
    int g = 0;                       // VCS: group (round-relative) of the window's first position
    T acc[NC][VEC];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] = T(0);
    auto finish = [&]() {  // slice i is complete: reduce, store, reset
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            xor_reduce<T, VEC>(acc[j], 1 << sp.log_ww, 64);
            if (slot == 0 && act[j]) store_vec<T, VEC>(out + (size_t)(r.sa + i) * w + col[j], acc[j]);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[j][e] = T(0);
        }
    };
#pragma unroll
    for (int k = 0; k < NWR; ++k) {
        const int wbase = r.E0 + 64 * k;
        if (wbase >= r.E1) break;
        T vk;
        if constexpr (VCS) {
            const int P = wbase + lane;
            const int wend = min(wbase + 64, r.E1);
            vk = lanes_at(GV, g);
            for (;;) {
                const int ns = lanes_at(GS, g + 1);
                if (ns >= wend) break;
                ++g;
                const T nv = lanes_at(GV, g);
                vk = (P >= ns) ? nv : vk;
            }
        } else {
            vk = V[k];
        }
        ring[(64 * k + lane) & (ring_n - 1)] = RingEntry<T>{W[k], vk};
        // a deep ring is walked once four windows are in it (or the round's
        // last), so window-wide steps come four to a batch
        if (ring_n > kRing && (k & 3) != 3 && wbase + 64 < r.E1) continue;
        const int ready = min(wbase + 64, r.E1);
        for (;;) {
            while (q >= e1) {  // slice i is complete
                finish();
                ++i;
                q = e1;  // slice i starts where slice i - 1 ends
                if (i >= r.nsl) break;
                e1 = readlane(r.he, i + 1);
            }
            if (i >= r.nsl) break;
            // steps of slice i whose entries are all in the ring: every step
            // up to the slice's end if it ends before `ready`, else whole steps
            const int avail = min(e1, ready);
            if (avail <= q) break;
            int nb = avail == e1 ? (avail - q + G - 1) >> sp.log_g : (avail - q) >> sp.log_g;
            if (nb == 0) break;
            nb = min(nb, SBN);
            // gathers are issued for every lane of the batch without branches
            // (a lane past the slice's end, or past what the ring holds, reads
            // row 0; a lane past the width reads column 0), so the batch's
            // loads are in flight together; only the FMAs are masked. An FMA
            // skipped here would have added 0 * 0 to an accumulator that is
            // never -0, so the result is the same bit for bit.
            RingEntry<T> re[SBN];
#pragma unroll
            for (int t = 0; t < SBN; ++t) re[t] = ring[(q + t * G + slot - r.E0) & (ring_n - 1)];
            T bv[SBN][NC][VEC];
            bool live[SBN];
#pragma unroll
            for (int t = 0; t < SBN; ++t) {
                live[t] = t < nb && q + t * G + slot < e1;
                const size_t row = (size_t)(live[t] ? re[t].ix : 0) * w;
#pragma unroll
                for (int j = 0; j < NC; ++j)
                    load_vec<T, VEC>(Bs + row + (act[j] ? col[j] : 0), bv[t][j]);
            }
#pragma unroll
            for (int t = 0; t < SBN; ++t) {
                if (live[t]) {
#pragma unroll
                    for (int j = 0; j < NC; ++j)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[j][e] = fma_t(re[t].v, bv[t][j][e], acc[j][e]);
                }
            }
            q += nb * G;
        }
    }
    // slices left after the last window are empty (no entries): zeros
    while (i < r.nsl) {
        if (q >= e1) {
            finish();
            ++i;
            q = e1;
            if (i < r.nsl) e1 = readlane(r.he, i + 1);
        } else {
            break;  // unreachable for a well-formed round
        }
    }
}

// A slice too big for a round: walked alone, window by window, with the
// plain per-step group cursor.
template <bool VCS, typename T, int VEC, int SB, typename VP>
__device__ __forceinline__ void big_slice(int s, int lane, int slot, int cl, const Split &sp,
                                          const int *__restrict__ sptr,
                                          const int *__restrict__ vptr,
                                          VP vals, const int *__restrict__ idx,
                                          const T *Bs, T *__restrict__ out, int w) {
    const int G = 1 << sp.log_g;
    const int chunk = VEC << sp.log_ww;
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
    for (int c0 = 0; c0 < w; c0 += chunk) {
        const int col = c0 + cl * VEC;
        const bool act = col < w;
        T acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = T(0);
        Groups<T> g;
        if constexpr (VCS) groups_load(g, ka, kb, lane, vptr, vals);
        for (int base = e0; base < e1; base += 64) {
            const int p = min(base + lane, e1 - 1);
            const int wi = idx[p];
            T wv = T(0);
            if constexpr (!VCS) wv = vals[p];
            const int nsteps = 64 / G;
            for (int j0 = 0; j0 < nsteps; j0 += SB) {
                if (base + j0 * G >= e1) break;
                T bv[SB][VEC];
                T vj[SB];
#pragma unroll
                for (int t = 0; t < SB; ++t) {
                    const int j = j0 + t;
                    const int q = base + j * G;
                    const bool live = j < nsteps && q < e1;
                    const int src = (j * G + slot) & 63;
                    const int ix = __shfl(wi, src);
                    if constexpr (VCS)
                        vj[t] = live ? groups_value(g, q + slot, min(q + G, e1), lane, vptr, vals)
                                     : T(0);
                    else
                    {
                        const T v = __shfl(wv, src);  // all lanes shuffle
                        vj[t] = (live && q + slot < e1) ? v : T(0);
                    }
                    if (live && act && q + slot < e1) {
                        load_vec<T, VEC>(Bs + (size_t)ix * w + col, bv[t]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) bv[t][e] = T(0);
                    }
                }
#pragma unroll
                for (int t = 0; t < SB; ++t) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = fma_t(vj[t], bv[t][e], acc[e]);
                }
            }
        }
        xor_reduce<T, VEC>(acc, 1 << sp.log_ww, 64);
        if (slot == 0 && act) store_vec<T, VEC>(out + (size_t)s * w + col, acc);
    }
}

constexpr int kLongWaves = 8;  // waves walking one long slice (see long_walk)

template <bool VCS, typename T, int VEC, int NC, int SBN, int NWR, typename VP>
__device__ __forceinline__ void long_walk(int first, int stride, int n_walk,
                                          const int *__restrict__ list, int group, int wave,
                                          T *part, const int *__restrict__ sptr,
                                          const int *__restrict__ vptr, VP vals,
                                          const int *__restrict__ idx, const T *__restrict__ B,
                                          T *__restrict__ out, int w, Split sp, int waves);

// Short slices; requires G * WW == 64. Each wave walks a contiguous block of
// slices in rounds. LDS_B stages B (n_in x w) in dynamic LDS first (one
// 1024-thread block per CU), so gathers use the LDS pipe. A slice too long
// for one round (more than 64 * NWR entries) is walked by the wave alone, or,
// with skip_big, left to k_long over the list of such slices. NC width chunks
// are walked together (1, 2 or 4, so that NC chunks cover the width or come
// closest to it).
template <bool VCS, typename T, int VEC, bool LDS_B, int NC, typename VP = const T *>
__global__ void __launch_bounds__(1024)
k_short(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
        VP vals, const int *__restrict__ idx, const T *__restrict__ B,
        T *__restrict__ out, int w, int n_in, Split sp, int skip_big, int long_len,
        const int *__restrict__ parts, int n_parts, const int *__restrict__ long_list,
        int n_long, int long_blocks, int ring_n) {
    constexpr int NWR = sizeof(T) == 8 ? 12 : 24;
    constexpr int GWR = 4;
    constexpr int SB = sizeof(T) == 8 ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int slot = lane >> sp.log_ww;
    const int cl = lane & ((1 << sp.log_ww) - 1);
    const int chunk = VEC << sp.log_ww;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int)blockIdx.x < long_blocks) {
        // the first blocks walk the listed long slices, kLongWaves waves each
        // (blocks of 8 or 16 waves: one or two groups), beside the short walk
        const int groups = waves / kLongWaves;
        const int group = wave / kLongWaves;
        T *part = reinterpret_cast<T *>(smem) + group * (kLongWaves * NC * 64 * VEC);
        // (under this kernel's register bound: one step's gathers per NC)
        constexpr int LSBN = SB / NC > 0 ? SB / NC : 1;
        long_walk<VCS, T, VEC, NC, LSBN, 8>(blockIdx.x * groups, long_blocks * groups, n_long, long_list,
                                   group, wave - group * kLongWaves, part, sptr, vptr, vals, idx,
                                   B, out, w, sp, kLongWaves);
        return;
    }
    // dynamic LDS: [B staged (LDS_B), 16-byte aligned][one ring per wave]
    const size_t b_bytes = LDS_B ? (((size_t)n_in * w * sizeof(T) + 15) & ~size_t(15)) : 0;
    RingEntry<T> *ring = reinterpret_cast<RingEntry<T> *>(smem + b_bytes) + wave * ring_n;
    const long long tw = (long long)(gridDim.x - long_blocks) * waves;
    const long long gw = (long long)(blockIdx.x - long_blocks) * waves + wave;
    int s_beg = (int)(gw * n_slices / tw);
    int s_end = (int)((gw + 1) * n_slices / tw);
    if (parts && n_parts == tw) {  // entry-balanced row ranges
        s_beg = parts[gw];
        s_end = parts[gw + 1];
    }

    Round r;
    int W[NWR], GS[GWR];
    T V[NWR], GV[GWR];
    if (s_beg < s_end) {
        round_plan<VCS, NWR, GWR>(r, s_beg, s_end, n_slices, lane, sptr, vptr, long_len);
        if (r.nsl > 0) round_load<VCS, T, NWR, GWR>(r, W, V, GS, GV, lane, vptr, vals, idx);
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
        if (r.nsl < 0) {  // one slice larger than a round, or than long_len
            // (with skip_big the long walk over the list of such slices writes it)
            if (!skip_big)
                big_slice<VCS, T, VEC, SB>(sa, lane, slot, cl, sp, sptr, vptr, vals, idx, Bs, out, w);
            sa += 1;
        } else {
            for (int c0 = 0; c0 < w; c0 += NC * chunk)
                round_compute<VCS, T, VEC, NWR, GWR, SB, NC>(r, W, V, GS, GV, c0, lane, slot, cl,
                                                             sp, Bs, ring, ring_n, out, w);
            sa += r.nsl;
        }
        if (sa < s_end) {
            round_plan<VCS, NWR, GWR>(r, sa, s_end, n_slices, lane, sptr, vptr, long_len);
            if (r.nsl > 0) round_load<VCS, T, NWR, GWR>(r, W, V, GS, GV, lane, vptr, vals, idx);
        }
    }
}

// ------------------------------------------------------------------- long

// Long slices: each is walked by a group of waves; wave k of the group takes
// the k-th of the group's contiguous pieces of the slice's entries; a piece
// (up to 64*NWR entries per pass) and the slice's group window are loaded at
// once, then walked from registers. The waves' partial rows are added in wave
// order. The group size depends only on the matrix (and on whether the slice
// is on a long-row list), so a column's arithmetic is the same at every
// width.
//
// long_walk: the block's `groups` groups of `waves` waves (kLongWaves for the
// handle's long-row list; for a matrix walked by k_long alone, as many as its
// mean row fills passes, at most kLongWaves) take the slices li = first +
// group, then li + stride, ... (li < n_walk; the slice is list[li], or li
// without a list); every wave of the block runs the same iterations (the
// barriers are block-wide). part: LDS for the group, waves x NC*64*VEC
// elements.
// SBN steps have their gathers in flight together, and a pass loads NWR
// windows; both set registers, not the arithmetic: a pass holds a multiple of
// G entries, so each lane gets the same entries in the same order either way.
template <bool VCS, typename T, int VEC, int NC, int SBN, int NWR, typename VP>
__device__ __forceinline__ void long_walk(int first, int stride, int n_walk,
                                          const int *__restrict__ list, int group, int wave,
                                          T *part, const int *__restrict__ sptr,
                                          const int *__restrict__ vptr, VP vals,
                                          const int *__restrict__ idx, const T *__restrict__ B,
                                          T *__restrict__ out, int w, Split sp, int waves) {
    constexpr int PW = NC * 64 * VEC;  // part elements per wave
    const int lane = threadIdx.x & 63;
    const int G = 1 << sp.log_g;
    const int slot = lane >> sp.log_ww;
    const int cl = lane & ((1 << sp.log_ww) - 1);
    const int chunk_w = VEC << sp.log_ww;
    for (int base = first; base < n_walk; base += stride) {
        const int li = base + group;
        const bool live = li < n_walk;  // uniform in the group
        const int s = live ? (list ? list[li] : li) : 0;
        int e0 = 0, e1 = 0, ka = 0, kb = 0;
        if (!live) {
        } else if constexpr (VCS) {
            ka = sptr[s];
            kb = sptr[s + 1];
            e0 = vptr[ka];
            e1 = vptr[kb];
        } else {
            e0 = sptr[s];
            e1 = sptr[s + 1];
        }
        const long long len = e1 - e0;
        const int ps = e0 + (int)(len * wave / waves);
        const int pe = e0 + (int)(len * (wave + 1) / waves);
        // NC width chunks per walk of the piece (a column's arithmetic is the
        // same for any NC)
        for (int c0 = 0; c0 < w; c0 += NC * chunk_w) {
            int col[NC];
            bool act[NC];
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                col[j] = c0 + j * chunk_w + cl * VEC;
                act[j] = col[j] < w;
            }
            T acc[NC][VEC];
#pragma unroll
            for (int j = 0; j < NC; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[j][e] = T(0);
            for (int P0 = ps; P0 < pe; P0 += 64 * NWR) {
                const int P1 = min(pe, P0 + 64 * NWR);
                int W[NWR];
                T V[NWR];
                // every window is loaded (clamped to the pass), so the loads
                // carry no branches and go out back to back
#pragma unroll
                for (int k = 0; k < NWR; ++k) {
                    const int p = min(P0 + 64 * k + lane, P1 - 1);
                    W[k] = idx[p];
                    if constexpr (!VCS) V[k] = vals[p];
                }
                Groups<T> g;
                if constexpr (VCS) {
                    Groups<T> g0;
                    groups_load(g0, ka, kb, lane, vptr, vals);
                    groups_seek(g, g0, ka, kb, P0, lane, vptr, vals);
                }
                for (int q0 = P0; q0 < P1; q0 += SBN * G) {
                    // as in round_compute: gathers without branches (dead
                    // lanes read row 0 or column 0 of the pass), masked FMAs
                    T bv[SBN][NC][VEC];
                    T vj[SBN];
                    bool lv[SBN];
#pragma unroll
                    for (int t = 0; t < SBN; ++t) {
                        const int q = q0 + t * G;
                        const int p = q + slot;
                        const bool live = q < P1;  // wave-uniform
                        const int o = live ? q - P0 : 0;
                        lv[t] = live && p < P1;
                        const int ix = window_pick(W, o, slot, G);  // the windows are clamped
                        if constexpr (VCS)
                            vj[t] = live ? groups_value(g, p, min(q + G, P1), lane, vptr, vals)
                                         : T(0);
                        else
                            vj[t] = window_pick(V, o, slot, G);
                        const size_t row = (size_t)(lv[t] ? ix : 0) * w;
#pragma unroll
                        for (int j = 0; j < NC; ++j)
                            load_vec<T, VEC>(B + row + (act[j] ? col[j] : 0), bv[t][j]);
                    }
#pragma unroll
                    for (int t = 0; t < SBN; ++t) {
                        if (lv[t]) {
#pragma unroll
                            for (int j = 0; j < NC; ++j)
#pragma unroll
                                for (int e = 0; e < VEC; ++e)
                                    acc[j][e] = fma_t(vj[t], bv[t][j][e], acc[j][e]);
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                xor_reduce<T, VEC>(acc[j], 1 << sp.log_ww, 64);
                if (slot == 0) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) part[wave * PW + j * chunk_w + cl * VEC + e] = acc[j][e];
                }
            }
            __syncthreads();
            if (live && wave == 0 && slot == 0) {
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    if (!act[j]) continue;
                    T tot[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) tot[e] = part[j * chunk_w + cl * VEC + e];
                    for (int k = 1; k < waves; ++k) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) tot[e] += part[k * PW + j * chunk_w + cl * VEC + e];
                    }
                    store_vec<T, VEC>(out + (size_t)s * w + col[j], tot);
                }
            }
            __syncthreads();
        }
    }
}


// k_long: a group of wps waves (1, 2, 4 or 8; kLongWaves / wps groups per
// block) per slice, grid-stride over the slices, or over the slices in `list`
// when it is given; requires G * WW == 64.
template <bool VCS, typename T, int VEC, int NC, typename VP = const T *>
__global__ void __launch_bounds__(64 * kLongWaves)
k_long(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
       VP vals, const int *__restrict__ idx, const T *__restrict__ B,
       T *__restrict__ out, int w, Split sp, const int *__restrict__ list, int n_list, int wps) {
    constexpr int PW = NC * 64 * VEC;
    __shared__ T part[kLongWaves * PW];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int groups = kLongWaves / wps;
    const int group = wave / wps;
    constexpr int SB = sizeof(T) == 8 ? 2 : 4;
    long_walk<VCS, T, VEC, NC, SB, sizeof(T) == 8 ? 12 : 24>(
        blockIdx.x * groups, gridDim.x * groups, list ? n_list : n_slices, list, group,
        wave - group * wps, part + group * wps * PW, sptr, vptr, vals, idx, B, out, w, sp, wps);
}

}  // namespace vspmm
