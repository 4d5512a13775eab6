// The scatter walk: the misaligned direction in atomic mode. For every entry
// (s, i, v) of the walked layout, out[i][:] += v * B[s][:] (B: one row per
// slice, out: one row per minor index, zeroed first). This is the product the
// vsparse page's "The kernels" section pairs with atomic adds for a layout
// whose slices run across the output.
//
// Work is split by entries, not slices: wave k of the grid takes the entries
// [nnz * k / W, nnz * (k + 1) / W) whatever slices and groups they fall in, so
// long and short slices balance alike. A wave walks its range in windows of
// up to 64 consecutive entries, one per lane: it holds in lanes the starts of
// the 64 groups from the window's first group on (VCS) and the starts of the
// 64 slices from the window's first slice on, and finds each entry's group
// and slice by a binary search over those lanes. The adds then go in rounds:
// the wave is G = 64 / WW lane groups of WW lanes (one column each), lane
// group k takes in round r the entry held by its own lane r, passed across
// the group by a DPP broadcast. All rounds' B loads are issued before the
// next window's lanes are loaded and before the first add, so both stay in
// flight while the adds run.
//
// With PRIV the block first adds into a copy of out in LDS (out must fit in a
// CU's LDS), then adds each non-zero element of its copy into out once.
#include <utility>

#include "launch.hpp"
#include "walk.hpp"

namespace vspmm {
namespace {

// Largest x in [lo, hi) with key(x) <= t, for keys nondecreasing in x and
// key(lo) <= t. The wave probes 64 points a step, so a range of n takes
// about log64(n) dependent loads.
template <typename K>
__device__ __forceinline__ int wave_search(int lo, int hi, int t, int lane, K key) {
    while (hi - lo > 1) {
        const int step = int((int64_t(hi) - lo + 63) >> 6);
        const int64_t x = int64_t(lo) + int64_t(lane) * step;
        const bool le = x < hi && key(int(x)) <= t;
        const int c = __popcll(__ballot(le));  // a prefix of the lanes, lane 0 included
        lo = __builtin_amdgcn_readfirstlane(lo + (c - 1) * step);
        hi = min(hi, lo + step);
    }
    return lo;
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Lane l gets x from lane (l & ~(WW - 1)) | R of its lane group.
template <int LOG_WW, int R>
__device__ __forceinline__ int bcast(int x) {
    if constexpr (LOG_WW == 0) {
        return x;
    } else if constexpr (LOG_WW == 1) {
        return __builtin_amdgcn_mov_dpp(x, R == 0 ? 0xA0 : 0xF5, 0xf, 0xf, false);  // quad_perm
    } else if constexpr (LOG_WW == 2) {
        return __builtin_amdgcn_mov_dpp(x, R * 0x55, 0xf, 0xf, false);  // quad_perm [R,R,R,R]
    } else if constexpr (LOG_WW == 3) {
        // row_newbcast takes lane R of the 16-lane row: the upper half of
        // each row takes its lane 8 + R instead
        const int lo = __builtin_amdgcn_mov_dpp(x, 0x150 + R, 0xf, 0xf, false);
        const int hi = __builtin_amdgcn_mov_dpp(x, 0x158 + R, 0xf, 0xf, false);
        return (__lane_id() & 8) ? hi : lo;
    } else {
        static_assert(LOG_WW == 4, "DPP broadcasts cover lane groups of up to 16");
        return __builtin_amdgcn_mov_dpp(x, 0x150 + R, 0xf, 0xf, false);  // row_newbcast
    }
}
template <int LOG_WW, int R>
__device__ __forceinline__ float bcast(float x) {
    return __int_as_float(bcast<LOG_WW, R>(__float_as_int(x)));
}
template <int LOG_WW, int R>
__device__ __forceinline__ double bcast(double x) {
    const long long u = __double_as_longlong(x);
    const int lo = bcast<LOG_WW, R>(int(u)), hi = bcast<LOG_WW, R>(int(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Groups of 32 or 64 lanes: r is wave-uniform, the value read with readlane.
template <int LOG_WW>
__device__ __forceinline__ int bcast_rt(int x, int r) {
    if constexpr (LOG_WW == 6) {
        return __builtin_amdgcn_readlane(x, r);
    } else {
        const int lo = __builtin_amdgcn_readlane(x, r), hi = __builtin_amdgcn_readlane(x, r + 32);
        return (__lane_id() & 32) ? hi : lo;
    }
}
template <int LOG_WW>
__device__ __forceinline__ float bcast_rt(float x, int r) {
    return __int_as_float(bcast_rt<LOG_WW>(__float_as_int(x), r));
}
template <int LOG_WW>
__device__ __forceinline__ double bcast_rt(double x, int r) {
    const long long u = __double_as_longlong(x);
    const int lo = bcast_rt<LOG_WW>(int(u), r), hi = bcast_rt<LOG_WW>(int(u >> 32), r);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

template <typename F, int... Rs>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Rs...>, F &&f) {
    (f(std::integral_constant<int, Rs>{}), ...);
}

template <bool VCS, typename T, int LOG_WW, bool PRIV, typename VP = const T *>
__global__ void __launch_bounds__(1024)
k_scatter(ScatterArgs<T> a, VP vals) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    T *priv = reinterpret_cast<T *>(smem);
    const size_t n_el = size_t(a.n_out) * size_t(a.w);
    if constexpr (PRIV) {
        for (size_t k = threadIdx.x; k < n_el; k += blockDim.x) priv[k] = T(0);
        __syncthreads();
    }
    T *dst = PRIV ? priv : a.out;
    constexpr int WW = 1 << LOG_WW;
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int gw = blockIdx.x * waves + uni(threadIdx.x >> 6);
    const int64_t n_waves = int64_t(gridDim.x) * waves;
    const int slot = lane >> LOG_WW;  // lane group: its lane r holds its round-r entry
    const int cl = lane & (WW - 1);
    const int w = a.w;
    const int nnz = a.nnz;
    int q = uni(int(int64_t(nnz) * gw / n_waves));
    const int qend = uni(int(int64_t(nnz) * (gw + 1) / n_waves));
    if (q < qend) {
        // the group holding entry q (VCS) and the slice holding that group
        int g0 = q;
        if constexpr (VCS) g0 = wave_search(0, a.n_groups, q, lane, [&](int x) { return a.vptr[x]; });
        int s0 = wave_search(0, a.n_slices, g0, lane, [&](int x) { return a.sptr[x]; });
        // lanes of a window: group starts gs and values gv (for CSR, gv is
        // the entry's own value), slice starts ss, entry indices ix
        int gs = 0, ss, ix;
        T gv;
        auto load = [&](int q_, int g0_, int s0_, int &gs_, T &gv_, int &ss_, int &ix_) {
            if constexpr (VCS) {
                gs_ = a.vptr[lane < a.n_groups - g0_ ? g0_ + lane : a.n_groups];
                gv_ = vals[lane < a.n_groups - g0_ ? g0_ + lane : a.n_groups - 1];
            } else {
                gv_ = vals[lane < nnz - q_ ? q_ + lane : nnz - 1];
            }
            ss_ = a.sptr[lane < a.n_slices - s0_ ? s0_ + lane : a.n_slices];
            ix_ = a.idx[lane < nnz - q_ ? q_ + lane : nnz - 1];
        };
        load(q, g0, s0, gs, gv, ss, ix);
        while (q < qend) {
            // The window: entries whose group (VCS) has a held end and lies in
            // one of the held slices s0 .. s0 + 62. It may be empty when many
            // empty groups or slices pile up at q; then only g0 or s0 moves.
            const int ss_last = readlane(ss, 63);
            const int lim = qend - q < 64 ? qend : q + 64;
            int J, qe;
            if constexpr (VCS) {
                J = uni(max(0, min(63, ss_last - g0)));
                qe = uni(min(lim, readlane(gs, J)));
            } else {
                J = uni(max(0, min(64, ss_last - q)));
                qe = uni(min(lim, q + J));
            }
            const int n = uni(max(qe - q, 0));
            // the next window's first group and slice, from the held lanes
            const int qn = q + n;
            int g0n = qn;
            if constexpr (VCS) g0n = uni(g0 + __popcll(__ballot(gs <= qn)) - 1);
            const int s0n = uni(s0 + __popcll(__ballot(ss <= g0n)) - 1);
            int gs2 = 0, ss2, ix2;
            T gv2;
            if (n == 0) {
                load(qn, g0n, s0n, gs2, gv2, ss2, ix2);
            } else {
                // each lane's entry: its group (largest j < J with gs_j <= p)
                // and its slice (largest t with ss_t <= its group); a window
                // inside one group or one slice skips that search
                const int p = q + lane;
                T v = gv;
                int g = p, g_last = qe - 1;
                if constexpr (VCS) {
                    int j = 0;
                    if (readlane(gs, 1) < qe) {
#pragma unroll
                        for (int st = 32; st; st >>= 1) {
                            const int c = j + st;
                            const int x = __shfl(gs, c & 63);
                            if (c < J && x <= p) j = c;
                        }
                    }
                    v = __shfl(gv, j);
                    g = g0 + j;
                    g_last = uni(g0 + __popcll(__ballot(gs <= qe - 1)) - 1);
                }
                int t = 0;
                if (readlane(ss, 1) <= g_last) {
#pragma unroll
                    for (int st = 32; st; st >>= 1) {
                        const int c = t + st;
                        const int x = __shfl(ss, c & 63);
                        if (x <= g) t = c;
                    }
                }
                const int s = lane < n ? s0 + t : s0;  // a real slice on every lane
                // rounds: lane group k adds in round r the entry of its lane r
                const int nr = min(WW, n);  // rounds with any entry
                const int my_n = n - slot * WW;  // entries of this lane group
                for (int c0 = 0; c0 < w; c0 += WW) {
                    const int col = c0 + cl;
                    const bool act = col < w;
                    if constexpr (LOG_WW <= 4) {
                        T b[WW];
                        static_for(std::make_integer_sequence<int, WW>{}, [&](auto rc) {
                            constexpr int r = decltype(rc)::value;
                            if (r < nr) {
                                const int se = bcast<LOG_WW, r>(s);
                                const bool ok = r < my_n && act;
                                b[r] = a.B[ok ? size_t(se) * w + col : 0];
                            }
                        });
                        if (c0 == 0) load(qn, g0n, s0n, gs2, gv2, ss2, ix2);
                        static_for(std::make_integer_sequence<int, WW>{}, [&](auto rc) {
                            constexpr int r = decltype(rc)::value;
                            if (r < nr) {
                                const int i = bcast<LOG_WW, r>(ix);
                                const T vr = bcast<LOG_WW, r>(v);
                                if (r < my_n && act) {
                                    if constexpr (PRIV) atomicAdd(dst + size_t(i) * w + col, vr * b[r]);
                                    else atomic_add_t(dst + size_t(i) * w + col, vr * b[r]);
                                }
                            }
                        });
                    } else {
                        // 32 or 64 lanes per entry: batches of 16 rounds
                        for (int r0 = 0; r0 < nr; r0 += 16) {
                            T b[16];
#pragma unroll
                            for (int k = 0; k < 16; ++k) {
                                const int r = r0 + k;
                                if (r < nr) {
                                    const int se = bcast_rt<LOG_WW>(s, r);
                                    const bool ok = r < my_n && act;
                                    b[k] = a.B[ok ? size_t(se) * w + col : 0];
                                }
                            }
                            if (c0 == 0 && r0 == 0) load(qn, g0n, s0n, gs2, gv2, ss2, ix2);
#pragma unroll
                            for (int k = 0; k < 16; ++k) {
                                const int r = r0 + k;
                                if (r < nr) {
                                    const int i = bcast_rt<LOG_WW>(ix, r);
                                    const T vr = bcast_rt<LOG_WW>(v, r);
                                    if (r < my_n && act) {
                                        if constexpr (PRIV) atomicAdd(dst + size_t(i) * w + col, vr * b[k]);
                                        else atomic_add_t(dst + size_t(i) * w + col, vr * b[k]);
                                    }
                                }
                            }
                        }
                    }
                }
            }
            q = qn;
            g0 = g0n;
            s0 = s0n;
            gs = gs2;
            gv = gv2;
            ss = ss2;
            ix = ix2;
        }
    }
    if constexpr (PRIV) {
        __syncthreads();
        for (size_t k = threadIdx.x; k < n_el; k += blockDim.x) {
            const T x = priv[k];
            if (x != T(0)) atomic_add_t(a.out + k, x);
        }
    }
}

}  // namespace

template <bool VCS, typename T>
void launch_scatter(const Plan &pl, const ScatterArgs<T> &a, hipStream_t s) {
    if (a.nnz <= 0 || a.w <= 0) return;
    const dim3 g(pl.grid), b(pl.block);
#define VSPMM_SCATTER(L, P)                                                                   \
    do {                                                                                      \
        if (P) allow_lds(reinterpret_cast<const void *>(&k_scatter<VCS, T, L, P, VP>));      \
        hipLaunchKernelGGL((k_scatter<VCS, T, L, P, VP>), g, b, P ? pl.lds_bytes : 0, s, a,  \
                           vals);                                                             \
    } while (0)
#define VSPMM_SCATTER_L(L)                                                                    \
    case L:                                                                                   \
        if (pl.lds) VSPMM_SCATTER(L, true);                                                   \
        else VSPMM_SCATTER(L, false);                                                         \
        break
    with_vals<T>(a, [&](auto vals) {
        using VP = decltype(vals);
        switch (pl.sp.log_ww) {
            VSPMM_SCATTER_L(0);
            VSPMM_SCATTER_L(1);
            VSPMM_SCATTER_L(2);
            VSPMM_SCATTER_L(3);
            VSPMM_SCATTER_L(4);
            VSPMM_SCATTER_L(5);
            default: VSPMM_SCATTER_L(6);
        }
    });
#undef VSPMM_SCATTER_L
#undef VSPMM_SCATTER
}

template void launch_scatter<true, float>(const Plan &, const ScatterArgs<float> &, hipStream_t);
template void launch_scatter<false, float>(const Plan &, const ScatterArgs<float> &, hipStream_t);
template void launch_scatter<false, double>(const Plan &, const ScatterArgs<double> &, hipStream_t);

}  // namespace vspmm
