// Launcher of k_short (short CSR slices). Built once per element type
// (-DVSPMM_ELT=float or double), each object holding that type's instances.
#include <algorithm>

#include "launch.hpp"
#include "walk_fast.hpp"

#ifndef VSPMM_ELT
#error "build with -DVSPMM_ELT=float or double"
#endif

namespace vspmm {

namespace {

// With long blocks, the grid grows by them and the dynamic LDS holds at least
// their partial rows (kLongWaves x NC*64*VEC elements per group of waves).
template <typename T, int VEC, int NC>
void launch_short_nc(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    const dim3 g(pl.grid + a.long_blocks), b(pl.block);
    size_t lds = pl.lds_bytes;
    if (a.long_blocks > 0)
        lds = std::max(lds, size_t(pl.block / (64 * kLongWaves)) * kLongWaves * NC * 64 * VEC *
                                sizeof(T));
    with_vals<T>(a, [&](auto vals) {
        using VP = decltype(vals);
        if (pl.lds) {
            allow_lds(reinterpret_cast<const void *>(&k_short<false, T, VEC, true, NC, VP>));
            hipLaunchKernelGGL((k_short<false, T, VEC, true, NC, VP>), g, b, lds, s, a.n_slices,
                               a.sptr, a.vptr, vals, a.idx, a.B, a.out, a.w, a.n_in, pl.sp,
                               a.long_list ? 1 : 0, a.long_len, a.parts, a.n_parts, a.long_list,
                               a.n_long, a.long_blocks, pl.ring);
        } else {
            hipLaunchKernelGGL((k_short<false, T, VEC, false, NC, VP>), g, b, lds, s, a.n_slices,
                               a.sptr, a.vptr, vals, a.idx, a.B, a.out, a.w, a.n_in, pl.sp,
                               a.long_list ? 1 : 0, a.long_len, a.parts, a.n_parts, a.long_list,
                               a.n_long, a.long_blocks, pl.ring);
        }
    });
}

// Width chunks walked together: the power of two (at most 4) that comes
// closest to covering the width in one walk.
template <typename T, int VEC>
void launch_short_v(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    const int chunk = VEC << pl.sp.log_ww;
    const int n_chunks = (a.w + chunk - 1) / chunk;
    if (n_chunks >= 4) launch_short_nc<T, VEC, 4>(pl, a, s);
    else if (n_chunks >= 2) launch_short_nc<T, VEC, 2>(pl, a, s);
    else launch_short_nc<T, VEC, 1>(pl, a, s);
}

}  // namespace

template <typename T>
void launch_short(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    if constexpr (sizeof(T) == 4) {
        if (pl.vec == 4) return launch_short_v<T, 4>(pl, a, s);
    }
    if (pl.vec == 2) return launch_short_v<T, 2>(pl, a, s);
    launch_short_v<T, 1>(pl, a, s);
}

template void launch_short<VSPMM_ELT>(const Plan &, const WalkArgs<VSPMM_ELT> &, hipStream_t);

}  // namespace vspmm
