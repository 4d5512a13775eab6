// Launcher of k_long (long CSR slices, a block per slice).
#include "launch.hpp"
#include "walk_fast.hpp"

namespace vspmm {

template <bool VCS, typename T, int VEC>
void launch_long_v(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    const dim3 g(pl.grid), b(pl.block);
    // width chunks per walk of a piece: the power of two (at most 4) that
    // comes closest to covering the width in one walk
    const int chunk = VEC << pl.sp.log_ww;
    const int n_chunks = (a.w + chunk - 1) / chunk;
#define VSPMM_LONG(NC)                                                                           \
    hipLaunchKernelGGL((k_long<VCS, T, VEC, NC, decltype(vals)>), g, b, 0, s, a.n_slices, a.sptr, \
                       a.vptr, vals, a.idx, a.B, a.out, a.w, pl.sp, a.long_list, a.n_long, pl.wps)
    with_vals<T>(a, [&](auto vals) {
        if (n_chunks >= 4) VSPMM_LONG(4);
        else if (n_chunks >= 2) VSPMM_LONG(2);
        else VSPMM_LONG(1);
    });
#undef VSPMM_LONG
}

template <bool VCS, typename T>
void launch_long(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    if constexpr (sizeof(T) == 4) {
        if (pl.vec == 4) return launch_long_v<VCS, T, 4>(pl, a, s);
    }
    if (pl.vec == 2) return launch_long_v<VCS, T, 2>(pl, a, s);
    launch_long_v<VCS, T, 1>(pl, a, s);
}

template void launch_long<false, float>(const Plan &, const WalkArgs<float> &, hipStream_t);
template void launch_long<false, double>(const Plan &, const WalkArgs<double> &, hipStream_t);

}  // namespace vspmm
