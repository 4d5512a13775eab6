// Launcher of k_long (long CSR slices, a block per slice).
#include "launch.hpp"
#include "walk_fast.hpp"

namespace vspmm {

template <bool VCS, typename T>
void launch_long(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    const dim3 g(pl.grid), b(pl.block);
#define VSPMM_LONG(V)                                                                            \
    hipLaunchKernelGGL((k_long<VCS, T, V>), g, b, 0, s, a.n_slices, a.sptr, a.vptr, a.vals,      \
                       a.idx, a.B, a.out, a.w, pl.sp, a.long_list, a.n_long)
    if constexpr (sizeof(T) == 4) {
        if (pl.vec == 4) {
            VSPMM_LONG(4);
            return;
        }
    }
    if (pl.vec == 2) VSPMM_LONG(2);
    else VSPMM_LONG(1);
#undef VSPMM_LONG
}

template void launch_long<false, float>(const Plan &, const WalkArgs<float> &, hipStream_t);
template void launch_long<false, double>(const Plan &, const WalkArgs<double> &, hipStream_t);

}  // namespace vspmm
