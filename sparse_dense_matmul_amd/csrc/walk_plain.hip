// Launcher of the plain aligned walk (k_aligned).
#include "launch.hpp"
#include "walk.hpp"

namespace vspmm {

template <bool VCS, typename T>
void launch_plain(const Plan &pl, const WalkArgs<T> &a, hipStream_t s) {
    const dim3 g(pl.grid), b(pl.block);
    // a slice per wave (R == 1) lets VCS walks keep the slice bounds uniform
#define VSPMM_PLAIN(V, U)                                                                        \
    hipLaunchKernelGGL((k_aligned<VCS, T, V, U, decltype(vals)>), g, b, 0, s, a.n_slices, a.sptr, \
                       a.vptr, vals, a.idx, a.B, a.out, a.w, pl.sp, a.long_len)
#define VSPMM_PLAIN_V(V)                                                                         \
    do {                                                                                         \
        if (VCS && pl.R == 1) VSPMM_PLAIN(V, VCS);                                               \
        else VSPMM_PLAIN(V, false);                                                              \
    } while (0)
    with_vals<T>(a, [&](auto vals) {
        if constexpr (sizeof(T) == 4) {
            if (pl.vec == 4) {
                VSPMM_PLAIN_V(4);
                return;
            }
        }
        if (pl.vec == 2) VSPMM_PLAIN_V(2);
        else VSPMM_PLAIN_V(1);
    });
#undef VSPMM_PLAIN_V
#undef VSPMM_PLAIN
}

template void launch_plain<true, float>(const Plan &, const WalkArgs<float> &, hipStream_t);
template void launch_plain<false, float>(const Plan &, const WalkArgs<float> &, hipStream_t);
template void launch_plain<false, double>(const Plan &, const WalkArgs<double> &, hipStream_t);

}  // namespace vspmm
