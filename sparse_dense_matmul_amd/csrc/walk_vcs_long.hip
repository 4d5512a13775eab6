// Launcher of k_vcs_long (long VCS slices, float). Built once per VEC (1, 2
// and 4, set by -DVSPMM_VEC), each object holding that VEC's instances.
#include "launch.hpp"
#include "walk_vcs.hpp"

#ifndef VSPMM_VEC
#error "build with -DVSPMM_VEC=1, 2 or 4"
#endif

namespace vspmm {

template <int VEC>
void launch_vcs_long(const Plan &pl, const WalkArgs<float> &a, hipStream_t s) {
    const dim3 g(pl.grid), b(pl.block);
#define VSPMM_VLONG(LW)                                                                          \
    hipLaunchKernelGGL((k_vcs_long<LW, VEC>), g, b, 0, s, a.n_slices, a.sptr, a.vptr, a.vals,    \
                       a.idx, a.B, a.out, a.w, pl.wps)
    switch (pl.sp.log_ww) {
        case 0: VSPMM_VLONG(0); break;
        case 1: VSPMM_VLONG(1); break;
        case 2: VSPMM_VLONG(2); break;
        case 3: VSPMM_VLONG(3); break;
        case 4: VSPMM_VLONG(4); break;
        case 5: VSPMM_VLONG(5); break;
        default: VSPMM_VLONG(6); break;
    }
#undef VSPMM_VLONG
}

template void launch_vcs_long<VSPMM_VEC>(const Plan &, const WalkArgs<float> &, hipStream_t);

}  // namespace vspmm
