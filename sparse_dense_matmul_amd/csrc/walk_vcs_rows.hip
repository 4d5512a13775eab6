// Launcher of k_vcs_rows (short VCS slices, float). Built once per VEC (1, 2
// and 4, set by -DVSPMM_VEC), each object holding that VEC's instances.
#include "launch.hpp"
#include "walk_vcs.hpp"

#ifndef VSPMM_VEC
#error "build with -DVSPMM_VEC=1, 2 or 4"
#endif

namespace vspmm {

template <int VEC>
void launch_vcs_rows(const Plan &pl, const WalkArgs<float> &a, hipStream_t s) {
    const dim3 g(pl.grid), b(pl.block);
#define VSPMM_VROWS(LW)                                                                          \
    do {                                                                                         \
        if (pl.lds) {                                                                            \
            allow_lds(reinterpret_cast<const void *>(&k_vcs_rows<LW, true, VEC>));               \
            hipLaunchKernelGGL((k_vcs_rows<LW, true, VEC>), g, b, pl.lds_bytes, s, a.n_slices,   \
                               a.sptr, a.vptr, a.vals, a.idx, a.B, a.out, a.w, a.n_in, a.tiles,   \
                               a.n_b_rows);                                                 \
        } else {                                                                                 \
            hipLaunchKernelGGL((k_vcs_rows<LW, false, VEC>), g, b, pl.lds_bytes, s, a.n_slices,  \
                               a.sptr, a.vptr, a.vals, a.idx, a.B, a.out, a.w, a.n_in, a.tiles,   \
                               a.n_b_rows);                                                 \
        }                                                                                        \
    } while (0)
    switch (pl.sp.log_ww) {
        case 0: VSPMM_VROWS(0); break;
        case 1: VSPMM_VROWS(1); break;
        case 2: VSPMM_VROWS(2); break;
        case 3: VSPMM_VROWS(3); break;
        case 4: VSPMM_VROWS(4); break;
        case 5: VSPMM_VROWS(5); break;
        default: VSPMM_VROWS(6); break;
    }
#undef VSPMM_VROWS
}

template void launch_vcs_rows<VSPMM_VEC>(const Plan &, const WalkArgs<float> &, hipStream_t);

}  // namespace vspmm
