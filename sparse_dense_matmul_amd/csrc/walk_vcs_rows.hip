// Launcher of the short VCS walks (k_vcs_seg, k_vcs_rows; float). Built once
// per VEC (1, 2 and 4, set by -DVSPMM_VEC), each object holding that VEC's
// instances.
#include "launch.hpp"
#include "walk_seg.hpp"
#include "walk_vcs.hpp"

#ifndef VSPMM_VEC
#error "build with -DVSPMM_VEC=1, 2 or 4"
#endif

namespace vspmm {

template <int VEC>
void launch_vcs_rows(const Plan &pl, const WalkArgs<float> &a, hipStream_t s) {
    // k_vcs_seg (up to 4 width lanes per entry: its steps per window are
    // unrolled) when the walk's per-wave plan is there; k_vcs_rows otherwise
    const bool seg = a.seg && a.he && pl.sp.log_ww <= 2;
    const dim3 g(seg ? a.seg_grid : pl.grid), b(seg ? 64 * a.seg_wpb : pl.block);
    const size_t b_al = pl.lds ? (size_t(a.n_in) * size_t(a.w) * sizeof(float) + 15) & ~size_t(15) : 0;
    const size_t lds = seg ? b_al + size_t(a.seg_wpb) * kRowsWaveLds : pl.lds_bytes;
#define VSPMM_VROWS_K(KERN, LW, ...)                                                             \
    do {                                                                                         \
        if (pl.lds) {                                                                            \
            allow_lds(reinterpret_cast<const void *>(&KERN<LW, true, VEC>));                     \
            hipLaunchKernelGGL((KERN<LW, true, VEC>), g, b, lds, s, a.n_slices, a.sptr, a.vptr,  \
                               a.vals, a.idx, a.B, a.out, a.w, a.n_in, a.tiles,                  \
                               a.n_b_rows __VA_ARGS__);                                          \
        } else {                                                                                 \
            hipLaunchKernelGGL((KERN<LW, false, VEC>), g, b, lds, s, a.n_slices, a.sptr, a.vptr, \
                               a.vals, a.idx, a.B, a.out, a.w, a.n_in, a.tiles,                  \
                               a.n_b_rows __VA_ARGS__);                                          \
        }                                                                                        \
    } while (0)
#define VSPMM_VROWS(LW)                                                                          \
    do {                                                                                         \
        if constexpr (LW <= 2) {                                                                 \
            if (seg) {                                                                           \
                VSPMM_VROWS_K(k_vcs_seg, LW, , a.he, a.seg);                                     \
                break;                                                                           \
            }                                                                                    \
        }                                                                                        \
        VSPMM_VROWS_K(k_vcs_rows, LW);                                                           \
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
#undef VSPMM_VROWS_K
}

template void launch_vcs_rows<VSPMM_VEC>(const Plan &, const WalkArgs<float> &, hipStream_t);

}  // namespace vspmm
