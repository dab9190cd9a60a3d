// fused1d_save.hip -- instantiations of the fused 1D kernels for the convolution mode that also
// stores the pre-gate output (kernels in fused1d_kernels.h).
#include "fused1d_kernels.h"

namespace lcv {

hipError_t launch_fused1d_save(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                               hipStream_t st) {
    return for_r(R, [&](auto r) {
        constexpr int RR = decltype(r)::value;
        if (dtype == CT_F32) return launch_conv<RR, CT_F32, MODE_SAVE>(gq, gv, a, cus, st);
        if (dtype == CT_F16) return launch_conv<RR, CT_F16, MODE_SAVE>(gq, gv, a, cus, st);
        return launch_conv<RR, CT_BF16, MODE_SAVE>(gq, gv, a, cus, st);
    });
}

}  // namespace lcv
