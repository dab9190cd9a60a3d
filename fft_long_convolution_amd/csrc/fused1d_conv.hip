// fused1d_conv.hip -- instantiations of the fused 1D kernels for the convolution mode (kernels in fused1d_kernels.h).
#include "fused1d_kernels.h"

namespace lcv {

hipError_t launch_fused1d_conv(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                               hipStream_t st) {
    return for_r(R, [&](auto r) {
        constexpr int RR = decltype(r)::value;
        if (dtype == CT_F32) return launch_conv<RR, CT_F32, MODE_CONV>(gq, gv, a, cus, st);
        if (dtype == CT_F16) return launch_conv<RR, CT_F16, MODE_CONV>(gq, gv, a, cus, st);
        return launch_conv<RR, CT_BF16, MODE_CONV>(gq, gv, a, cus, st);
    });
}

}  // namespace lcv
