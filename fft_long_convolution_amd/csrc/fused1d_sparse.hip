// fused1d_sparse.hip -- instantiations of the fused 1D kernels for the frequency-sparse mode
// (kernels in fused1d_kernels.h).
#include "fused1d_kernels.h"

namespace lcv {

hipError_t launch_fused1d_sparse(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                                 hipStream_t st) {
    return for_r(R, [&](auto r) {
        constexpr int RR = decltype(r)::value;
        if (dtype == CT_F32) return launch_sparse<RR, CT_F32>(gq, gv, a, cus, st);
        if (dtype == CT_F16) return launch_sparse<RR, CT_F16>(gq, gv, a, cus, st);
        return launch_sparse<RR, CT_BF16>(gq, gv, a, cus, st);
    });
}

}  // namespace lcv
