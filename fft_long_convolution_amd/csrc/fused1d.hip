// fused1d.hip -- instantiations of the fused 1D kernels for the filter, row and row-forward modes, and the mode dispatcher (kernels in fused1d_kernels.h).
#include "fused1d_kernels.h"

namespace lcv {

template <int R>
static hipError_t launch_misc(int dtype, int mode, const Fused1DArgs& a, int cus, hipStream_t st) {
    if (mode == MODE_FILTER) {
        if (dtype == CT_F32) return launch_t<R, CT_F32, CT_F32, MODE_FILTER, false, false>(a, cus, st);
        if (dtype == CT_F16) return launch_t<R, CT_F32, CT_F16, MODE_FILTER, false, false>(a, cus, st);
        return launch_t<R, CT_F32, CT_BF16, MODE_FILTER, false, false>(a, cus, st);
    }
    if constexpr (R == 32) {
        if (mode == MODE_ROW) {
            if (dtype == CT_F32) return launch_t<32, CT_F32, CT_F32, MODE_ROW, false, false>(a, cus, st);
            // 16-bit: the pipelined kernel's row variant
            if (dtype == CT_F16) return launch_8k<CT_F16, false, false, false, false, true>(a, cus, st);
            return launch_8k<CT_BF16, false, false, false, false, true>(a, cus, st);
        }
        if (mode == MODE_ROWFWD) {
            if (dtype == CT_F32) return launch_t<32, CT_F32, CT_F32, MODE_ROWFWD, false, false>(a, cus, st);
            if (dtype == CT_F16) return launch_t<32, CT_F32, CT_F16, MODE_ROWFWD, false, false>(a, cus, st);
            return launch_t<32, CT_F32, CT_BF16, MODE_ROWFWD, false, false>(a, cus, st);
        }
        if (mode == MODE_ROWFWD16) {
            if (dtype == CT_F16) return launch_t<32, CT_F16, CT_F16, MODE_ROWFWD, false, false>(a, cus, st);
            if (dtype == CT_BF16) return launch_t<32, CT_BF16, CT_BF16, MODE_ROWFWD, false, false>(a, cus, st);
            return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fused1d(int R, int dtype, int mode, bool gq, bool gv, const Fused1DArgs& a, int cus,
                          hipStream_t stream) {
    switch (mode) {
    case MODE_CONV: return launch_fused1d_conv(R, dtype, gq, gv, a, cus, stream);
    case MODE_ADJ: return launch_fused1d_adj(R, dtype, gq, gv, a, cus, stream);
    case MODE_PART: return launch_fused1d_part(R, dtype, gq, gv, a, cus, stream);
    case MODE_SPARSE: return launch_fused1d_sparse(R, dtype, gq, gv, a, cus, stream);
    case MODE_SAVE: return launch_fused1d_save(R, dtype, gq, gv, a, cus, stream);
    case MODE_LBF: return launch_fused1d_lbf(R, dtype, gq, gv, a, cus, stream);
    default:
        return for_r(R, [&](auto r) { return launch_misc<decltype(r)::value>(dtype, mode, a, cus, stream); });
    }
}

}  // namespace lcv
