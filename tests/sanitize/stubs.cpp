// Host-only stand-ins for the device launchers, so the C ABI's host code (argument checks, plans,
// workspace layouts, dispatch) can be built with the address and undefined-behaviour sanitizers
// without device code.  Each returns an error, as a failed launch would.
#include "kernels.h"

namespace lcv {
#define LCV_STUB(sig) sig { return hipErrorInvalidValue; }
LCV_STUB(hipError_t launch_fused1d(int, int, int, bool, bool, const Fused1DArgs&, int, hipStream_t))
LCV_STUB(hipError_t launch_dk1d(int, int, bool, bool, const Fused1DArgs&, int, hipStream_t))
LCV_STUB(hipError_t launch_col_fwd(int, const ColArgs&, hipStream_t))
LCV_STUB(hipError_t launch_col_inv(int, const ColArgs&, hipStream_t))
LCV_STUB(hipError_t launch_conv2d(int, const Conv2DArgs&, hipStream_t))
LCV_STUB(hipError_t launch_conv3d(int, const Conv3DArgs&, hipStream_t))
LCV_STUB(hipError_t launch_mul_rows(const void*, const void*, void*, int64_t, int, hipStream_t))
LCV_STUB(hipError_t launch_pad_rows(const void*, void*, int64_t, int64_t, int64_t, int, hipStream_t))
LCV_STUB(hipError_t launch_unpad_rows(const void*, void*, int64_t, int64_t, int64_t, int, hipStream_t))
LCV_STUB(hipError_t launch_rev_gate(const void*, const void*, void*, int64_t, int64_t, int, hipStream_t))
LCV_STUB(hipError_t launch_rev_gated_out(const void*, const void*, const void*, void*, void*, int64_t, int64_t,
                                         int, hipStream_t))
LCV_STUB(hipError_t launch_rev_batch_sum(const void*, float*, float*, int64_t, int64_t, int64_t, int, hipStream_t))
LCV_STUB(hipError_t launch_zero_words(void*, int64_t, hipStream_t))
LCV_STUB(hipError_t launch_copy_cols(const float*, float*, int64_t, int64_t, int64_t, hipStream_t))
LCV_STUB(hipError_t launch_adj2d(const void*, void*, int64_t, hipStream_t))
LCV_STUB(hipError_t launch_dk2d_sum(int, const void*, float*, int64_t, int64_t, int, int, hipStream_t))
LCV_STUB(hipError_t launch_dd2d(int, const void*, const void*, float*, int64_t, int64_t, int64_t, hipStream_t))
LCV_STUB(hipError_t launch_dot_lag0(const void*, const void*, const void*, const void*, float*, float*, float*, int64_t,
                                    int64_t, int64_t, int, hipStream_t))
LCV_STUB(hipError_t launch_bfly_images(const void*, void*, int, int, const FusedTableLayout&, hipStream_t))
LCV_STUB(hipError_t launch_ssm_prepare(int, const float*, const float*, const SsmArgs&, hipStream_t))
LCV_STUB(hipError_t launch_ssm_state(int, const SsmArgs&, bool, bool, hipStream_t))
#undef LCV_STUB
}  // namespace lcv
