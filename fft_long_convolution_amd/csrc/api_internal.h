// api_internal.h -- entry-point internals shared by lconv_api.cpp and noalloc.hip.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "lconv.h"

namespace lcv {

// lconv_fftconv_fwd with the multi-pass chunks limited to `chunk_target` workspace bytes.
// With may_build = false the constant tables are looked up, never built (a missing one gives
// LCONV_ERR_NOT_PREPARED before any launch), so the call allocates nothing.
lconv_status_t fftconv_fwd_call(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                void* workspace, size_t workspace_bytes, size_t chunk_target, bool may_build,
                                hipStream_t stream);

// Workspace bytes the forward call stages ragged rows in (0 when N is a multiple of 8 or the
// arguments are invalid).
size_t fftconv_fwd_staging_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype);

// Builds the forward call's constant tables for length N on the current device.
lconv_status_t prepare_tables(int64_t N, lconv_dtype_t dtype);

}  // namespace lcv
