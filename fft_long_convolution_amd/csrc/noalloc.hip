// noalloc.hip -- the set-up call and the forward call for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The forward call's workspace (the multi-pass chunks, and the staging of rows that are not a
// multiple of 8) comes from `scratch`, a static device array: each GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name is only a host-side
// stand-in, not a device address, so the set-up call looks up each device's address once with
// hipGetSymbolAddress, with that device current, and every later use goes through that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "lconv.h"

// The scratch buffer: file scope, one copy per GPU.  Host code never uses this name as an
// address; it goes through the per-device pointer below.
static __device__ __align__(256) unsigned char scratch[LCONV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each GPU's copy; null until set up

lconv_status_t current_device(int* dev) {
    if (hipGetDevice(dev) != hipSuccess) return LCONV_ERR_HIP;
    if (*dev < 0 || *dev >= kMaxDevices) return LCONV_ERR_UNSUPPORTED;
    return LCONV_SUCCESS;
}

// Once per device, with that device current.
lconv_status_t scratch_setup(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch[dev]) return LCONV_SUCCESS;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LCONV_ERR_HIP;
    g_scratch[dev] = ptr;
    return LCONV_SUCCESS;
}

void* scratch_of(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    return g_scratch[dev];
}

}  // namespace

extern "C" {

lconv_status_t lconv_prepare(int64_t N, lconv_dtype_t dtype) {
    int dev = 0;
    lconv_status_t st = current_device(&dev);
    if (st != LCONV_SUCCESS) return st;
    st = lcv::prepare_tables(N, dtype);
    if (st != LCONV_SUCCESS) return st;
    return scratch_setup(dev);
}

lconv_status_t lconv_fftconv_fwd_noalloc(const void* u, const void* k_f, const void* D, void* y,
                                         const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                         lconv_dtype_t dtype, hipStream_t stream) {
    int dev = 0;
    lconv_status_t st = current_device(&dev);
    if (st != LCONV_SUCCESS) return st;
    void* ws = scratch_of(dev);
    if (!ws) return LCONV_ERR_NOT_PREPARED;
    // the staging comes first in the workspace; the multi-pass chunks get the rest
    const size_t cap = LCONV_NOALLOC_SCRATCH_BYTES;
    const size_t stage = lcv::fftconv_fwd_staging_bytes(B, H, N, dtype);
    const size_t target = stage < cap ? cap - stage : 0;
    st = lcv::fftconv_fwd_call(u, k_f, D, y, q, v, B, H, N, dtype, ws, cap, target, false, stream);
    return st == LCONV_ERR_WORKSPACE ? LCONV_ERR_SCRATCH_LIMIT : st;
}

}  // extern "C"
