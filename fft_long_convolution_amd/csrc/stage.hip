// stage.hip -- row staging for sequence lengths that are not a multiple of 8: copies of
// [rows][N] into [rows][N8] with a zero tail (N8 = N rounded up to 8) and back.  The fused and
// multi-pass kernels move 8 elements per access, which needs rows of whole 16-byte groups; a
// causal convolution's first N outputs do not depend on inputs or taps past N, so the zero tail
// changes nothing.  Elements are copied as raw 2- or 4-byte words (zero bits are 0.0 in every
// supported type).  Also the elementwise product that gives the v-gradient from a saved
// pre-gate output.
#include "coldft.h"
#include "kernels.h"

namespace lcv {

namespace {

template <typename W>
__global__ void __launch_bounds__(256) pad_rows_kernel(const W* src, W* dst, int64_t rows, int64_t N, int64_t N8) {
    const int64_t total = rows * N8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / N8, c = i - r * N8;
        dst[i] = c < N ? src[r * N + c] : (W)0;
    }
}

template <typename W>
__global__ void __launch_bounds__(256) unpad_rows_kernel(const W* src, W* dst, int64_t rows, int64_t N, int64_t N8) {
    const int64_t total = rows * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / N, c = i - r * N;
        dst[i] = src[r * N8 + c];
    }
}

unsigned grid_for(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

// y = a * b elementwise, 8 elements per thread and step (n8 groups of 8), fp32 arithmetic
template <int IO>
__global__ void __launch_bounds__(256) mul_rows_kernel(const void* a, const void* b, void* y, int64_t n8) {
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n8; g += (int64_t)gridDim.x * 256) {
        float x[8], w[8];
        ld8<IO>(a, 8 * g, x);
        ld8<IO>(b, 8 * g, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] *= w[i];
        st8<IO>(y, 8 * g, x);
    }
}

}  // namespace

hipError_t launch_mul_rows(const void* dy, const void* c, void* y, int64_t n, int dtype, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (n % 8 != 0) return hipErrorInvalidValue;
    const int64_t n8 = n / 8, blocks = (n8 + 255) / 256 < 8192 ? (n8 + 255) / 256 : 8192;
    if (dtype == CT_F32) hipLaunchKernelGGL(mul_rows_kernel<CT_F32>, dim3((unsigned)blocks), dim3(256), 0, st, dy, c, y, n8);
    else if (dtype == CT_F16) hipLaunchKernelGGL(mul_rows_kernel<CT_F16>, dim3((unsigned)blocks), dim3(256), 0, st, dy, c, y, n8);
    else hipLaunchKernelGGL(mul_rows_kernel<CT_BF16>, dim3((unsigned)blocks), dim3(256), 0, st, dy, c, y, n8);
    return hipGetLastError();
}

hipError_t launch_pad_rows(const void* src, void* dst, int64_t rows, int64_t N, int64_t N8, int esize,
                           hipStream_t st) {
    if (esize == 2)
        hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, dim3(grid_for(rows * N8)), dim3(256), 0, st,
                           (const uint16_t*)src, (uint16_t*)dst, rows, N, N8);
    else
        hipLaunchKernelGGL(pad_rows_kernel<uint32_t>, dim3(grid_for(rows * N8)), dim3(256), 0, st,
                           (const uint32_t*)src, (uint32_t*)dst, rows, N, N8);
    return hipGetLastError();
}

hipError_t launch_unpad_rows(const void* src, void* dst, int64_t rows, int64_t N, int64_t N8, int esize,
                             hipStream_t st) {
    if (esize == 2)
        hipLaunchKernelGGL(unpad_rows_kernel<uint16_t>, dim3(grid_for(rows * N)), dim3(256), 0, st,
                           (const uint16_t*)src, (uint16_t*)dst, rows, N, N8);
    else
        hipLaunchKernelGGL(unpad_rows_kernel<uint32_t>, dim3(grid_for(rows * N)), dim3(256), 0, st,
                           (const uint32_t*)src, (uint32_t*)dst, rows, N, N8);
    return hipGetLastError();
}

}  // namespace lcv
