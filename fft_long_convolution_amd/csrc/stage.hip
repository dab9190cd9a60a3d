// stage.hip -- row staging for sequence lengths that are not a multiple of 8: copies of
// [rows][N] into [rows][N8] with a zero tail (N8 = N rounded up to 8) and back.  The fused and
// multi-pass kernels move 8 elements per access, which needs rows of whole 16-byte groups; a
// causal convolution's first N outputs do not depend on inputs or taps past N, so the zero tail
// changes nothing.  Elements are copied as raw 2- or 4-byte words (zero bits are 0.0 in every
// supported type).  Also the elementwise product that gives the v-gradient from a saved
// pre-gate output, a zero fill and a row-prefix copy.
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

// Time reversal within rows, for the gradients of long sequences: the correlation sums of the
// gradient are causal convolutions of reversed rows (dx = rev(k * rev(ds)), and
// dk[t] = (x * rev(ds))[N-1-t]).  Rows are [rows][N] with N a multiple of 8; thread g handles
// the 8-element group g of the output, whose sources are the mirrored group, reversed.

// out = rev(a (.) b)   (b optional)
template <int IO>
__global__ void __launch_bounds__(256) rev_gate_kernel(const void* a, const void* b, void* out, int64_t rows,
                                                       int64_t N) {
    const int64_t gpr = N / 8, total = rows * gpr;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t r = g / gpr, j = g - r * gpr, src = r * N + 8 * (gpr - 1 - j);
        float x[8], w[8], o[8];
        ld8<IO>(a, src, x);
        if (b) {
            ld8<IO>(b, src, w);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] *= w[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = x[7 - i];
        st8<IO>(out, r * N + 8 * j, o);
    }
}

// d1 = g1 (.) rev(t), d2 = g2 (.) rev(t)   (g1 optional: d1 = rev(t); d2 only when set)
template <int IO>
__global__ void __launch_bounds__(256) rev_gated_out_kernel(const void* t, const void* g1, const void* g2, void* d1,
                                                            void* d2, int64_t rows, int64_t N) {
    const int64_t gpr = N / 8, total = rows * gpr;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t r = g / gpr, j = g - r * gpr, dst = r * N + 8 * j;
        float x[8], rt[8], w[8];
        ld8<IO>(t, r * N + 8 * (gpr - 1 - j), x);
#pragma unroll
        for (int i = 0; i < 8; ++i) rt[i] = x[7 - i];
        if (d2) {
            ld8<IO>(g2, dst, w);
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] *= rt[i];
            st8<IO>(d2, dst, w);
        }
        if (g1) {
            ld8<IO>(g1, dst, w);
#pragma unroll
            for (int i = 0; i < 8; ++i) rt[i] *= w[i];
        }
        st8<IO>(d1, dst, rt);
    }
}

// dk[h][t] = sum_b r[b][h][N-1-t] (fp32, ascending b), dD[h] = dk[h][0]   (either may be null)
template <int IO>
__global__ void __launch_bounds__(256) rev_batch_sum_kernel(const void* rr, float* dk, float* dD, int64_t B,
                                                            int64_t H, int64_t N) {
    const int64_t gpr = N / 8, total = H * gpr;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t h = g / gpr, j = g - h * gpr;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t b = 0; b < B; ++b) {
            float x[8];
            ld8<IO>(rr, (b * H + h) * N + 8 * (gpr - 1 - j), x);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += x[7 - i];
        }
        if (dk) {
            float4* o = (float4*)(dk + h * N + 8 * j);
            o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
        if (dD && j == 0) dD[h] = acc[0];
    }
}

// The lag-0 filter gradient directly, in fp32: dD[h] = sum_b sum_t (q u)[b][h][t] (dy v)[b][h][t]
// (absent gates are 1).  Part 1: workgroup (s, h) sums slice s of the S slices of channel h's rows.
template <int IO>
__global__ void __launch_bounds__(256) dot_part_kernel(const void* u, const void* q, const void* dy, const void* v,
                                                       float* part, int64_t B, int64_t H, int64_t N, int S) {
    const int64_t h = blockIdx.y, s = blockIdx.x, gpr = N / 8;
    const int64_t g0 = gpr * s / S, g1 = gpr * (s + 1) / S;
    float acc = 0.f;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t base = (b * H + h) * N;
        for (int64_t gi = g0 + threadIdx.x; gi < g1; gi += 256) {
            float x[8], e[8], t[8];
            ld8<IO>(u, base + 8 * gi, x);
            ld8<IO>(dy, base + 8 * gi, e);
            if (q) {
                ld8<IO>(q, base + 8 * gi, t);
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] *= t[i];
            }
            if (v) {
                ld8<IO>(v, base + 8 * gi, t);
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] *= t[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf(x[i], e[i], acc);
        }
    }
    __shared__ float red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[h * S + s] = red[0];
}

// Part 2: dD[h] = sum of the S partial sums (ascending s), also stored as dk[h][0].
__global__ void __launch_bounds__(256) dot_final_kernel(const float* part, float* dk, float* dD, int64_t H,
                                                        int64_t N, int S) {
    for (int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x; h < H; h += (int64_t)gridDim.x * 256) {
        float a = 0.f;
        for (int s = 0; s < S; ++s) a += part[h * S + s];
        if (dD) dD[h] = a;
        if (dk) dk[h * N] = a;
    }
}

// dst[r][t] = src[r][t] for t < min(N, L), 0 for N <= t < L: the first L lags of fp32 rows of
// length N (a short filter's gradient from the full-length correlation)
__global__ void __launch_bounds__(256) copy_cols_kernel(const float* src, float* dst, int64_t rows, int64_t N,
                                                        int64_t L) {
    const int64_t total = rows * L;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / L, t = i - r * L;
        dst[i] = t < N ? src[r * N + t] : 0.f;
    }
}

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

unsigned grid_groups(int64_t groups) {
    const int64_t b = (groups + 255) / 256;
    return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t launch_rev_gate(const void* a, const void* b, void* out, int64_t rows, int64_t N, int dtype,
                           hipStream_t st) {
    if (rows <= 0 || N <= 0) return hipSuccess;
    if (N % 8 != 0) return hipErrorInvalidValue;
    const dim3 grid(grid_groups(rows * (N / 8)));
    if (dtype == CT_F32) hipLaunchKernelGGL(rev_gate_kernel<CT_F32>, grid, dim3(256), 0, st, a, b, out, rows, N);
    else if (dtype == CT_F16) hipLaunchKernelGGL(rev_gate_kernel<CT_F16>, grid, dim3(256), 0, st, a, b, out, rows, N);
    else hipLaunchKernelGGL(rev_gate_kernel<CT_BF16>, grid, dim3(256), 0, st, a, b, out, rows, N);
    return hipGetLastError();
}

hipError_t launch_rev_gated_out(const void* t, const void* g1, const void* g2, void* d1, void* d2, int64_t rows,
                                int64_t N, int dtype, hipStream_t st) {
    if (rows <= 0 || N <= 0) return hipSuccess;
    if (N % 8 != 0) return hipErrorInvalidValue;
    const dim3 grid(grid_groups(rows * (N / 8)));
    if (dtype == CT_F32)
        hipLaunchKernelGGL(rev_gated_out_kernel<CT_F32>, grid, dim3(256), 0, st, t, g1, g2, d1, d2, rows, N);
    else if (dtype == CT_F16)
        hipLaunchKernelGGL(rev_gated_out_kernel<CT_F16>, grid, dim3(256), 0, st, t, g1, g2, d1, d2, rows, N);
    else
        hipLaunchKernelGGL(rev_gated_out_kernel<CT_BF16>, grid, dim3(256), 0, st, t, g1, g2, d1, d2, rows, N);
    return hipGetLastError();
}

hipError_t launch_rev_batch_sum(const void* r, float* dk, float* dD, int64_t B, int64_t H, int64_t N, int dtype,
                                hipStream_t st) {
    if (H <= 0 || N <= 0) return hipSuccess;
    if (N % 8 != 0) return hipErrorInvalidValue;
    const dim3 grid(grid_groups(H * (N / 8)));
    if (dtype == CT_F32) hipLaunchKernelGGL(rev_batch_sum_kernel<CT_F32>, grid, dim3(256), 0, st, r, dk, dD, B, H, N);
    else if (dtype == CT_F16) hipLaunchKernelGGL(rev_batch_sum_kernel<CT_F16>, grid, dim3(256), 0, st, r, dk, dD, B, H, N);
    else hipLaunchKernelGGL(rev_batch_sum_kernel<CT_BF16>, grid, dim3(256), 0, st, r, dk, dD, B, H, N);
    return hipGetLastError();
}

hipError_t launch_dot_lag0(const void* u, const void* q, const void* dy, const void* v, float* part, float* dk,
                           float* dD, int64_t B, int64_t H, int64_t N, int dtype, hipStream_t st) {
    if (H <= 0 || N <= 0 || (!dk && !dD)) return hipSuccess;
    if (N % 8 != 0 || H > 65535) return hipErrorInvalidValue;
    const int S = dot_slices(N);
    const dim3 grid((unsigned)S, (unsigned)H);
    if (dtype == CT_F32) hipLaunchKernelGGL(dot_part_kernel<CT_F32>, grid, dim3(256), 0, st, u, q, dy, v, part, B, H, N, S);
    else if (dtype == CT_F16) hipLaunchKernelGGL(dot_part_kernel<CT_F16>, grid, dim3(256), 0, st, u, q, dy, v, part, B, H, N, S);
    else hipLaunchKernelGGL(dot_part_kernel<CT_BF16>, grid, dim3(256), 0, st, u, q, dy, v, part, B, H, N, S);
    hipLaunchKernelGGL(dot_final_kernel, dim3(grid_groups(H)), dim3(256), 0, st, part, dk, dD, H, N, S);
    return hipGetLastError();
}

hipError_t launch_copy_cols(const float* src, float* dst, int64_t rows, int64_t N, int64_t L, hipStream_t st) {
    if (rows <= 0 || L <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_cols_kernel, dim3(grid_for(rows * L)), dim3(256), 0, st, src, dst, rows, N, L);
    return hipGetLastError();
}

hipError_t launch_zero_words(void* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(n)), dim3(256), 0, st, (uint32_t*)p, n);
    return hipGetLastError();
}

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
