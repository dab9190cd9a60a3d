// multipass.hip -- column passes of the chunked path for sequences past one workgroup.
//
// "FlashConv" (AIMech page, Mechanism) handles sequences beyond the on-chip capacity in
// chunks; the page's own chunk recursion passes a state-space boundary state, which needs an
// SSM-generated filter, so for arbitrary long filters this path uses the textbook four-step
// split of the same FFT instead (M = M1 x 8192):
//     n = 8192 n_hi + n_lo,   f = k_hi + M1 k_lo
//     X[k_hi + M1 k_lo] = sum_{n_lo} w_8192^{n_lo k_lo} [ w_M^{n_lo k_hi}
//                              sum_{n_hi} w_{M1}^{n_hi k_hi} x[8192 n_hi + n_lo] ].
// Pass A (here): the inner DFT over n_hi (zero for n_hi >= M1/2) and the twiddle.
// Pass B (fused1d.hip, row mode): DFT over n_lo, spectral product, inverse DFT over n_lo.
// Pass C (here): inverse twiddle, inverse DFT over k_hi for n_hi < M1/2 only (the causal
// truncation), gating, store.
//
// A workgroup owns CB consecutive columns of one sequence (all M1 rows).  Global rows are read
// and written 8 columns per 16-byte access; the column DFTs run in LDS (fp32 complex, one
// column-major block) as self-sorting radix-8/4/2 passes (Stockham order: natural order out,
// no bit reversal), each thread doing whole small DFTs in registers.  The n_lo-dependent
// twiddle w_M^{n_lo k_hi} is formed once per 8 columns from the two-level table and advanced
// by w_M^{k_hi} along them.
#include "coldft.h"
#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

namespace {

constexpr int64_t kM2 = 8192;
constexpr int kLdsBytes = 64 * 1024;    // column block: CB x M1 fp32 complex (plus one pad row)

__host__ __device__ constexpr int cols_per_wg(int M1) {
    return kLdsBytes / (8 * M1) < 256 ? kLdsBytes / (8 * M1) : 256;
}

}  // namespace

template <int CT, int IO, int kThreads>
__global__ void __launch_bounds__(kThreads) col_fwd_kernel(const ColArgs a) {
    extern __shared__ float2 buf[];
    // column-major block, column stride M1 + 1: the column passes walk rows of one column
    // (consecutive words), the row-wise load and store see at most 2-way bank conflicts
    const int M1 = (int)a.M1, CB = cols_per_wg(M1), ld = M1 + 1;
    const int64_t s = blockIdx.y, gs = a.seq0 + s;
    const int64_t n_lo0 = (int64_t)blockIdx.x * CB;
    int64_t row0, row1;
    seq_rows(a, gs, row0, row1);
    const int g8 = CB / 8;  // 8-column groups per row
    // load rows n_hi < M1/2 (zero past N), gated, as complex pairs (row b, row b+1)
    for (int it = threadIdx.x; it < (M1 / 2) * g8; it += kThreads) {
        const int nh = it / g8, cg = it % g8;
        const int64_t n = kM2 * nh + n_lo0 + 8 * cg;
        float xr[8], xi[8];
        if (n < a.N) {  // N is a multiple of 8: a group is all in or all out
            ld8<IO>(a.u, row0 + n, xr);
            if (a.q) {
                float t[8];
                ld8<IO>(a.q, row0 + n, t);
#pragma unroll
                for (int k = 0; k < 8; ++k) xr[k] *= t[k];
            }
            if (row1 >= 0) {
                ld8<IO>(a.u, row1 + n, xi);
                if (a.q) {
                    float t[8];
                    ld8<IO>(a.q, row1 + n, t);
#pragma unroll
                    for (int k = 0; k < 8; ++k) xi[k] *= t[k];
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) xi[k] = 0.f;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) xr[k] = xi[k] = 0.f;
        }
        float2* d = buf + 8 * cg * ld + nh;
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k * ld] = make_float2(xr[k], xi[k]);
    }
    __syncthreads();
    column_dft<kThreads, false>(buf, M1, ld, CB, a.tw_col, M1);
    // twiddle w_M^{n_lo k_hi} and store row k_hi, 8 columns per thread
    for (int it = threadIdx.x; it < M1 * g8; it += kThreads) {
        const int kh = it / g8, cg = it % g8;
        const int64_t n_lo = n_lo0 + 8 * cg;
        float2 w = tw_m(a.tw_lo, a.tw_hi, (n_lo * kh) & (a.M - 1));
        const float2 step = ((const float2*)a.tw_lo)[kh];  // kh < 2048
        float2 z[8];
        const float2* src = buf + 8 * cg * ld + kh;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            z[k] = cmulf(src[k * ld], w);
            w = cmulf(w, step);
        }
        ws_st8<CT>(a.ws, (s * a.M1 + kh) * kM2 + n_lo, z);
    }
}

template <int CT, int IO, int kThreads>
__global__ void __launch_bounds__(kThreads) col_inv_kernel(const ColArgs a) {
    extern __shared__ float2 buf[];
    const int M1 = (int)a.M1, CB = cols_per_wg(M1), ld = M1 + 1;  // column-major, as above
    const int64_t s = blockIdx.y, gs = a.seq0 + s;
    const int64_t n_lo0 = (int64_t)blockIdx.x * CB;
    int64_t row0, row1;
    seq_rows(a, gs, row0, row1);
    const int g8 = CB / 8;
    // load rows k_hi, inverse twiddle conj(w_M^{n_lo k_hi})
    for (int it = threadIdx.x; it < M1 * g8; it += kThreads) {
        const int kh = it / g8, cg = it % g8;
        const int64_t n_lo = n_lo0 + 8 * cg;
        float2 w = tw_m(a.tw_lo, a.tw_hi, (n_lo * kh) & (a.M - 1));
        const float2 step = ((const float2*)a.tw_lo)[kh];
        float2 z[8];
        ws_ld8<CT>(a.ws, (s * a.M1 + kh) * kM2 + n_lo, z);
        float2* d = buf + 8 * cg * ld + kh;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            d[k * ld] = cmulcf(z[k], w);
            w = cmulf(w, step);
        }
    }
    __syncthreads();
    column_dft<kThreads, true>(buf, M1, ld, CB, a.tw_col, M1);
    // rows n_hi < M1/2 (and n < N): gate and store
    for (int it = threadIdx.x; it < (M1 / 2) * g8; it += kThreads) {
        const int nh = it / g8, cg = it % g8;
        const int64_t n = kM2 * nh + n_lo0 + 8 * cg;
        if (n >= a.N) continue;
        const float2* src = buf + 8 * cg * ld + nh;
        float yr[8], yi[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            yr[k] = src[k * ld].x;
            yi[k] = src[k * ld].y;
        }
        if (a.v) {
            float t[8];
            ld8<IO>(a.v, row0 + n, t);
#pragma unroll
            for (int k = 0; k < 8; ++k) yr[k] *= t[k];
        }
        st8<IO>(a.y, row0 + n, yr);
        if (row1 >= 0) {
            if (a.v) {
                float t[8];
                ld8<IO>(a.v, row1 + n, t);
#pragma unroll
                for (int k = 0; k < 8; ++k) yi[k] *= t[k];
            }
            st8<IO>(a.y, row1 + n, yi);
        }
    }
}


// ---- short columns (M1 <= 16): one column per thread, DFT in registers ----------------------
// LDS column position of column c in a row of the 256-column block: the three low bits rotated
// by bits 5-7.  A row-wise access of one instruction (thread cg of a row at columns 8 cg + k, k
// fixed) then spreads over all the banks instead of landing every fourth group on the same
// ones; the column-wise access (thread t at column t) stays a permutation inside groups of 8.
__device__ __forceinline__ int col_swz(int c) { return (c & ~7) | ((c + (c >> 5)) & 7); }

// Forward, H = M1/2 nonzero inputs: X[2m + e] = DFT_H( x[n] w_M1^{n e} )[m], e = 0, 1.
// Inverse, outputs n < H only:  y[n] = E[n] + w_M1^{-n} O[n] with E, O the inverse DFT_H of the
// even and odd inputs.  Rows pass through LDS so global rows are read and written 8 columns per
// 16-byte access; each thread then owns one of the 256 columns of the block.
template <int CT, int IO, int M1>
__global__ void __launch_bounds__(256) col_small_fwd_kernel(const ColArgs a) {
    constexpr int H = M1 / 2, CB = 256, LDW = CB + 1;
    __shared__ float2 sin_[H * LDW];
    __shared__ float2 sout[M1 * LDW];
    const int64_t s = blockIdx.y, gs = a.seq0 + s;
    const int64_t n_lo0 = (int64_t)blockIdx.x * CB;
    int64_t row0, row1;
    seq_rows(a, gs, row0, row1);
    constexpr int g8 = CB / 8;
    for (int it = threadIdx.x; it < H * g8; it += 256) {
        const int nh = it / g8, cg = it % g8;
        const int64_t n = kM2 * nh + n_lo0 + 8 * cg;
        float xr[8], xi[8];
        if (n < a.N) {
            ld8<IO>(a.u, row0 + n, xr);
            if (a.q) {
                float t[8];
                ld8<IO>(a.q, row0 + n, t);
#pragma unroll
                for (int k = 0; k < 8; ++k) xr[k] *= t[k];
            }
            if (row1 >= 0) {
                ld8<IO>(a.u, row1 + n, xi);
                if (a.q) {
                    float t[8];
                    ld8<IO>(a.q, row1 + n, t);
#pragma unroll
                    for (int k = 0; k < 8; ++k) xi[k] *= t[k];
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) xi[k] = 0.f;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) xr[k] = xi[k] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) sin_[nh * LDW + col_swz(8 * cg + k)] = make_float2(xr[k], xi[k]);
    }
    __syncthreads();
    {
        const int t = threadIdx.x, ts = col_swz(t);
        float2 ev[H], od[H];
#pragma unroll
        for (int n = 0; n < H; ++n) {
            const float2 x = sin_[n * LDW + ts];
            ev[n] = x;
            od[n] = n == 0 ? x : cmulf(x, ((const float2*)a.tw_col)[n]);  // w_M1^n
        }
        dft_small<H, false>(ev);
        dft_small<H, false>(od);
        // four-step twiddle w_M^{n_lo k}, k = 0 .. M1-1, as powers of w_M^{n_lo}
        const int64_t n_lo = n_lo0 + t;
        const float2 w1 = tw_m(a.tw_lo, a.tw_hi, n_lo & (a.M - 1));
        float2 w = make_float2(1.f, 0.f);
#pragma unroll
        for (int k = 0; k < M1; ++k) {
            const float2 x = (k & 1) ? od[k >> 1] : ev[k >> 1];
            sout[k * LDW + ts] = cmulf(x, w);
            w = cmulf(w, w1);
        }
    }
    __syncthreads();
    for (int it = threadIdx.x; it < M1 * g8; it += 256) {
        const int kh = it / g8, cg = it % g8;
        float2 z[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) z[k] = sout[kh * LDW + col_swz(8 * cg + k)];
        ws_st8<CT>(a.ws, (s * a.M1 + kh) * kM2 + n_lo0 + 8 * cg, z);
    }
}

template <int CT, int IO, int M1>
__global__ void __launch_bounds__(256) col_small_inv_kernel(const ColArgs a) {
    constexpr int H = M1 / 2, CB = 256, LDW = CB + 1;
    __shared__ float2 sin_[M1 * LDW];
    __shared__ float2 sout[H * LDW];
    const int64_t s = blockIdx.y, gs = a.seq0 + s;
    const int64_t n_lo0 = (int64_t)blockIdx.x * CB;
    int64_t row0, row1;
    seq_rows(a, gs, row0, row1);
    constexpr int g8 = CB / 8;
    for (int it = threadIdx.x; it < M1 * g8; it += 256) {
        const int kh = it / g8, cg = it % g8;
        float2 z[8];
        ws_ld8<CT>(a.ws, (s * a.M1 + kh) * kM2 + n_lo0 + 8 * cg, z);
#pragma unroll
        for (int k = 0; k < 8; ++k) sin_[kh * LDW + col_swz(8 * cg + k)] = z[k];
    }
    __syncthreads();
    {
        const int t = threadIdx.x, ts = col_swz(t);
        const int64_t n_lo = n_lo0 + t;
        const float2 w1 = tw_m(a.tw_lo, a.tw_hi, n_lo & (a.M - 1));
        float2 w = make_float2(1.f, 0.f);
        float2 ev[H], od[H];
#pragma unroll
        for (int k = 0; k < M1; ++k) {
            const float2 z = cmulcf(sin_[k * LDW + ts], w);  // inverse four-step twiddle
            if (k & 1) od[k >> 1] = z;
            else ev[k >> 1] = z;
            w = cmulf(w, w1);
        }
        dft_small<H, true>(ev);
        dft_small<H, true>(od);
#pragma unroll
        for (int n = 0; n < H; ++n) {
            const float2 o = n == 0 ? od[0] : cmulcf(od[n], ((const float2*)a.tw_col)[n]);  // w_M1^{-n}
            sout[n * LDW + ts] = make_float2(ev[n].x + o.x, ev[n].y + o.y);
        }
    }
    __syncthreads();
    for (int it = threadIdx.x; it < H * g8; it += 256) {
        const int nh = it / g8, cg = it % g8;
        const int64_t n = kM2 * nh + n_lo0 + 8 * cg;
        if (n >= a.N) continue;
        float yr[8], yi[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float2 z = sout[nh * LDW + col_swz(8 * cg + k)];
            yr[k] = z.x;
            yi[k] = z.y;
        }
        if (a.v) {
            float t[8];
            ld8<IO>(a.v, row0 + n, t);
#pragma unroll
            for (int k = 0; k < 8; ++k) yr[k] *= t[k];
        }
        st8<IO>(a.y, row0 + n, yr);
        if (row1 >= 0) {
            if (a.v) {
                float t[8];
                ld8<IO>(a.v, row1 + n, t);
#pragma unroll
                for (int k = 0; k < 8; ++k) yi[k] *= t[k];
            }
            st8<IO>(a.y, row1 + n, yi);
        }
    }
}

template <int CT, int IO, int M1>
static hipError_t launch_small_t(bool fwd, const ColArgs& a, hipStream_t st) {
    dim3 grid((unsigned)(kM2 / 256), (unsigned)a.nseq);
    if (fwd) hipLaunchKernelGGL((col_small_fwd_kernel<CT, IO, M1>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((col_small_inv_kernel<CT, IO, M1>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int CT, int IO, int TPB>
static hipError_t launch_cols_t(bool fwd, const ColArgs& a, hipStream_t st) {
    const int M1 = (int)a.M1;
    const int CB = cols_per_wg(M1);
    const size_t lds = (size_t)CB * (M1 + 1) * sizeof(float2);
    dim3 grid((unsigned)(kM2 / CB), (unsigned)a.nseq);
    // dynamic LDS above the default limit has to be allowed per kernel (once, at the device
    // maximum: the block size depends on M1, at most 66,560 bytes)
    static bool attr_set[2] = {false, false};
    auto kfwd = col_fwd_kernel<CT, IO, TPB>;
    auto kinv = col_inv_kernel<CT, IO, TPB>;
    if (!attr_set[fwd ? 0 : 1]) {
        hipError_t e = hipFuncSetAttribute(fwd ? (const void*)kfwd : (const void*)kinv,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set[fwd ? 0 : 1] = true;
    }
    if (fwd) hipLaunchKernelGGL(kfwd, grid, dim3(TPB), lds, st, a);
    else hipLaunchKernelGGL(kinv, grid, dim3(TPB), lds, st, a);
    return hipGetLastError();
}

template <int CT, int IO>
static hipError_t launch_cols(bool fwd, const ColArgs& a, hipStream_t st) {
    if (a.nseq <= 0) return hipSuccess;
    const int M1 = (int)a.M1;
    if (M1 < 2 || M1 > 1024 || (M1 & (M1 - 1))) return hipErrorInvalidValue;
    if constexpr (CT != CT_F32) {  // 16-bit long columns: the matrix-core passes (colmx.hip)
        if (!a.filter && a.img && colmx_supported(M1)) return launch_colmx(fwd, CT, a, st);
    }
    switch (M1) {  // one column per thread, DFT in registers
    case 2: return launch_small_t<CT, IO, 2>(fwd, a, st);
    case 4: return launch_small_t<CT, IO, 4>(fwd, a, st);
    case 8: return launch_small_t<CT, IO, 8>(fwd, a, st);
    case 16: return launch_small_t<CT, IO, 16>(fwd, a, st);
    default: break;
    }
    // LDS passes: many small blocks per CU for short columns; 8 waves for a 64 KB block (two
    // blocks per CU, so that one block's loads and stores overlap the other's column DFTs)
    return M1 <= 64 ? launch_cols_t<CT, IO, 256>(fwd, a, st) : launch_cols_t<CT, IO, 512>(fwd, a, st);
}

// dtype: io type.  The workspace holds the compute type: fp32 for fp32 io and for filters,
// else the io type.
// rows = 0 stands for M1 (every row stored); fewer rows only on the matrix-core passes
static bool rows_ok(ColArgs& a, bool mx) {
    if (a.rows == 0) a.rows = a.M1;
    return a.rows == a.M1 || mx;
}

hipError_t launch_col_fwd(int dtype, const ColArgs& a0, hipStream_t st) {
    ColArgs a = a0;
    const bool mx = dtype != CT_F32 && !a.filter && a.img && colmx_supported(a.M1);
    if (!rows_ok(a, mx)) return hipErrorInvalidValue;
    if (a.filter) {
        if (dtype == CT_F32) return launch_cols<CT_F32, CT_F32>(true, a, st);
        if (dtype == CT_F16) return launch_cols<CT_F32, CT_F16>(true, a, st);
        return launch_cols<CT_F32, CT_BF16>(true, a, st);
    }
    if (dtype == CT_F32) return launch_cols<CT_F32, CT_F32>(true, a, st);
    if (dtype == CT_F16) return launch_cols<CT_F16, CT_F16>(true, a, st);
    return launch_cols<CT_BF16, CT_BF16>(true, a, st);
}

hipError_t launch_col_inv(int dtype, const ColArgs& a0, hipStream_t st) {
    ColArgs a = a0;
    const bool mx = dtype != CT_F32 && !a.filter && a.img && colmx_supported(a.M1);
    if (!rows_ok(a, mx)) return hipErrorInvalidValue;
    if (dtype == CT_F32) return launch_cols<CT_F32, CT_F32>(false, a, st);
    if (dtype == CT_F16) return launch_cols<CT_F16, CT_F16>(false, a, st);
    return launch_cols<CT_BF16, CT_BF16>(false, a, st);
}

}  // namespace lcv
