// fftconv3d.hip -- the 3D (volume) centred linear convolution, HyenaND-style, for S = 16 and 32.
//
//   y[b,c] = (k[c] * u[b,c])_full[S/2 : S/2+S]^3 + D[c] u[b,c]
//
// The 2D operation one dimension up ("Native Multi-Dimensional Subquadratic Operators via Input
// Dependent Long Convolutions", abstract: global convolutions on the native multi-dimensional
// grid, through a fused FFT-convolution path).  The transform is P^3 with P = 2S (zero-padded,
// so the linear convolution does not wrap into the window) and separable.  Its intermediate
// (S P^2 complex per image pair: 2 MB at S = 32 in fp32) does not fit one workgroup, so the path
// makes three passes over a workspace W[unit][S][P][P] (compute type):
//   A  per input slice z < S: 2D DFT over x then y (both half-zero), to W[z][ky][kx]
//   Z  per row ky (all kx): DFT over z (half-zero), times (K + D (-i)^(kx+ky+kz)) / P^3 -- D is a
//      delta at the kernel centre, whose spectrum is (-i)^(kx+ky+kz) -- then the inverse DFT,
//      keeping the window slices m_z = S/2 + zo, back to W[zo][ky][kx]
//   C  per window slice zo: inverse 2D DFT, keep the (y, x) window, store
// The filter spectrum K = DFT_P^3(k) / P^3 comes from passes A and Z in filter mode, stored as
// [c][kz][ky][kx] complex.  Two batch images of one channel ride in one complex transform
// (u_b + i u_{b+1}; the kernel is real).  All DFTs run in LDS on fp32 columns (coldft.h).
#include "coldft.h"
#include "fused_io.h"
#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

namespace {

// unit -> (channel c, element offsets of the two volumes; row1 < 0 when there is no second)
__device__ __forceinline__ void unit_rows(const Conv3DArgs& a, int64_t unit, int64_t S3, int64_t& c,
                                          int64_t& row0, int64_t& row1) {
    if (a.filter) {
        c = unit;
        row0 = c * S3;
        row1 = -1;
    } else {
        const int64_t Bp = (a.B + 1) / 2;
        c = unit / Bp;
        const int64_t b = 2 * (unit - c * Bp);
        row0 = (b * a.C + c) * S3;
        row1 = b + 1 < a.B ? row0 + a.C * S3 : -1;
    }
}

}  // namespace

// Pass A: one input slice z of one unit: DFT over x (columns y), transpose, DFT over y.
template <int S, int CT, int IO>
__global__ void __launch_bounds__(256) k3_slices_fwd(const Conv3DArgs a) {
    constexpr int P = 2 * S, LD = P + 1;
    __shared__ float2 A[S * LD];   // column y, rows x
    __shared__ float2 Bf[P * LD];  // column kx, rows y
    const int tid = threadIdx.x, z = blockIdx.x;
    const int64_t ul = blockIdx.y, unit = a.unit0 + ul;
    int64_t c, row0, row1;
    unit_rows(a, unit, (int64_t)S * S * S, c, row0, row1);
    for (int it = tid; it < S * (S / 8); it += 256) {
        const int y = it / (S / 8), x0 = 8 * (it % (S / 8));
        const int64_t off = ((int64_t)z * S + y) * S + x0;
        float xr[8], xi[8];
        ld8<IO>(a.u, row0 + off, xr);
        if (row1 >= 0) {
            ld8<IO>(a.u, row1 + off, xi);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xi[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) A[y * LD + x0 + i] = make_float2(xr[i], xi[i]);
    }
    __syncthreads();
    column_dft<256, false>(A, P, LD, S, a.tw, P);   // x -> kx (rows x >= S are zero)
    for (int it = tid; it < S * P; it += 256) {
        const int y = it / P, kx = it % P;
        Bf[kx * LD + y] = A[y * LD + kx];
    }
    __syncthreads();
    column_dft<256, false>(Bf, P, LD, P, a.tw, P);  // y -> ky (rows y >= S are zero)
    for (int it = tid; it < P * (P / 8); it += 256) {
        const int ky = it / (P / 8), kx0 = 8 * (it % (P / 8));
        float2 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = Bf[(kx0 + i) * LD + ky];
        ws_st8<CT>(a.ws, ((ul * S + z) * P + ky) * P + kx0, v);
    }
}

// Pass Z: one row ky of one unit (all kx): DFT over z; filter mode stores the spectrum, else the
// product with the filter spectrum (skip folded in), the inverse DFT and the window slices.
template <int S, int CT, int IO, bool FILTER>
__global__ void __launch_bounds__(256) k3_zpass(const Conv3DArgs a) {
    constexpr int P = 2 * S, LD = P + 1;
    __shared__ float2 Z[P * LD];   // column kx, rows z / kz
    const int tid = threadIdx.x, ky = blockIdx.x;
    const int64_t ul = blockIdx.y, unit = a.unit0 + ul;
    int64_t c, row0, row1;
    unit_rows(a, unit, (int64_t)S * S * S, c, row0, row1);
    for (int it = tid; it < S * (P / 8); it += 256) {
        const int z = it / (P / 8), kx0 = 8 * (it % (P / 8));
        float2 v[8];
        ws_ld8<CT>(a.ws, ((ul * S + z) * P + ky) * P + kx0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) Z[(kx0 + i) * LD + z] = v[i];
    }
    __syncthreads();
    column_dft<256, false>(Z, P, LD, P, a.tw, P);   // z -> kz (slices z >= S are zero)
    if constexpr (FILTER) {
        for (int it = tid; it < P * (P / 8); it += 256) {
            const int kz = it / (P / 8), kx0 = 8 * (it % (P / 8));
            float2 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float2 t = Z[(kx0 + i) * LD + kz];
                v[i] = make_float2(t.x * a.inv_p3, t.y * a.inv_p3);
            }
            ws_st8<IO>(a.y, ((c * P + kz) * P + ky) * P + kx0, v);
        }
        return;
    } else {
        const float d = raw1_to_f32<IO>(load1_raw<IO>(a.D, c)) * a.inv_p3;
        for (int it = tid; it < P * (P / 8); it += 256) {
            const int kz = it / (P / 8), kx0 = 8 * (it % (P / 8));
            float2 kv[8];
            ws_ld8<IO>(a.kf, ((c * P + kz) * P + ky) * P + kx0, kv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // + D (-i)^(kx + ky + kz) / P^3: the skip as a delta at the kernel centre
                const int ph = (kx0 + i + ky + kz) & 3;
                const float2 dk = ph == 0 ? make_float2(d, 0.f)
                                : ph == 1 ? make_float2(0.f, -d)
                                : ph == 2 ? make_float2(-d, 0.f)
                                          : make_float2(0.f, d);
                const float2 kk = make_float2(kv[i].x + dk.x, kv[i].y + dk.y);
                float2& zz = Z[(kx0 + i) * LD + kz];
                zz = cmulf(zz, kk);
            }
        }
        __syncthreads();
        column_dft<256, true>(Z, P, LD, P, a.tw, P);   // kz -> m_z
        for (int it = tid; it < S * (P / 8); it += 256) {
            const int zo = it / (P / 8), kx0 = 8 * (it % (P / 8));
            float2 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = Z[(kx0 + i) * LD + S / 2 + zo];
            ws_st8<CT>(a.ws, ((ul * S + zo) * P + ky) * P + kx0, v);
        }
    }
}

// Pass C: one window slice zo of one unit: inverse DFT over ky (columns kx), keep the window
// rows, transpose, inverse DFT over kx, keep the window columns, store both images.
template <int S, int CT, int IO>
__global__ void __launch_bounds__(256) k3_slices_inv(const Conv3DArgs a) {
    constexpr int P = 2 * S, LD = P + 1;
    __shared__ float2 Bi[P * LD];  // column kx, rows ky / m_y
    __shared__ float2 A[S * LD];   // column y, rows kx / m_x
    const int tid = threadIdx.x, zo = blockIdx.x;
    const int64_t ul = blockIdx.y, unit = a.unit0 + ul;
    int64_t c, row0, row1;
    unit_rows(a, unit, (int64_t)S * S * S, c, row0, row1);
    for (int it = tid; it < P * (P / 8); it += 256) {
        const int ky = it / (P / 8), kx0 = 8 * (it % (P / 8));
        float2 v[8];
        ws_ld8<CT>(a.ws, ((ul * S + zo) * P + ky) * P + kx0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) Bi[(kx0 + i) * LD + ky] = v[i];
    }
    __syncthreads();
    column_dft<256, true>(Bi, P, LD, P, a.tw, P);   // ky -> m_y
    for (int it = tid; it < S * P; it += 256) {
        const int y = it / P, kx = it % P;
        A[y * LD + kx] = Bi[kx * LD + S / 2 + y];
    }
    __syncthreads();
    column_dft<256, true>(A, P, LD, S, a.tw, P);    // kx -> m_x
    for (int it = tid; it < S * (S / 8); it += 256) {
        const int y = it / (S / 8), x0 = 8 * (it % (S / 8));
        float yr[8], yi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float2 v = A[y * LD + S / 2 + x0 + i];
            yr[i] = v.x;
            yi[i] = v.y;
        }
        const int64_t off = ((int64_t)zo * S + y) * S + x0;
        st8<IO>(a.y, row0 + off, yr);
        if (row1 >= 0) st8<IO>(a.y, row1 + off, yi);
    }
}

template <int S, int CT, int IO>
static hipError_t launch3_t(const Conv3DArgs& a, hipStream_t st) {
    if (a.nunit <= 0) return hipSuccess;
    const dim3 blk(256);
    hipLaunchKernelGGL((k3_slices_fwd<S, CT, IO>), dim3(S, (unsigned)a.nunit), blk, 0, st, a);
    if (a.filter) {
        hipLaunchKernelGGL((k3_zpass<S, CT, IO, true>), dim3(2 * S, (unsigned)a.nunit), blk, 0, st, a);
    } else {
        hipLaunchKernelGGL((k3_zpass<S, CT, IO, false>), dim3(2 * S, (unsigned)a.nunit), blk, 0, st, a);
        hipLaunchKernelGGL((k3_slices_inv<S, CT, IO>), dim3(S, (unsigned)a.nunit), blk, 0, st, a);
    }
    return hipGetLastError();
}

template <int S>
static hipError_t launch3_s(int dtype, const Conv3DArgs& a, hipStream_t st) {
    // the filter transform runs in fp32; the convolution in the io type's compute type
    if (a.filter) {
        if (dtype == CT_F32) return launch3_t<S, CT_F32, CT_F32>(a, st);
        if (dtype == CT_F16) return launch3_t<S, CT_F32, CT_F16>(a, st);
        return launch3_t<S, CT_F32, CT_BF16>(a, st);
    }
    if (dtype == CT_F32) return launch3_t<S, CT_F32, CT_F32>(a, st);
    if (dtype == CT_F16) return launch3_t<S, CT_F16, CT_F16>(a, st);
    return launch3_t<S, CT_BF16, CT_BF16>(a, st);
}

hipError_t launch_conv3d(int dtype, const Conv3DArgs& a, hipStream_t stream) {
    if (a.S == 16) return launch3_s<16>(dtype, a, stream);
    if (a.S == 32) return launch3_s<32>(dtype, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lcv
