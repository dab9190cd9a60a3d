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
// The column DFTs are short (M1 = 2..512) and run as radix-2 butterflies in fp32 in LDS.
#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

namespace {

constexpr int kColLds = 8192;  // complex fp32 elements of LDS per workgroup (64 KB)
constexpr int64_t kM2 = 8192;

__device__ __forceinline__ int bitrev(int x, int bits) { return (int)(__brev((unsigned)x) >> (32 - bits)); }

template <int IO>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
    if constexpr (IO == CT_F32) return ((const float*)p)[i];
    else return unpack_lo<IO>(((const uint16_t*)p)[i]);
}
template <int IO>
__device__ __forceinline__ void st1(void* p, int64_t i, float x) {
    if constexpr (IO == CT_F32) {
        ((float*)p)[i] = x;
    } else {
        ((uint16_t*)p)[i] = (uint16_t)(pack2<IO>(x, 0.f) & 0xffffu);
    }
}
// workspace complex element in compute type CT
template <int CT>
__device__ __forceinline__ float2 ws_ld(const void* p, int64_t i) {
    if constexpr (CT == CT_F32) return ((const float2*)p)[i];
    else {
        uint32_t w = ((const uint32_t*)p)[i];
        return make_float2(unpack_lo<CT>(w), unpack_hi<CT>(w));
    }
}
template <int CT>
__device__ __forceinline__ void ws_st(void* p, int64_t i, float2 v) {
    if constexpr (CT == CT_F32) ((float2*)p)[i] = v;
    else ((uint32_t*)p)[i] = pack2<CT>(v.x, v.y);
}

// exp(-2 pi i r / M) from the two-level table
__device__ __forceinline__ float2 tw_m(const float* lo, const float* hi, int64_t r) {
    float2 a = ((const float2*)lo)[r & 2047];
    float2 b = ((const float2*)hi)[r >> 11];
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// In-place radix-2 DIT over rows of buf[M1][CB] (input already in bit-reversed row order).
// sign = -1 forward, +1 inverse (conjugate twiddles).
__device__ void col_fft(float2* buf, int M1, int CB, const float* tw_col, bool inverse) {
    const int nb = M1 / 2 * CB;
    for (int len = 2; len <= M1; len <<= 1) {
        const int half = len / 2, step = M1 / len;
        for (int idx = threadIdx.x; idx < nb; idx += blockDim.x) {
            const int col = idx % CB, bf = idx / CB;
            const int grp = bf / half, pos = bf % half;
            const int i0 = grp * len + pos, i1 = i0 + half;
            float2 w = ((const float2*)tw_col)[pos * step];
            if (inverse) w.y = -w.y;
            float2 x0 = buf[i0 * CB + col], x1 = buf[i1 * CB + col];
            float2 t = make_float2(x1.x * w.x - x1.y * w.y, x1.x * w.y + x1.y * w.x);
            buf[i0 * CB + col] = make_float2(x0.x + t.x, x0.y + t.y);
            buf[i1 * CB + col] = make_float2(x0.x - t.x, x0.y - t.y);
        }
        __syncthreads();
    }
}

}  // namespace

template <int CT, int IO>
__global__ void __launch_bounds__(256) col_fwd_kernel(const ColArgs a) {
    __shared__ float2 buf[kColLds];
    const int M1 = (int)a.M1, CB = kColLds / M1 < 256 ? kColLds / M1 : 256;
    const int bits = 31 - __clz(M1);
    const int64_t s = blockIdx.y;               // sequence within the chunk
    const int64_t gs = a.seq0 + s;              // global sequence
    const int64_t n_lo0 = (int64_t)blockIdx.x * CB;
    int64_t row0 = 0, row1 = -1;
    if (a.filter) {
        row0 = gs * a.N;                         // k[h]
    } else {
        const int64_t h = gs / a.seq_per_h, b = 2 * (gs % a.seq_per_h);
        row0 = (b * a.H + h) * a.N;
        if (b + 1 < a.B) row1 = row0 + a.H * a.N;
    }
    // load the nonzero half (n_hi < M1/2) into bit-reversed rows, zero the rest
    for (int idx = threadIdx.x; idx < M1 * CB; idx += blockDim.x) {
        const int col = idx % CB, nh = idx / CB;
        float2 z = make_float2(0.f, 0.f);
        const int64_t n = kM2 * nh + n_lo0 + col;
        if (nh < M1 / 2 && n < a.N) {
            float xr = ld1<IO>(a.u, row0 + n);
            if (a.q) xr *= ld1<IO>(a.q, row0 + n);
            float xi = 0.f;
            if (row1 >= 0) {
                xi = ld1<IO>(a.u, row1 + n);
                if (a.q) xi *= ld1<IO>(a.q, row1 + n);
            }
            z = make_float2(xr, xi);
        }
        buf[bitrev(nh, bits) * CB + col] = z;
    }
    __syncthreads();
    col_fft(buf, M1, CB, a.tw_col, false);
    // twiddle w_M^{n_lo k_hi}, store [k_hi][n_lo]
    for (int idx = threadIdx.x; idx < M1 * CB; idx += blockDim.x) {
        const int col = idx % CB, kh = idx / CB;
        const int64_t n_lo = n_lo0 + col;
        const int64_t r = (n_lo * kh) & (a.M - 1);
        float2 w = tw_m(a.tw_lo, a.tw_hi, r);
        float2 x = buf[kh * CB + col];
        float2 o = make_float2(x.x * w.x - x.y * w.y, x.x * w.y + x.y * w.x);
        ws_st<CT>(a.ws, (s * a.M1 + kh) * kM2 + n_lo, o);
    }
}

template <int CT, int IO>
__global__ void __launch_bounds__(256) col_inv_kernel(const ColArgs a) {
    __shared__ float2 buf[kColLds];
    const int M1 = (int)a.M1, CB = kColLds / M1 < 256 ? kColLds / M1 : 256;
    const int bits = 31 - __clz(M1);
    const int64_t s = blockIdx.y;
    const int64_t gs = a.seq0 + s;
    const int64_t n_lo0 = (int64_t)blockIdx.x * CB;
    const int64_t h = gs / a.seq_per_h, b = 2 * (gs % a.seq_per_h);
    const int64_t row0 = (b * a.H + h) * a.N;
    const int64_t row1 = b + 1 < a.B ? row0 + a.H * a.N : -1;
    // load [k_hi][n_lo], inverse twiddle, bit-reversed rows
    for (int idx = threadIdx.x; idx < M1 * CB; idx += blockDim.x) {
        const int col = idx % CB, kh = idx / CB;
        const int64_t n_lo = n_lo0 + col;
        const int64_t r = (n_lo * kh) & (a.M - 1);
        float2 w = tw_m(a.tw_lo, a.tw_hi, r);
        float2 x = ws_ld<CT>(a.ws, (s * a.M1 + kh) * kM2 + n_lo);
        buf[bitrev(kh, bits) * CB + col] = make_float2(x.x * w.x + x.y * w.y, x.y * w.x - x.x * w.y);
    }
    __syncthreads();
    col_fft(buf, M1, CB, a.tw_col, true);
    for (int idx = threadIdx.x; idx < M1 / 2 * CB; idx += blockDim.x) {
        const int col = idx % CB, nh = idx / CB;
        const int64_t n = kM2 * nh + n_lo0 + col;
        if (n >= a.N) continue;
        float2 z = buf[nh * CB + col];
        float yr = z.x, yi = z.y;
        if (a.v) yr *= ld1<IO>(a.v, row0 + n);
        st1<IO>(a.y, row0 + n, yr);
        if (row1 >= 0) {
            if (a.v) yi *= ld1<IO>(a.v, row1 + n);
            st1<IO>(a.y, row1 + n, yi);
        }
    }
}

template <int CT, int IO>
static hipError_t launch_cols(bool fwd, const ColArgs& a, hipStream_t st) {
    if (a.nseq <= 0) return hipSuccess;
    const int CB = kColLds / (int)a.M1 < 256 ? kColLds / (int)a.M1 : 256;
    dim3 grid((unsigned)(kM2 / CB), (unsigned)a.nseq);
    if (fwd) hipLaunchKernelGGL((col_fwd_kernel<CT, IO>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((col_inv_kernel<CT, IO>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// dtype: io type.  The workspace holds the compute type: fp32 for fp32 io and for filters,
// else the io type.
hipError_t launch_col_fwd(int dtype, const ColArgs& a, hipStream_t st) {
    if (a.filter) {
        if (dtype == CT_F32) return launch_cols<CT_F32, CT_F32>(true, a, st);
        if (dtype == CT_F16) return launch_cols<CT_F32, CT_F16>(true, a, st);
        return launch_cols<CT_F32, CT_BF16>(true, a, st);
    }
    if (dtype == CT_F32) return launch_cols<CT_F32, CT_F32>(true, a, st);
    if (dtype == CT_F16) return launch_cols<CT_F16, CT_F16>(true, a, st);
    return launch_cols<CT_BF16, CT_BF16>(true, a, st);
}

hipError_t launch_col_inv(int dtype, const ColArgs& a, hipStream_t st) {
    if (dtype == CT_F32) return launch_cols<CT_F32, CT_F32>(false, a, st);
    if (dtype == CT_F16) return launch_cols<CT_F16, CT_F16>(false, a, st);
    return launch_cols<CT_BF16, CT_BF16>(false, a, st);
}

}  // namespace lcv
