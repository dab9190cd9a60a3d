// fftconv2d.hip -- 2D linear convolution with a centred full-size kernel (HyenaND-style).
//
// "Native Multi-Dimensional Subquadratic Operators via Input Dependent Long Convolutions"
// (abstract) applies global convolutions on the native 2D grid and fuses the FFT-convolution
// path.  For S x S images and S x S kernels the linear convolution fits a P x P = 2S x 2S
// transform (P >= 2S - 1, so nothing wraps around); the output is the S x S window starting at
// (S/2, S/2) of the full convolution, i.e. the kernel's tap (S/2, S/2) is its centre.
//
// One workgroup handles two images of the same channel as one complex image (their spectra
// multiply by the same real kernel's spectrum):
//   S0  row DFTs (length 256) of the 128 nonzero rows; each row is one 16 x 16 register tile,
//       two radix-16 matrix-core stages with one twiddle between them            -> LDS
//   S1  per frequency column: column DFT, product with the kernel spectrum (the D skip folded
//       in), inverse column DFT computing only the 128 rows of the output window  -> LDS
//   S2  inverse row DFTs computing only the 128 columns of the output window       -> LDS
//   S3  coalesced store of both images.
// The 128 x 256 complex intermediate (bf16/fp16 pairs, 128 KB) stays in LDS throughout.
#include <type_traits>

#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

namespace {

constexpr int S2D = 128;   // image side
constexpr int P2D = 256;   // transform side
constexpr int RS = 257;    // LDS row stride (words): odd, so row index enters the bank number

// Column index swizzle: flips bits 4-5 of v by the 64-blocks of row and column, which makes
// both the row-tile pattern (fixed r) and the column-tile pattern (fixed v) bank-conflict free.
__device__ __forceinline__ int swz(int r, int v) { return v ^ ((((r >> 6) ^ (v >> 6)) & 3) << 4); }

template <int IO>
__device__ __forceinline__ uint32_t ld_raw2(const void* p, int64_t i) {
    return ((const uint16_t*)p)[i];
}

}  // namespace

template <int CT>
__global__ void __launch_bounds__(512) conv2d_kernel(const Conv2DArgs a) {
    static_assert(CT != CT_F32, "2D path runs 16-bit operands");
    constexpr int IO = CT;
    constexpr int IMG = ImgBytes<CT>::value;
    // tables of the 256-point transform (R = 1 layout): F2[0] / F3[0] are the plain radix-16
    // DFT block, I1[0] / I2[0] its conjugate, then the w_256 twiddles.
    constexpr int T_F1 = 0;
    constexpr int T_I3 = T_F1 + IMG;
    constexpr int T_F2 = T_I3 + IMG;
    constexpr int T_F3 = T_F2 + IMG;
    constexpr int T_I1 = T_F3 + IMG;
    constexpr int T_I2 = T_I1 + IMG;
    constexpr int T_TW = T_I2 + IMG;
    constexpr int BUF_W = S2D * RS;
    constexpr int STG_W = 32 * S2D;

    __shared__ __attribute__((aligned(16))) uint32_t lds[BUF_W + STG_W];
    uint32_t* BUF = lds;
    uint32_t* STG = lds + BUF_W;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const char* tab = (const char*)a.tables;
    const MatImg<CT> Gf = load_img<CT>(tab + T_F2, 0, lane);
    const MatImg<CT> Gi = load_img<CT>(tab + T_I1, 0, lane);
    f32x4 twr, twi;
    {
        const float4* tp = (const float4*)(tab + T_TW) + lane * 2;
        float4 t0 = tp[0], t1 = tp[1];
        twr = f32x4{t0.x, t0.z, t1.x, t1.z};
        twi = f32x4{t0.y, t0.w, t1.y, t1.w};
    }

    // Items are channel-major (a channel's batch pairs are consecutive).  A workgroup takes items
    // v, v + G, v + 2G, ... (G workgroups), where v renumbers the workgroups XCD by XCD: the
    // dispatcher deals workgroup ids round-robin over the 8 XCDs, so consecutive v, and hence
    // the pairs of one channel at one step, run on the same XCD and share its L2 copy of the
    // channel's 256 KB spectrum.
    const int64_t Bp = (a.B + 1) / 2, nitems = Bp * a.C, G = gridDim.x;
    const int64_t v = G % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : (int64_t)blockIdx.x;
    constexpr int64_t IMGSZ = (int64_t)S2D * S2D;

    // staged input chunk of this thread: row (tid / 16) of a 32-row quarter, elements 8*(tid%16)..
    const int srow = tid >> 4, scol = 8 * (tid & 15);
    uint4 pre0, pre1;  // u of image b and b+1 (next chunk)
    auto issue = [&](int64_t item, int q) LCV_INLINE {
        const int64_t ch = item / Bp, b = 2 * (item % Bp);
        const int64_t base0 = (b * a.C + ch) * IMGSZ + (int64_t)(32 * q + srow) * S2D + scol;
        const int64_t base1 = b + 1 < a.B ? base0 + a.C * IMGSZ : base0;
        pre0 = *(const uint4*)((const uint16_t*)a.u + base0);
        pre1 = *(const uint4*)((const uint16_t*)a.u + base1);
    };
    if (v < nitems) issue(v, 0);

    for (int64_t item = v; item < nitems; item += G) {
        const int64_t ch = item / Bp, b = 2 * (item % Bp);
        const bool has1 = b + 1 < a.B;

        // ================= S0: row DFTs, 4 quarters of 32 rows ================================
        for (int q = 0; q < 4; ++q) {
            {   // pack (image b, image b+1) as complex words into the staging area
                const uint32_t w0[4] = {pre0.x, pre0.y, pre0.z, pre0.w};
                const uint32_t w1[4] = {pre1.x, pre1.y, pre1.z, pre1.w};
                uint32_t o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t hi = has1 ? w1[i] : 0u;
                    o[2 * i] = __byte_perm(w0[i], hi, 0x5410);      // (lo(w0), lo(w1))
                    o[2 * i + 1] = __byte_perm(w0[i], hi, 0x7632);  // (hi(w0), hi(w1))
                }
                uint4* dst = (uint4*)(STG + srow * S2D + scol);
                dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
                dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
            }
            // next chunk: next quarter, or the next item's first quarter
            if (q < 3) issue(item, q + 1);
            else if (item + G < nitems) issue(item + G, 0);
            __syncthreads();
            // 4 row tiles per wave: rows r = 32 q + 4 wave + i
            Operand<CT> opd[4];
            Tile xs[4];
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int lr = 4 * wave + i;
                Operand<CT> o;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o.w[jj] = g < 2 ? STG[lr * S2D + 16 * (4 * g + jj) + c] : 0u;
                opd[i] = o;
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_swap<CT>(Gf, opd[i]);  // (L = k2, K = n3)
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                cmul4(xs[i], twr, twi);
                opd[i] = to_operand<CT>(xs[i]);
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_keep<CT>(Gf, opd[i]);  // (L = k2, K = k3): v = k2 + 16 k3
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int r = 32 * q + 4 * wave + i;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int v = c + 16 * (4 * g + jj);
                    BUF[r * RS + swz(r, v)] = pack2<CT>(xs[i].re[jj], xs[i].im[jj]);
                }
            });
            __syncthreads();
        }

        // ================= S1: columns: DFT, spectrum product, inverse DFT (window rows) =====
        const float dsc = unpack_lo<IO>(ld_raw2<IO>(a.D, ch)) * a.inv_p2;
        for (int v0 = 32 * wave; v0 < 32 * wave + 32; v0 += 4) {
            uint4 kr4[4];
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                kr4[i] = *((const uint4*)a.kf + ((ch * P2D + v0 + i) * 64 + lane));
            });
            Operand<CT> opd[4];
            Tile xs[4];
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int v = v0 + i;
                Operand<CT> o;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 16 * (4 * g + jj) + c;
                    o.w[jj] = g < 2 ? BUF[r * RS + swz(r, v)] : 0u;
                }
                opd[i] = o;
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_swap<CT>(Gf, opd[i]);
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                cmul4(xs[i], twr, twi);
                opd[i] = to_operand<CT>(xs[i]);
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_keep<CT>(Gf, opd[i]);  // (L = k2, K = k3): u = k2 + 16 k3
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int v = v0 + i;
                // kernel spectrum + D * exp(-2 pi i 64 (u + v) / 256) / P^2: the skip is a
                // delta at the kernel centre, whose spectrum is (-i)^(u+v)
                const int m = (c + v) & 3;
                const float dr = m == 0 ? dsc : (m == 2 ? -dsc : 0.f);
                const float di = m == 1 ? -dsc : (m == 3 ? dsc : 0.f);
                f32x4 kr, ki;
                const uint32_t kw[4] = {kr4[i].x, kr4[i].y, kr4[i].z, kr4[i].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    kr[jj] = unpack_lo<CT>(kw[jj]) + dr;
                    ki[jj] = unpack_hi<CT>(kw[jj]) + di;
                }
                cmul4(xs[i], kr, ki);
                opd[i] = to_operand<CT>(xs[i]);
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_swap<CT>(Gi, opd[i]);  // (L = r3, K = k2)
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                cmulc4(xs[i], twr, twi);
                opd[i] = to_operand<CT>(xs[i]);
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_keep<CT>(Gi, opd[i]);  // (L = r3, K = r2): row r' = 16 r2 + r3
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int v = v0 + i;
                if (g == 1 || g == 2) {  // rows 64 .. 191 of the full convolution
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = 16 * (4 * g + jj) + c - 64;
                        BUF[r * RS + swz(r, v)] = pack2<CT>(xs[i].re[jj], xs[i].im[jj]);
                    }
                }
            });
        }
        __syncthreads();

        // ================= S2: inverse row DFTs (window columns) ==============================
        for (int r0 = 16 * wave; r0 < 16 * wave + 16; r0 += 4) {
            Operand<CT> opd[4];
            Tile xs[4];
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int r = r0 + i;
                Operand<CT> o;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o.w[jj] = BUF[r * RS + swz(r, c + 16 * (4 * g + jj))];
                opd[i] = o;
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_swap<CT>(Gi, opd[i]);  // (L = n3, K = k2)
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                cmulc4(xs[i], twr, twi);
                opd[i] = to_operand<CT>(xs[i]);
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                xs[i] = stage_keep<CT>(Gi, opd[i]);  // (L = n3, K = n2): column j' = 16 n2 + n3
            });
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int r = r0 + i;
                if (g == 1 || g == 2) {  // columns 64 .. 191: output column j = j' - 64
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        BUF[r * RS + 16 * (4 * g + jj) + c - 64] = pack2<CT>(xs[i].re[jj], xs[i].im[jj]);
                }
            });
        }
        __syncthreads();

        // ================= S3: store both images ==============================================
        if (a.y) {
            for (int rr = 0; rr < S2D; rr += 32) {
                const int r = rr + srow;
                uint32_t w[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = BUF[r * RS + scol + i];
                const int64_t o0 = (b * a.C + ch) * IMGSZ + (int64_t)r * S2D + scol;
                uint4 y0, y1;
                y0.x = __byte_perm(w[0], w[1], 0x5410); y0.y = __byte_perm(w[2], w[3], 0x5410);
                y0.z = __byte_perm(w[4], w[5], 0x5410); y0.w = __byte_perm(w[6], w[7], 0x5410);
                y1.x = __byte_perm(w[0], w[1], 0x7632); y1.y = __byte_perm(w[2], w[3], 0x7632);
                y1.z = __byte_perm(w[4], w[5], 0x7632); y1.w = __byte_perm(w[6], w[7], 0x7632);
                *(uint4*)((uint16_t*)a.y + o0) = y0;
                if (has1) *(uint4*)((uint16_t*)a.y + o0 + a.C * IMGSZ) = y1;
            }
        }
        // the next item's S0 writes STG first and BUF only after a barrier
    }
}

// 2D filter spectrum: K[u][v] = sum_{a,b} k[a][b] w^(u a + v b) / P^2 (w = exp(-2 pi i / 256)),
// computed as two explicit DFT-matrix passes in fp32 (one-off, not on the convolution path),
// stored in the order the column stage reads it: [channel][v][lane][jj], u = lane%16 +
// 16 (4 (lane/16) + jj).
template <int IO>
__global__ void __launch_bounds__(256) filter2d_kernel(const void* k, void* kf, float inv_p2) {
    __shared__ float2 T[S2D][32];
    __shared__ float2 W[P2D];
    const int ch = blockIdx.x, vb = blockIdx.y, tid = threadIdx.x;
    for (int e = tid; e < P2D; e += blockDim.x) {
        double s, cc;
        sincospi(-2.0 * e / P2D, &s, &cc);
        W[e] = make_float2((float)cc, (float)s);
    }
    __syncthreads();
    const uint16_t* kc = (const uint16_t*)k + (int64_t)ch * S2D * S2D;
    for (int idx = tid; idx < S2D * 32; idx += blockDim.x) {
        const int ar = idx / 32, vv = idx % 32, v = 32 * vb + vv;
        float re = 0.f, im = 0.f;
        for (int bb = 0; bb < S2D; ++bb) {
            const float x = unpack_lo<IO>(kc[ar * S2D + bb]);
            const float2 w = W[(v * bb) & (P2D - 1)];
            re += x * w.x;
            im += x * w.y;
        }
        T[ar][vv] = make_float2(re, im);
    }
    __syncthreads();
    for (int idx = tid; idx < P2D * 32; idx += blockDim.x) {
        const int vv = idx / P2D, u = idx % P2D, v = 32 * vb + vv;
        float re = 0.f, im = 0.f;
        for (int ar = 0; ar < S2D; ++ar) {
            const float2 t = T[ar][vv], w = W[(u * ar) & (P2D - 1)];
            re += t.x * w.x - t.y * w.y;
            im += t.x * w.y + t.y * w.x;
        }
        const int pos = ((16 * (u >> 6) + (u & 15)) * 4) + ((u >> 4) & 3);
        ((uint32_t*)kf)[((int64_t)ch * P2D + v) * P2D + pos] = pack2<IO>(re * inv_p2, im * inv_p2);
    }
}

hipError_t launch_conv2d(int dtype, const Conv2DArgs& a, hipStream_t st) {
    if (a.filter) {
        dim3 grid((unsigned)a.C, P2D / 32);
        if (dtype == CT_F16) hipLaunchKernelGGL((filter2d_kernel<CT_F16>), grid, dim3(256), 0, st, a.u, (void*)a.kf, a.inv_p2);
        else hipLaunchKernelGGL((filter2d_kernel<CT_BF16>), grid, dim3(256), 0, st, a.u, (void*)a.kf, a.inv_p2);
        return hipGetLastError();
    }
    const int64_t nitems = (a.B + 1) / 2 * a.C;
    if (nitems <= 0) return hipSuccess;
    const int64_t nwg = nitems < a.cus ? nitems : a.cus;
    if (dtype == CT_F16) hipLaunchKernelGGL((conv2d_kernel<CT_F16>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    else hipLaunchKernelGGL((conv2d_kernel<CT_BF16>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcv
