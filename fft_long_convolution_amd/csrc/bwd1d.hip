// bwd1d.hip -- filter gradient of the causal FFT convolution, transform lengths M = 256 R <= 8192.
//
// With x = q u, ds = dy v and y = v (k * x + D x), the gradient of sum(dy y) with respect to the
// filter is the cross-correlation  dk[t] = sum_b sum_{s >= t} ds_b[s] x_b[s - t]  and
// dD = dk[0].  In the frequency domain (length M >= 2N, so nothing wraps around) this is
//     dk = Re( IDFT( sum_b conj(X_b) DS_b ) )[:N].
// Batch rows ride in pairs, z = x_b + i x_{b+1}: for real rows the real part of
// conj(Zx) Zds is conj(X_b) DS_b + conj(X_{b+1}) DS_{b+1} after the inverse transform (the cross
// terms are purely imaginary), so one complex product per pair gives both rows.  An odd batch's
// last pair has a zero second row.
//
// The transforms are the forward chain of the fused convolution (F1 on matrix cores from LDS,
// F2, twiddle, F3 in registers; same digit order and tables), and the inverse is its mirror
// image with the causal truncation n1 < R/2.  The FFT convolution the pages describe is linear
// in the filter, so its filter gradient is the same machinery run on the two inputs of the
// correlation ("FlashFFTConv" abstract: exact FFT convolution on matrix units; "FlashConv" page,
// Mechanism: fused transform -> pointwise product -> inverse).
//
// Work split: one item = one channel.  A workgroup keeps the spectral sum of its channels in
// registers over all batch pairs and runs the inverse once per channel, so no partial sums
// leave the chip and nothing needs a second reduction pass.
#include <type_traits>

#include "fused_io.h"
#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

// c + lo(a) lo(b) + hi(a) hi(b) for two packed 16-bit pairs, accumulated in fp32
template <int CT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    static_assert(CT != CT_F32, "packed 16-bit pairs");
    if constexpr (CT == CT_BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    }
}


template <int R, int CT, int IO, bool GQ, bool GV>
__global__ void __launch_bounds__(512) dk1d_kernel(const Fused1DArgs a) {
    constexpr int P = 32 / R;                  // channels per workgroup iteration
    constexpr int M = 256 * R;
    constexpr int NH = R / 2;                  // nonzero input rows n1; output rows n1
    constexpr int KCF = (R + 15) / 16;         // table grid (full variant)
    constexpr int KC1 = (NH + 15) / 16;
    constexpr int RB1 = (R + 15) / 16;
    constexpr int KC3 = (R + 15) / 16;
    constexpr int RB3 = (NH + 15) / 16;
    constexpr int EW = CT == CT_F32 ? 2 : 1;   // LDS words per complex element
    constexpr int SV = 260;                    // V: row stride (elements) per n1 row
    constexpr int ST = 324, SR = 20;           // XY: tile stride, row stride inside a tile
    constexpr int SO = 260;                    // O: row stride (complex fp32)
    constexpr int V_W = P * NH * SV * EW;
    constexpr int XY_W = 32 * ST * EW;
    constexpr int O_W = P * NH * SO * 2;
    constexpr bool RES = (CT != CT_F32);       // F2 / F3 images resident in registers
    constexpr int IMG = ImgBytes<CT>::value;
    constexpr int T_F1 = 0;
    constexpr int T_I3 = T_F1 + IMG * RB1 * KCF;
    constexpr int T_F2 = T_I3 + IMG * KCF * KCF;
    constexpr int T_F3 = T_F2 + IMG * R;
    constexpr int T_I1 = T_F3 + IMG * R;
    constexpr int T_I2 = T_I1 + IMG * R;
    constexpr int T_TW = T_I2 + IMG * R;
    constexpr int NBLK = P * 16;               // (sequence, n2) column blocks
    constexpr int BPW = NBLK / 8;              // blocks per wave
    constexpr int IMGS_W = RES ? (T_F2 - T_F1) / 4 : 0;  // F1 and I3 images in LDS
    constexpr int IOW = IO == CT_F32 ? 2 : 1;  // uint4 per 8 io elements

    __shared__ __attribute__((aligned(16))) uint32_t lds[V_W + XY_W + O_W + IMGS_W];
    __shared__ float red[16];   // lag-0 partial sums, one per 32-lane half of a wave
    uint32_t* V = lds;
    uint32_t* XY = lds + V_W;
    float* O = (float*)(lds + V_W + XY_W);
    uint32_t* IMGS = lds + V_W + XY_W + O_W;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const char* tab = (const char*)a.tables;
    const int64_t first = (int64_t)blockIdx.x * a.per_wg;
    const int64_t last = first + a.per_wg < a.nitems ? first + a.per_wg : a.nitems;
    if (first >= last) return;

    f32x4 twr, twi;
    {
        const float4* tp = (const float4*)(tab + T_TW) + lane * 2;
        float4 t0 = tp[0], t1 = tp[1];
        twr = f32x4{t0.x, t0.z, t1.x, t1.z};
        twi = f32x4{t0.y, t0.w, t1.y, t1.w};
    }
    MatImg<CT> mf2[4], mf3[4];
    if constexpr (RES) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k1 = (wave * 4 + i) % R;
            mf2[i] = load_img<CT>(tab + T_F2, k1, lane);
            mf3[i] = load_img<CT>(tab + T_F3, k1, lane);
        }
        for (int w = tid; w < IMGS_W / 4; w += 512) ((uint4*)IMGS)[w] = ((const uint4*)(tab + T_F1))[w];
        __syncthreads();  // every wave reads all of them
    }
    auto F1 = [&](int rb, int kc) LCV_INLINE {
        if constexpr (RES) return load_img_lds<CT>(IMGS, rb * KCF + kc, lane);
        else return load_img<CT>(tab + T_F1, rb * KCF + kc, lane);
    };
    auto I3 = [&](int rb, int kc) LCV_INLINE {
        if constexpr (RES) return load_img_lds<CT>(IMGS + (T_I3 - T_F1) / 4, rb * KCF + kc, lane);
        else return load_img<CT>(tab + T_I3, rb * KCF + kc, lane);
    };
    auto F2 = [&](int i) LCV_INLINE { return RES ? mf2[i] : load_img<CT>(tab + T_F2, (wave * 4 + i) % R, lane); };
    auto F3 = [&](int i) LCV_INLINE { return RES ? mf3[i] : load_img<CT>(tab + T_F3, (wave * 4 + i) % R, lane); };

    // This lane's slot (8 consecutive elements of one sequence row), as in the fused
    // convolution: row n1 = ci / (2 BPW), block wave*BPW + (ci / 2) % BPW, half ci % 2.  A wave's
    // slots are the columns of its own radix-R blocks, so P0 -> P1 and P3 -> P4 stay wave-local.
    auto slot = [&](int ci, int& p, int& n0) LCV_INLINE {
        const int n1 = ci / (2 * BPW), blk = wave * BPW + (ci >> 1) % BPW;
        p = blk >> 4;
        n0 = 256 * n1 + 16 * (blk & 15) + 8 * (ci & 1);
    };
    int p_io, n0_io;
    slot(lane, p_io, n0_io);
    const int64_t Bp = (a.B + 1) / 2;
    const int64_t HN = a.H * a.N;

    // Element offsets of the slot in batch rows 2j, 2j+1 of channel it0 + p_io, clamped into
    // range so that loads are unconditional; ok0 / ok1 say which rows hold data.
    auto offsets = [&](int64_t it0, int64_t j, int64_t& o0, int64_t& o1, bool& ok0, bool& ok1) LCV_INLINE {
        const int64_t h = it0 + p_io;
        const int64_t b = 2 * j;
        ok0 = h < last && n0_io < a.N;
        ok1 = ok0 && b + 1 < a.B;
        const int64_t hc = h < last ? h : last - 1;
        const int64_t n0c = n0_io < a.N ? n0_io : a.N - 8;
        o0 = (b * a.H + hc) * a.N + n0c;
        o1 = (b + 1 < a.B ? o0 + HN : o0);
    };
    // raw inputs of one half: (u, q) for x or (dy, v) for ds, both batch rows
    uint4 ra[2][IOW], rb[2][IOW];
    auto issue = [&](auto which, int64_t it0, int64_t j) LCV_INLINE {
        constexpr bool DS = decltype(which)::value;
        constexpr bool GATE = DS ? GV : GQ;
        int64_t o0, o1;
        bool k0, k1;
        offsets(it0, j < Bp ? j : Bp - 1, o0, o1, k0, k1);
        const void* pa = DS ? a.e2 : a.u;
        load_raw<IO>(pa, o0, ra[0]);
        load_raw<IO>(pa, o1, ra[1]);
        if constexpr (GATE) {
            const void* pb = DS ? a.v : a.q;
            load_raw<IO>(pb, o0, rb[0]);
            load_raw<IO>(pb, o1, rb[1]);
        }
    };

    // P0: gate and pack the slot (pair z = row 2j + i row 2j+1) into V
    // 16-bit types: dD and dk[h][0] from the direct lag-0 sum (fp32 keeps the spectral one, whose
    // rounding is far below its tolerance)
    constexpr bool LAG0 = CT != CT_F32;
    float dsum = 0.f;  // this lane's share of the lag-0 sum of its channel group
    auto P0 = [&](auto which, int64_t it0, int64_t j) LCV_INLINE {
        constexpr bool GATE = decltype(which)::value ? GV : GQ;
        int64_t o0, o1;
        bool ok0, ok1;
        offsets(it0, j, o0, o1, ok0, ok1);
        float xr[8], xi[8];
        unpack_raw<IO>(ra[0], xr);
        unpack_raw<IO>(ra[1], xi);
        if constexpr (GATE) {
            float t[8];
            unpack_raw<IO>(rb[0], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[i] *= t[i];
            unpack_raw<IO>(rb[1], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) xi[i] *= t[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xr[i] = ok0 ? xr[i] : 0.f;
            xi[i] = ok1 ? xi[i] : 0.f;
        }
        uint32_t* dst = V + ((p_io * NH + (n0_io >> 8)) * SV + (n0_io & 255)) * EW;
        if constexpr (decltype(which)::value && LAG0) {
            // the slot still holds this pair's x (the x pass wrote it; nothing since): lag 0
            // directly, sum of x ds over the slot, as packed (re, im) pairs of x and of ds (one
            // two-term dot product per element pair, accumulated in fp32)
            const uint4 w0 = ((const uint4*)dst)[0], w1 = ((const uint4*)dst)[1];
            const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) dsum = dot2<CT>(w[i], pack2<CT>(xr[i], xi[i]), dsum);
        }
        if constexpr (CT == CT_F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ((float4*)dst)[i] = make_float4(xr[2 * i], xi[2 * i], xr[2 * i + 1], xi[2 * i + 1]);
        } else {
            uint4 w0, w1;
            w0.x = pack2<CT>(xr[0], xi[0]); w0.y = pack2<CT>(xr[1], xi[1]);
            w0.z = pack2<CT>(xr[2], xi[2]); w0.w = pack2<CT>(xr[3], xi[3]);
            w1.x = pack2<CT>(xr[4], xi[4]); w1.y = pack2<CT>(xr[5], xi[5]);
            w1.z = pack2<CT>(xr[6], xi[6]); w1.w = pack2<CT>(xr[7], xi[7]);
            ((uint4*)dst)[0] = w0;
            ((uint4*)dst)[1] = w1;
        }
    };
    // P1: F1 (radix R over n1 < R/2), this wave's column blocks, V -> XY
    auto P1 = [&]() LCV_INLINE {
        MatImg<CT> img1[RB1][KC1];
        static_for<0, RB1>([&](auto rr) LCV_INLINE {
            static_for<0, KC1>([&](auto kk) LCV_INLINE {
                img1[decltype(rr)::value][decltype(kk)::value] = F1(decltype(rr)::value, decltype(kk)::value);
            });
        });
#pragma unroll 1
        for (int b0 = 0; b0 < BPW; ++b0) {
            const int blk = wave * BPW + b0, p = blk >> 4, b = blk & 15;
            Operand<CT> din[KC1];
            static_for<0, KC1>([&](auto kk) LCV_INLINE {
                constexpr int kc = decltype(kk)::value;
                din[kc] = lds_operand<CT>(V, [&](int j) {
                    const int n1 = 16 * kc + 4 * g + j;
                    return n1 < NH ? (p * NH + n1) * SV + 16 * b + c : -1;
                });
            });
            static_for<0, RB1>([&](auto rr) LCV_INLINE {
                constexpr int rb_ = decltype(rr)::value;
                Tile acc;
                acc.re = f32x4{0.f, 0.f, 0.f, 0.f};
                acc.im = f32x4{0.f, 0.f, 0.f, 0.f};
                static_for<0, KC1>([&](auto kk) LCV_INLINE {
                    constexpr int kc = decltype(kk)::value;
                    stage_keep_acc<CT>(img1[rb_][kc], din[kc], acc.re, acc.im);
                });
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k1 = 16 * rb_ + 4 * g + j;
                    if (k1 < R) lds_put<CT>(XY, (p * R + k1) * ST + b * SR + c, acc.re[j], acc.im[j]);
                }
            });
        }
    };
    // P2 (forward half): this wave's four tiles from XY, then F2, twiddle, F3 in registers.
    // A barrier follows the LDS reads: XY is free for the next half once every wave has read.
    Tile xs[4];
    auto P2f = [&]() LCV_INLINE {
        Operand<CT> opd[4];
        static_for<0, 4>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            const int t = wave * 4 + i;
            opd[i] = lds_operand<CT>(XY, [&](int j) { return t * ST + (4 * g + j) * SR + c; });
        });
        __syncthreads();
        static_for<0, 4>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            xs[i] = stage_swap<CT>(F2(i), opd[i]);   // (L = k2, K = n3)
            cmul4(xs[i], twr, twi);
            opd[i] = to_operand<CT>(xs[i]);
            xs[i] = stage_keep<CT>(F3(i), opd[i]);   // (L = k2, K = k3)
        });
    };

    const bool want_dk = a.y != nullptr, want_dd = a.y2 != nullptr;
    using X_ = std::integral_constant<bool, false>;
    using DS_ = std::integral_constant<bool, true>;
    issue(X_{}, first, 0);
    for (int64_t it0 = first; it0 < last; it0 += P) {
        dsum = 0.f;
        Tile acc[4], zx[4];
        static_for<0, 4>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            acc[i].re = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[i].im = f32x4{0.f, 0.f, 0.f, 0.f};
        });
#pragma unroll 1
        for (int64_t j = 0; j < Bp; ++j) {
            // ---- x = q u: spectrum kept in registers
            P0(X_{}, it0, j);
            issue(DS_{}, it0, j);
            P1();
            __syncthreads();
            P2f();
            static_for<0, 4>([&](auto ii) LCV_INLINE { zx[decltype(ii)::value] = xs[decltype(ii)::value]; });
            // ---- ds = dy v: accumulate conj(Zx) Zds
            P0(DS_{}, it0, j);
            // next: the following pair of this channel group, or the first pair of the next group
            if (j + 1 < Bp) issue(X_{}, it0, j + 1);
            else issue(X_{}, it0 + P < last ? it0 + P : it0, 0);
            P1();
            __syncthreads();
            P2f();
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                acc[i].re += zx[i].re * xs[i].re + zx[i].im * xs[i].im;
                acc[i].im += zx[i].re * xs[i].im - zx[i].im * xs[i].re;
            });
        }
        // ---- inverse of the spectral sum (scaled by 1/M): I1, twiddle, I2 -> XY
        static_for<0, 4>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            const int t = wave * 4 + i, k1 = t % R;
            Tile z = acc[i];
            z.re *= a.inv_m;
            z.im *= a.inv_m;
            Operand<CT> opd = to_operand<CT>(z);
            z = stage_swap<CT>(load_img<CT>(tab + T_I1, k1, lane), opd);   // (L = n3, K = k2)
            cmulc4(z, twr, twi);
            opd = to_operand<CT>(z);
            z = stage_keep<CT>(load_img<CT>(tab + T_I2, k1, lane), opd);   // (L = n3, K = n2)
#pragma unroll
            for (int j = 0; j < 4; ++j) lds_put<CT>(XY, t * ST + (4 * g + j) * SR + c, z.re[j], z.im[j]);
        });
        __syncthreads();
        // ---- I3 (inverse radix R over k1, rows n1 < R/2), this wave's blocks, XY -> O
        {
            MatImg<CT> img3[RB3][KC3];
            static_for<0, RB3>([&](auto rr) LCV_INLINE {
                static_for<0, KC3>([&](auto kk) LCV_INLINE {
                    img3[decltype(rr)::value][decltype(kk)::value] = I3(decltype(rr)::value, decltype(kk)::value);
                });
            });
#pragma unroll 1
            for (int b0 = 0; b0 < BPW; ++b0) {
                const int blk = wave * BPW + b0, p = blk >> 4, b = blk & 15;
                Operand<CT> din[KC3];
                static_for<0, KC3>([&](auto kk) LCV_INLINE {
                    constexpr int kc = decltype(kk)::value;
                    din[kc] = lds_operand<CT>(XY, [&](int j) {
                        const int k1 = 16 * kc + 4 * g + j;
                        return k1 < R ? (p * R + k1) * ST + b * SR + c : -1;
                    });
                });
                static_for<0, RB3>([&](auto rr) LCV_INLINE {
                    constexpr int rb_ = decltype(rr)::value;
                    Tile o;
                    o.re = f32x4{0.f, 0.f, 0.f, 0.f};
                    o.im = f32x4{0.f, 0.f, 0.f, 0.f};
                    static_for<0, KC3>([&](auto kk) LCV_INLINE {
                        constexpr int kc = decltype(kk)::value;
                        stage_keep_acc<CT>(img3[rb_][kc], din[kc], o.re, o.im);
                    });
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n1 = 16 * rb_ + 4 * g + j;
                        if (n1 < NH) *(float2*)(O + 2 * ((p * NH + n1) * SO + 16 * b + c)) = make_float2(o.re[j], o.im[j]);
                    }
                });
            }
        }
        // ---- dk: real part of this lane's slot (wave-local O), and dD = dk[0]
        {
            const int64_t h = it0 + p_io;
            const float4* src = (const float4*)(O + 2 * ((p_io * NH + (n0_io >> 8)) * SO + (n0_io & 255)));
            float d[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 w = src[i];
                d[2 * i] = w.x;
                d[2 * i + 1] = w.z;
            }
            if (h < last && n0_io < a.N) {
                if (want_dk) {
                    float4* dst = (float4*)((float*)a.y + h * a.N + n0_io);
                    dst[0] = make_float4(d[0], d[1], d[2], d[3]);
                    dst[1] = make_float4(d[4], d[5], d[6], d[7]);
                }
                if (!LAG0 && want_dd && n0_io == 0) ((float*)a.y2)[h] = d[0];
            }
        }
        // ---- lag 0 again, as the direct sum of x ds over the channel's rows (fp32; x as the
        // transform input held it): the spectral sum's rounding can cancel there.  Summed per
        // channel over the lanes in a fixed order; dk[h][0] (stored above) is overwritten after
        // the barrier.
        if constexpr (LAG0) {
            // each 32-lane half of a wave holds slots of one channel: sum the half (fixed
            // shuffle order), then per channel the halves in order
            float v = dsum;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off, 64);
            if ((lane & 31) == 0) red[2 * wave + (lane >> 5)] = v;
            __syncthreads();
            if (tid < P && it0 + tid < last) {
                const int64_t h = it0 + tid;
                float sum = 0.f;
                for (int e = 0; e < 16; ++e) {
                    const int bl = (e >> 1) * BPW + ((32 * (e & 1)) >> 1) % BPW;  // the half's first slot (slot())
                    if ((bl >> 4) == tid) sum += red[e];
                }
                if (want_dk) ((float*)a.y)[h * a.N] = sum;
                if (want_dd) ((float*)a.y2)[h] = sum;
            }
            __syncthreads();
        }
    }
}

template <int R, int CT, int IO, bool GQ, bool GV>
static hipError_t launch_dk_t(const Fused1DArgs& a0, int cus, hipStream_t st) {
    Fused1DArgs a = a0;
    constexpr int P = 32 / R;
    if (a.nitems <= 0) return hipSuccess;
    const int64_t groups = (a.nitems + P - 1) / P;
    int64_t nwg = groups < cus ? groups : cus;
    const int64_t gpw = (groups + nwg - 1) / nwg;
    a.per_wg = gpw * P;
    nwg = (a.nitems + a.per_wg - 1) / a.per_wg;
    hipLaunchKernelGGL((dk1d_kernel<R, CT, IO, GQ, GV>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    return hipGetLastError();
}

template <int R, int T>
static hipError_t launch_dk_g(bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t st) {
    if (gq && gv) return launch_dk_t<R, T, T, true, true>(a, cus, st);
    if (gq) return launch_dk_t<R, T, T, true, false>(a, cus, st);
    if (gv) return launch_dk_t<R, T, T, false, true>(a, cus, st);
    return launch_dk_t<R, T, T, false, false>(a, cus, st);
}

template <int R>
static hipError_t launch_dk_r(int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t st) {
    if (dtype == CT_F32) return launch_dk_g<R, CT_F32>(gq, gv, a, cus, st);
    if (dtype == CT_F16) return launch_dk_g<R, CT_F16>(gq, gv, a, cus, st);
    return launch_dk_g<R, CT_BF16>(gq, gv, a, cus, st);
}

hipError_t launch_dk1d(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t stream) {
    switch (R) {
    case 2: return launch_dk_r<2>(dtype, gq, gv, a, cus, stream);
    case 4: return launch_dk_r<4>(dtype, gq, gv, a, cus, stream);
    case 8: return launch_dk_r<8>(dtype, gq, gv, a, cus, stream);
    case 16: return launch_dk_r<16>(dtype, gq, gv, a, cus, stream);
    case 32: return launch_dk_r<32>(dtype, gq, gv, a, cus, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace lcv
