// colmx.hip -- the column passes of the chunked long-sequence path on the matrix cores, for
// 16-bit types and column lengths P = M1 = 256, 512 and 1024 (transform lengths 2^21 .. 2^23).
//
// The passes compute what multipass.hip's column passes compute (A: the column DFT over
// n_hi < P/2 and the four-step twiddle, to the workspace; C: the inverse twiddle, the inverse
// column DFT for the kept rows n_hi < P/2, the gate and the store), with the P-point column
// DFT factored once more, n_hi = 16 n1 + n2 and k_hi = k1 + R k2 (R = P / 16):
//     X[k1 + R k2] = sum_{n2} w16^{n2 k2} w_P^{n2 k1} sum_{n1 < R/2} w_R^{n1 k1} x[16 n1 + n2]
//     y[16 n1 + n2] = sum_{k1} w_R^{-n1 k1} w_P^{-n2 k1} sum_{k2} w16^{-n2 k2} Z[k1 + R k2]
// Both factors are dense DFT blocks on the matrix cores ("FlashFFTConv" abstract; "FlashConv"
// page, Mechanism), as 16 x 16 complex tiles of v_mfma_f32_16x16x32_{bf16,f16} whose L index
// is 16 consecutive columns of the block (the tile layout of lconv_device.h).  The w_P twiddle
// runs on the vector ALU between the two stages, and one LDS exchange moves the contracted
// digit from n1 to n2 (forward) or from k2 to k1 (inverse).  Global rows go straight between
// memory and tile registers: one tile instruction touches 16 consecutive columns of 4 rows.
//
// A workgroup owns CB = 16384 / P consecutive columns of one sequence; workgroups whose columns
// share 128-byte lines of a 16-bit row are placed on one XCD (the dispatcher deals workgroup ids
// round-robin over the 8 XCDs), so that XCD's L2 fetches each line once.
#include "coldft.h"
#include "fused_io.h"
#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

namespace {

constexpr int64_t kRow = 8192;

template <int P>
struct Cm {
    static constexpr ColMxGrid G = colmx_grid(P);
    static constexpr int R = G.R, H = G.H, RB = G.rbk, HB = G.hb;
    static constexpr int CB = 16384 / P, NCG = CB / 16;  // columns, 16-column groups
    static constexpr int S = CB < 64 ? 64 / CB : 1;      // workgroups per 128-byte line of a 16-bit row
    static constexpr int YC = 17 * R + 1;                // LDS words per 4 columns, / 4 (odd)
    static constexpr int ZC = 16 * (R + 1) + 1;
};

// First column of this workgroup: ids 8S m + 8 t + x (x < 8, t < S) take the blocks
// 8S m + S x + t, so the S blocks of one line go to XCD x one after another.
template <int P>
__device__ __forceinline__ int64_t block_col0() {
    constexpr int S = Cm<P>::S, GRP = 8 * S;
    const int bx = blockIdx.x;
    return (int64_t)(GRP * (bx / GRP) + S * (bx % 8) + (bx / 8) % S) * Cm<P>::CB;
}

// LDS word of (column c of the block, k1, n2) in the forward exchange and of (c, n2, k1) in the
// inverse one.  Four columns interleave word by word, and the per-4-column stride is odd: the
// stage-1 tile writes (lanes over c and the tile's output digit 4g + j) and the stage-2 operand
// reads (lanes over c and the contracted digit 4g + j) both hit 64 distinct banks.
template <int P>
__device__ __forceinline__ int yaddr(int c, int k1, int n2) {
    return (c & 3) + 4 * ((c >> 2) * Cm<P>::YC + 17 * k1 + n2);
}
template <int P>
__device__ __forceinline__ int zaddr(int c, int n2, int k1) {
    return (c & 3) + 4 * ((c >> 2) * Cm<P>::ZC + (Cm<P>::R + 1) * n2 + k1);
}

template <int CT>
__device__ __forceinline__ void store1h(void* p, int64_t i, float v) {
    ((uint16_t*)p)[i] = (uint16_t)(pack2<CT>(v, 0.f) & 0xffffu);
}

template <int CT, int P>
__global__ void __launch_bounds__(512, 2) colmx_fwd_kernel(const ColArgs a) {
    using C = Cm<P>;
    constexpr int R = C::R, H = C::H, RB = C::RB, HB = C::HB, NCG = C::NCG;
    __shared__ uint32_t Y[C::CB * C::YC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, x = lane & 15;
    const int64_t s = blockIdx.y, n_lo0 = block_col0<P>();
    int64_t row0, row1;
    seq_rows(a, a.seq0 + s, row0, row1);
    const float2* twc = (const float2*)a.tw_col;

    // Stage 1, per (n2, 16-column group): radix R over n1 < H (gated pairs packed as complex
    // x_b + i x_{b+1}), times w_P^{n2 k1}, into the exchange.
    MatImg<CT> f1[RB][HB];
    static_for<0, RB>([&](auto rb) LCV_INLINE {
        static_for<0, HB>([&](auto kc) LCV_INLINE {
            f1[rb][kc] = load_img<CT>(a.img, C::G.f1 + decltype(rb)::value * HB + decltype(kc)::value, lane);
        });
    });
    static_for<0, 2 * NCG>([&](auto ii) LCV_INLINE {
        const int u = wave + 8 * decltype(ii)::value, n2 = u & 15, c = 16 * (u >> 4) + x;
        const int64_t col = n_lo0 + c;
        Operand<CT> op[HB];
        static_for<0, HB>([&](auto kk) LCV_INLINE {
            constexpr int kc = decltype(kk)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n1 = 16 * kc + 4 * g + j;
                const int64_t n = kRow * (16 * n1 + n2) + col;
                const bool ok = n1 < H && n < a.N;
                const int64_t e = ok ? n : col;  // a valid element of the same rows
                float re = load1<CT>(a.u, row0 + e), im = 0.f;
                if (a.q) re *= load1<CT>(a.q, row0 + e);
                if (row1 >= 0) {
                    im = load1<CT>(a.u, row1 + e);
                    if (a.q) im *= load1<CT>(a.q, row1 + e);
                }
                op[kc].w[j] = ok ? pack2<CT>(re, im) : 0u;
            }
        });
        static_for<0, RB>([&](auto r) LCV_INLINE {
            constexpr int rb = decltype(r)::value;
            f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
            static_for<0, HB>([&](auto kk) LCV_INLINE {
                stage_keep_acc<CT>(f1[rb][decltype(kk)::value], op[decltype(kk)::value], re, im);
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k1 = 16 * rb + 4 * g + j;
                const float2 w = twc[n2 * k1];  // n2 k1 < P
                float xr = re[j], xi = im[j];
                cmul(xr, xi, w.x, w.y);
                Y[yaddr<P>(c, k1, n2)] = pack2<CT>(xr, xi);
            }
        });
    });
    __syncthreads();

    // Stage 2, per (k1, 16-column group): 16-point DFT over n2, the four-step twiddle
    // w_M^{n_lo k_hi}, store rows k_hi = k1 + R k2 of the workspace.
    const MatImg<CT> f16 = load_img<CT>(a.img, C::G.f16, lane);
    const int64_t mask = a.M - 1;
    uint32_t* ws = (uint32_t*)a.ws;
    static_for<0, R * NCG / 8>([&](auto ii) LCV_INLINE {
        const int u = wave + 8 * decltype(ii)::value, k1 = u % R, c = 16 * (u / R) + x;
        const int64_t n_lo = n_lo0 + c;
        Operand<CT> op;
#pragma unroll
        for (int j = 0; j < 4; ++j) op.w[j] = Y[yaddr<P>(c, k1, 4 * g + j)];
        Tile t = stage_keep<CT>(f16, op);  // rows k2 = 4 g + j
        float2 w = tw_m(a.tw_lo, a.tw_hi, (n_lo * (k1 + 4 * g * R)) & mask);
        const float2 st = tw_m(a.tw_lo, a.tw_hi, (n_lo * R) & mask);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float xr = t.re[j], xi = t.im[j];
            cmul(xr, xi, w.x, w.y);
            w = cmulf(w, st);
            ws[(s * P + k1 + R * (4 * g + j)) * kRow + n_lo] = pack2<CT>(xr, xi);
        }
    });
}

template <int CT, int P>
__global__ void __launch_bounds__(512, 2) colmx_inv_kernel(const ColArgs a) {
    using C = Cm<P>;
    constexpr int R = C::R, H = C::H, RB = C::RB, HB = C::HB, NCG = C::NCG;
    __shared__ uint32_t Z[C::CB * C::ZC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, x = lane & 15;
    const int64_t s = blockIdx.y, n_lo0 = block_col0<P>();
    int64_t row0, row1;
    seq_rows(a, a.seq0 + s, row0, row1);
    const float2* twc = (const float2*)a.tw_col;
    const int64_t mask = a.M - 1;
    const uint32_t* ws = (const uint32_t*)a.ws;

    // Stage 1, per (k1, 16-column group): rows k_hi = k1 + R k2 of the workspace, times
    // conj(w_M^{n_lo k_hi}), 16-point inverse DFT over k2, times conj(w_P^{n2 k1}), into the
    // exchange.
    const MatImg<CT> i16 = load_img<CT>(a.img, C::G.i16, lane);
    static_for<0, R * NCG / 8>([&](auto ii) LCV_INLINE {
        const int u = wave + 8 * decltype(ii)::value, k1 = u % R, c = 16 * (u / R) + x;
        const int64_t n_lo = n_lo0 + c;
        float2 w = tw_m(a.tw_lo, a.tw_hi, (n_lo * (k1 + 4 * g * R)) & mask);
        const float2 st = tw_m(a.tw_lo, a.tw_hi, (n_lo * R) & mask);
        Operand<CT> op;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t z = ws[(s * P + k1 + R * (4 * g + j)) * kRow + n_lo];
            float zr = unpack_lo<CT>(z), zi = unpack_hi<CT>(z);
            cmulc(zr, zi, w.x, w.y);
            w = cmulf(w, st);
            op.w[j] = pack2<CT>(zr, zi);
        }
        Tile t = stage_keep<CT>(i16, op);  // rows n2 = 4 g + j
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n2 = 4 * g + j;
            const float2 wc = twc[n2 * k1];
            float zr = t.re[j], zi = t.im[j];
            cmulc(zr, zi, wc.x, wc.y);
            Z[zaddr<P>(c, n2, k1)] = pack2<CT>(zr, zi);
        }
    });
    __syncthreads();

    // Stage 2, per (n2, 16-column group): inverse radix R over k1 for the kept rows n1 < H,
    // post-gate, store rows n_hi = 16 n1 + n2 (and n < N) of the output pair.
    MatImg<CT> i2[HB][RB];
    static_for<0, HB>([&](auto rb) LCV_INLINE {
        static_for<0, RB>([&](auto kc) LCV_INLINE {
            i2[rb][kc] = load_img<CT>(a.img, C::G.i2 + decltype(rb)::value * RB + decltype(kc)::value, lane);
        });
    });
    static_for<0, 2 * NCG>([&](auto ii) LCV_INLINE {
        const int u = wave + 8 * decltype(ii)::value, n2 = u & 15, c = 16 * (u >> 4) + x;
        const int64_t col = n_lo0 + c;
        Operand<CT> op[RB];
        static_for<0, RB>([&](auto kk) LCV_INLINE {
            constexpr int kc = decltype(kk)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j) op[kc].w[j] = Z[zaddr<P>(c, n2, 16 * kc + 4 * g + j)];
        });
        static_for<0, HB>([&](auto r) LCV_INLINE {
            constexpr int rb = decltype(r)::value;
            f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
            static_for<0, RB>([&](auto kk) LCV_INLINE {
                stage_keep_acc<CT>(i2[rb][decltype(kk)::value], op[decltype(kk)::value], re, im);
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n1 = 16 * rb + 4 * g + j;
                const int64_t n = kRow * (16 * n1 + n2) + col;
                const bool ok = n1 < H && n < a.N;
                const int64_t e = ok ? n : col;
                float yr = re[j], yi = im[j];
                if (a.v) yr *= load1<CT>(a.v, row0 + e);
                if (row1 >= 0 && a.v) yi *= load1<CT>(a.v, row1 + e);
                if (ok) {
                    store1h<CT>(a.y, row0 + n, yr);
                    if (row1 >= 0) store1h<CT>(a.y, row1 + n, yi);
                }
            }
        });
    });
}

template <int CT, int P>
hipError_t launch_t(bool fwd, const ColArgs& a, hipStream_t st) {
    static_assert(kRow / Cm<P>::CB % (8 * Cm<P>::S) == 0, "the XCD order needs whole groups");
    const dim3 grid((unsigned)(kRow / Cm<P>::CB), (unsigned)a.nseq);
    if (fwd) hipLaunchKernelGGL((colmx_fwd_kernel<CT, P>), grid, dim3(512), 0, st, a);
    else hipLaunchKernelGGL((colmx_inv_kernel<CT, P>), grid, dim3(512), 0, st, a);
    return hipGetLastError();
}

template <int CT>
hipError_t launch_ct(bool fwd, const ColArgs& a, hipStream_t st) {
    switch (a.M1) {
    case 256: return launch_t<CT, 256>(fwd, a, st);
    case 512: return launch_t<CT, 512>(fwd, a, st);
    case 1024: return launch_t<CT, 1024>(fwd, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_colmx(bool fwd, int dtype, const ColArgs& a, hipStream_t st) {
    if (a.nseq <= 0) return hipSuccess;
    if (!a.img || a.filter || a.nseq > 65535 || a.M != a.M1 * kRow) return hipErrorInvalidValue;
    if (dtype == CT_F16) return launch_ct<CT_F16>(fwd, a, st);
    if (dtype == CT_BF16) return launch_ct<CT_BF16>(fwd, a, st);
    return hipErrorInvalidValue;
}

}  // namespace lcv
