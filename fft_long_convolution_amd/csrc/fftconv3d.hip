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

// ---- matrix-core passes: 16-bit compute types, S = 32 (P = 64) -------------------------------
// Every DFT is the dense 64-point matrix in blocks of 16 x 16 (dense_dft_tables): forward inputs
// are half zero and inverse outputs are kept only in the window (rows 16 .. 47), so each transform
// uses half of its blocks, held in registers.  A tile is 16 x 16 complex values, lane (g, c)
// holding rows 4 g + j of column c (the operand and result layout of lconv_device.h); a stage
// with the data as the second operand keeps that layout, one with the data as the first operand
// transposes it, which turns the row DFT's output into the column DFT's input without a trip
// through LDS.  Along kx a lane holds two adjacent columns, 2 c and 2 c + 1 of a 32-column group
// kp, in two tiles (parity par): every workspace row access moves whole 128-byte lines.  Where a
// transform produces or contracts that interleaved kx order it uses the interleaved blocks.
// Each wave works on its own slices or rows: no LDS and no barrier.
// (The digit split of "FlashFFTConv" (abstract) and the "FlashConv" page's Mechanism, with the
// whole 64-point DFT as one matrix: at this size the blocks are cheaper than a second split.)
constexpr int M3_S = 32, M3_P = 64;
constexpr int M3_ZW = 2;  // slices per wave (passes A and C)
// (ky, 32-column group) rows per wave (pass Z): 4 gives 8 workgroups per unit, so workgroup ids
// of the two units of a channel differ by a multiple of 8 and the dispatcher puts them on one
// XCD, whose L2 then serves the channel's spectrum to both
constexpr int M3_TZ = 4;

template <int CT>
__device__ __forceinline__ MatImg<CT> img_f(const void* img, int kb, int nb, int lane) {
    return load_img<CT>(img, 4 * kb + nb, lane);
}
template <int CT>
__device__ __forceinline__ MatImg<CT> img_i(const void* img, int mb, int kb, int lane) {
    return load_img<CT>(img, 16 + 4 * mb + kb, lane);
}
// interleaved: forward rows kx = 32 kp + 2 r + par (kq = 2 kp + par); inverse inputs likewise
template <int CT>
__device__ __forceinline__ MatImg<CT> img_fq(const void* img, int kq, int nb, int lane) {
    return load_img<CT>(img, 32 + 4 * kq + nb, lane);
}
template <int CT>
__device__ __forceinline__ MatImg<CT> img_iq(const void* img, int mb, int kq, int lane) {
    return load_img<CT>(img, 48 + 4 * mb + kq, lane);
}

// Pass A: per input slice z, DFT over x then over y, into W[z][ky][kx].
template <int CT>
__global__ void __launch_bounds__(256) k3m_slices_fwd(const Conv3DArgs a) {
    constexpr int S = M3_S, P = M3_P;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    const int64_t ul = blockIdx.y, unit = a.unit0 + ul;
    int64_t ch, row0, row1;
    unit_rows(a, unit, (int64_t)S * S * S, ch, row0, row1);
    MatImg<CT> Fq[4][2], F[4][2];  // x: interleaved kx rows (kq), inputs x < S; y: rows ky, inputs y < S
    static_for<0, 4>([&](auto kk) LCV_INLINE {
        static_for<0, 2>([&](auto nn) LCV_INLINE {
            constexpr int k = decltype(kk)::value, n = decltype(nn)::value;
            Fq[k][n] = img_fq<CT>(a.img, k, n, lane);
            F[k][n] = img_f<CT>(a.img, k, n, lane);
        });
    });
    const uint16_t* const ua = (const uint16_t*)a.u + row0;
    const uint16_t* const ub = (const uint16_t*)a.u + (row1 >= 0 ? row1 : row0);
#pragma unroll 1
    for (int zi = 0; zi < M3_ZW; ++zi) {
        const int z = (blockIdx.x * 4 + wave) * M3_ZW + zi;
        // d(xb, yb): rows x = 16 xb + 4 g + j, column y = 16 yb + c; the two images as re, im
        Operand<CT> d[2][2];
        static_for<0, 2>([&](auto xx) LCV_INLINE {
            static_for<0, 2>([&](auto yy) LCV_INLINE {
                constexpr int xb = decltype(xx)::value, yb = decltype(yy)::value;
                const int64_t off = ((int64_t)z * S + 16 * yb + c) * S + 16 * xb + 4 * g;
                const uint2 pa = *(const uint2*)(ua + off);
                const uint2 pb = row1 >= 0 ? *(const uint2*)(ub + off) : make_uint2(0u, 0u);
                d[xb][yb].w[0] = __byte_perm(pa.x, pb.x, 0x5410);
                d[xb][yb].w[1] = __byte_perm(pa.x, pb.x, 0x7632);
                d[xb][yb].w[2] = __byte_perm(pa.y, pb.y, 0x5410);
                d[xb][yb].w[3] = __byte_perm(pa.y, pb.y, 0x7632);
            });
        });
        // DFT over x, transposed: x1(yb, kq) holds rows y, column kx = 32 kp + 2 c + par
        Operand<CT> x1[2][4];
        static_for<0, 2>([&](auto yy) LCV_INLINE {
            static_for<0, 4>([&](auto kk) LCV_INLINE {
                constexpr int yb = decltype(yy)::value, kq = decltype(kk)::value;
                f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                stage_swap_acc<CT>(Fq[kq][0], d[0][yb], re, im);
                stage_swap_acc<CT>(Fq[kq][1], d[1][yb], re, im);
                x1[yb][kq] = to_operand<CT>(tile_from_acc(re, im));
            });
        });
        // DFT over y: rows ky, columns 2 c, 2 c + 1 of group kp; stored as W[z][ky][kx]
        uint32_t* const wz = (uint32_t*)a.ws + (ul * S + z) * P * P;
        static_for<0, 2>([&](auto pp) LCV_INLINE {
            static_for<0, 4>([&](auto yy) LCV_INLINE {
                constexpr int kp = decltype(pp)::value, kyb = decltype(yy)::value;
                f32x4 re[2], im[2];
                static_for<0, 2>([&](auto qq) LCV_INLINE {
                    constexpr int par = decltype(qq)::value;
                    re[par] = f32x4{0.f, 0.f, 0.f, 0.f};
                    im[par] = f32x4{0.f, 0.f, 0.f, 0.f};
                    stage_keep_acc<CT>(F[kyb][0], x1[0][2 * kp + par], re[par], im[par]);
                    stage_keep_acc<CT>(F[kyb][1], x1[1][2 * kp + par], re[par], im[par]);
                });
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(uint2*)(wz + (16 * kyb + 4 * g + j) * P + 32 * kp + 2 * c) =
                        make_uint2(pack2<CT>(re[0][j], im[0][j]), pack2<CT>(re[1][j], im[1][j]));
            });
        });
    }
}

// Pass Z: per row (ky, 32-column group kp), DFT over z, product with (K + D (-i)^(kx+ky+kz)) / P^3,
// inverse DFT for the window slices, written back to W[zo][ky][kx] (the row's own elements).
template <int CT>
__global__ void __launch_bounds__(256) k3m_zpass(const Conv3DArgs a) {
    constexpr int S = M3_S, P = M3_P;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    const int64_t ul = blockIdx.y, unit = a.unit0 + ul;
    int64_t ch, row0, row1;
    unit_rows(a, unit, (int64_t)S * S * S, ch, row0, row1);
    MatImg<CT> F[4][2], Fi[2][4];  // forward (kz block, z block < 2); inverse (window block, kz block)
    static_for<0, 4>([&](auto kk) LCV_INLINE {
        constexpr int k = decltype(kk)::value;
        static_for<0, 2>([&](auto nn) LCV_INLINE {
            constexpr int n = decltype(nn)::value;
            F[k][n] = img_f<CT>(a.img, k, n, lane);
            Fi[n][k] = img_i<CT>(a.img, 1 + n, k, lane);
        });
    });
    const float dsk = raw1_to_f32<CT>(load1_raw<CT>(a.D, ch)) * a.inv_p3;
    constexpr uint32_t P2 = P * P;
    // scalar bases per row, 32-bit lane offsets (slice 4 g + j, columns 2 c, 2 c + 1) fixed for
    // the wave
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lo = (uint32_t)(4 * g) * P2 + 2 * (uint32_t)c;
    uint32_t* const wsu = (uint32_t*)a.ws + ul * S * P2;
    const uint32_t* const kfc = (const uint32_t*)a.kf + ch * P * P2;
#pragma unroll 1
    for (int ti = 0; ti < M3_TZ; ++ti) {
        const int task = (blockIdx.x * 4 + wv) * M3_TZ + ti;  // < 128, wave-uniform
        const int ky = task >> 1, kx0 = 32 * (task & 1);
        uint32_t* const wr = wsu + ky * P + kx0;          // + z P^2 + lane offset
        const uint32_t* const kr = kfc + ky * P + kx0;    // + kz P^2 + lane offset
        Operand<CT> w[2][2];   // [par][z block]
        static_for<0, 2>([&](auto zz) LCV_INLINE {
            constexpr int zb = decltype(zz)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint2 t = *(const uint2*)(wr + lo + (uint32_t)(16 * zb + j) * P2);
                w[0][zb].w[j] = t.x;
                w[1][zb].w[j] = t.y;
            }
        });
        uint2 kw[4][4];
        static_for<0, 4>([&](auto kk) LCV_INLINE {
            constexpr int kzb = decltype(kk)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j) kw[kzb][j] = *(const uint2*)(kr + lo + (uint32_t)(16 * kzb + j) * P2);
        });
        f32x4 yr[2][2], yi[2][2];  // [par][window block]
        static_for<0, 2>([&](auto qq) LCV_INLINE {
            constexpr int par = decltype(qq)::value;
            const int kx = kx0 + 2 * c + par;
            yr[par][0] = yr[par][1] = yi[par][0] = yi[par][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            // per kz block: forward, product, and its share of both window blocks of the inverse
            static_for<0, 4>([&](auto kk) LCV_INLINE {
                constexpr int kzb = decltype(kk)::value;
                f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                stage_keep_acc<CT>(F[kzb][0], w[par][0], re, im);
                stage_keep_acc<CT>(F[kzb][1], w[par][1], re, im);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // the skip: a delta at the kernel centre, spectrum (-i)^(kx + ky + kz)
                    const int ph = (kx + ky + 16 * kzb + 4 * g + j) & 3;
                    const uint32_t kv = par ? kw[kzb][j].y : kw[kzb][j].x;
                    const float kre = unpack_lo<CT>(kv) + (ph == 0 ? dsk : ph == 2 ? -dsk : 0.f);
                    const float kim = unpack_hi<CT>(kv) + (ph == 1 ? -dsk : ph == 3 ? dsk : 0.f);
                    float xr = re[j], xi = im[j];
                    cmul(xr, xi, kre, kim);
                    re[j] = xr;
                    im[j] = xi;
                }
                const Operand<CT> zp = to_operand<CT>(tile_from_acc(re, im));
                stage_keep_acc<CT>(Fi[0][kzb], zp, yr[par][0], yi[par][0]);
                stage_keep_acc<CT>(Fi[1][kzb], zp, yr[par][1], yi[par][1]);
            });
        });
        static_for<0, 2>([&](auto mm) LCV_INLINE {
            constexpr int mb = decltype(mm)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j)  // slice zo = 16 mb + 4 g + j
                *(uint2*)(wr + lo + (uint32_t)(16 * mb + j) * P2) =
                    make_uint2(pack2<CT>(yr[0][mb][j], yi[0][mb][j]), pack2<CT>(yr[1][mb][j], yi[1][mb][j]));
        });
    }
}

// Pass C: per window slice zo, inverse DFT over ky (window rows), then over kx (window columns),
// and the store of both images.
template <int CT>
__global__ void __launch_bounds__(256) k3m_slices_inv(const Conv3DArgs a) {
    constexpr int S = M3_S, P = M3_P;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    const int64_t ul = blockIdx.y, unit = a.unit0 + ul;
    int64_t ch, row0, row1;
    unit_rows(a, unit, (int64_t)S * S * S, ch, row0, row1);
    MatImg<CT> Fi[2][4], Fiq[2][4];  // inverse (window block, k block); the same over interleaved kx
    static_for<0, 2>([&](auto mm) LCV_INLINE {
        static_for<0, 4>([&](auto kk) LCV_INLINE {
            constexpr int m = decltype(mm)::value, k = decltype(kk)::value;
            Fi[m][k] = img_i<CT>(a.img, 1 + m, k, lane);
            Fiq[m][k] = img_iq<CT>(a.img, 1 + m, k, lane);
        });
    });
    uint16_t* const ya = (uint16_t*)a.y + row0;
    uint16_t* const yb2 = (uint16_t*)a.y + (row1 >= 0 ? row1 : row0);
#pragma unroll 1
    for (int zi = 0; zi < M3_ZW; ++zi) {
        const int zo = (blockIdx.x * 4 + wave) * M3_ZW + zi;
        const uint32_t* const wz = (const uint32_t*)a.ws + (ul * S + zo) * P * P;
        // inverse DFT over ky, transposed: y1(kq, myb) holds rows kx = 32 kp + 2 (4 g + j) + par,
        // column my (window)
        Operand<CT> y1[4][2];
        static_for<0, 2>([&](auto pp) LCV_INLINE {
            constexpr int kp = decltype(pp)::value;
            Operand<CT> w[2][4];  // [par][ky block]: rows ky = 16 kyb + 4 g + j, column 32 kp + 2 c + par
            static_for<0, 4>([&](auto yy) LCV_INLINE {
                constexpr int kyb = decltype(yy)::value;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint2 t = *(const uint2*)(wz + (16 * kyb + 4 * g + j) * P + 32 * kp + 2 * c);
                    w[0][kyb].w[j] = t.x;
                    w[1][kyb].w[j] = t.y;
                }
            });
            static_for<0, 2>([&](auto qq) LCV_INLINE {
                static_for<0, 2>([&](auto mm) LCV_INLINE {
                    constexpr int par = decltype(qq)::value, myb = decltype(mm)::value;
                    f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                    static_for<0, 4>([&](auto yy) LCV_INLINE {
                        stage_swap_acc<CT>(Fi[myb][decltype(yy)::value], w[par][decltype(yy)::value], re, im);
                    });
                    y1[2 * kp + par][myb] = to_operand<CT>(tile_from_acc(re, im));
                });
            });
        });
        // inverse DFT over kx (interleaved blocks): rows mx (window), column my; image A is the
        // real part, B the imaginary part: lane (g, c) stores x = 16 mxb + 4 g .. + 3 of row
        // y = 16 myb + c
        static_for<0, 2>([&](auto xx) LCV_INLINE {
            static_for<0, 2>([&](auto mm) LCV_INLINE {
                constexpr int mxb = decltype(xx)::value, myb = decltype(mm)::value;
                f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                static_for<0, 4>([&](auto kk) LCV_INLINE {
                    stage_keep_acc<CT>(Fiq[mxb][decltype(kk)::value], y1[decltype(kk)::value][myb], re, im);
                });
                const int64_t off = ((int64_t)zo * S + 16 * myb + c) * S + 16 * mxb + 4 * g;
                *(uint2*)(ya + off) = make_uint2(pack2<CT>(re[0], re[1]), pack2<CT>(re[2], re[3]));
                if (row1 >= 0) *(uint2*)(yb2 + off) = make_uint2(pack2<CT>(im[0], im[1]), pack2<CT>(im[2], im[3]));
            });
        });
    }
}

template <int S, int CT, int IO>
static hipError_t launch3_t(const Conv3DArgs& a, hipStream_t st) {
    if (a.nunit <= 0) return hipSuccess;
    const dim3 blk(256);
    if constexpr (S == M3_S && CT != CT_F32) {
        if (!a.filter && a.img) {
            hipLaunchKernelGGL((k3m_slices_fwd<CT>), dim3(S / (4 * M3_ZW), (unsigned)a.nunit), blk, 0, st, a);
            hipLaunchKernelGGL((k3m_zpass<CT>), dim3(M3_P * 2 / (4 * M3_TZ), (unsigned)a.nunit), blk, 0, st, a);
            hipLaunchKernelGGL((k3m_slices_inv<CT>), dim3(S / (4 * M3_ZW), (unsigned)a.nunit), blk, 0, st, a);
            return hipGetLastError();
        }
    }
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
