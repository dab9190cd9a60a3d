// fftconv2d.hip -- 2D linear convolution with a centred full-size kernel (HyenaND-style).
//
// "Native Multi-Dimensional Subquadratic Operators via Input Dependent Long Convolutions"
// (abstract) applies global convolutions on the native 2D grid and fuses the FFT-convolution
// path.  For Hs x Ws images (sides up to 128) and kernels of the same size the linear
// convolution fits a 256 x 256 transform; the output is the Hs x Ws window starting at
// (Hs/2, Ws/2) of the full convolution (halves rounded down), i.e. the kernel's tap
// (Hs/2, Ws/2) is its centre.
//
// Placement in the 256 x 256 grid: the image sits at rows [0, Hs) and columns [0, Ws); the
// kernel's tap (a, e) at (64 - Hs/2 + a, 64 - Ws/2 + e).  The full convolution then lies in
// rows [64 - Hs/2, 62 + 2 Hs - Hs/2] (inside [0, 256): nothing wraps) and output (i, j) is grid
// point (64 + i, 64 + j), so every shape reads the same window rows and columns 64 .. 191.  The
// D skip is a delta at grid (64, 64).
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
// The same with the 64-blocks given: row block rb = r >> 6, column block vb = v >> 6.  A lane's
// tile accesses keep rb (rows 16 (4 g + jj) + c lie in block g) or vb (columns c + 16 (4 g + jj)
// lie in block g) fixed over jj, so the XOR term is computed once per tile, not per element.
__device__ __forceinline__ int swz_b(int rb, int v) { return v ^ (((rb ^ (v >> 6)) & 3) << 4); }

template <int IO>
__device__ __forceinline__ uint32_t ld_raw2(const void* p, int64_t i) {
    return ((const uint16_t*)p)[i];
}

}  // namespace

// SPEC: spectrum mode for the filter gradient.  The items are single images (B = 1) and S1 stops
// after the column DFT: it stores w^(u A + v Bc) conj(Z[u][v]) / P^2 to a.y in the filter spectrum's
// order, A = Hs-1 + 64 - Hs/2, Bc = Ws-1 + 64 - Ws/2 -- the spectrum of the image rotated by
// 180 degrees and placed as a kernel (conj(Z) reverses the image, the phase moves its tap (0, 0) to
// grid point (64 - Hs/2 + Hs-1, 64 - Ws/2 + Ws-1)).  No product, no inverse, no S2 / S3.
template <int CT, bool SPEC>
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
    const int Hs = a.Hs, Ws = a.Ws;
    const int64_t IMGSZ = (int64_t)Hs * Ws;

    // staged input chunk of this thread: row (tid / 16) of a 32-row quarter, elements 8*(tid%16)..
    // (zero outside the Hs x Ws image)
    const int srow = tid >> 4, scol = 8 * (tid & 15);
    uint4 pre0, pre1;  // u of image b and b+1 (next chunk)
    auto issue = [&](int64_t item, int q) LCV_INLINE {
        const int64_t ch = item / Bp, b = 2 * (item % Bp);
        const int row = 32 * q + srow;
        if (row < Hs && scol < Ws) {
            const int64_t base0 = (b * a.C + ch) * IMGSZ + (int64_t)row * Ws + scol;
            const int64_t base1 = b + 1 < a.B ? base0 + a.C * IMGSZ : base0;
            pre0 = *(const uint4*)((const uint16_t*)a.u + base0);
            pre1 = *(const uint4*)((const uint16_t*)a.u + base1);
        } else {
            pre0 = make_uint4(0u, 0u, 0u, 0u);
            pre1 = pre0;
        }
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
                // v = c + 16 (4 g + jj) has v >> 6 = g: swz flips jj by t
                const int t = ((r >> 6) ^ g) & 3;
                uint32_t* row = BUF + r * RS + c + 64 * g;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) row[16 * (jj ^ t)] = pack2<CT>(xs[i].re[jj], xs[i].im[jj]);
            });
            __syncthreads();
        }

        // ================= S1: columns: DFT, spectrum product, inverse DFT (window rows) =====
        const float dsc = SPEC ? 0.f : unpack_lo<IO>(ld_raw2<IO>(a.D, ch)) * a.inv_p2;
        for (int v0 = 32 * wave; v0 < 32 * wave + 32; v0 += 4) {
            uint4 kr4[4];
            if constexpr (!SPEC) {
                static_for<0, 4>([&](auto ii) LCV_INLINE {
                    constexpr int i = decltype(ii)::value;
                    kr4[i] = *((const uint4*)a.kf + ((ch * P2D + v0 + i) * 64 + lane));
                });
            }
            Operand<CT> opd[4];
            Tile xs[4];
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int v = v0 + i;
                Operand<CT> o;
                // rows r = 16 (4 g + jj) + c lie in 64-block g
                const uint32_t* col = BUF + (64 * g + c) * RS + swz_b(g, v);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o.w[jj] = g < 2 ? col[16 * jj * RS] : 0u;
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
            if constexpr (SPEC) {
                const int sa = Hs - 1 + 64 - Hs / 2, sb = Ws - 1 + 64 - Ws / 2;
                static_for<0, 4>([&](auto ii) LCV_INLINE {
                    constexpr int i = decltype(ii)::value;
                    const int v = v0 + i;
                    uint32_t w[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int u = c + 16 * (4 * g + jj);
                        const int idx = (u * sa + v * sb) & (P2D - 1);
                        float sn, cs;
                        sincospif(-2.0f * (float)idx / (float)P2D, &sn, &cs);  // exact argument
                        const float zr = xs[i].re[jj], zi = xs[i].im[jj];
                        w[jj] = pack2<CT>((cs * zr + sn * zi) * a.inv_p2, (sn * zr - cs * zi) * a.inv_p2);
                    }
                    *((uint4*)a.y + ((ch * P2D + v) * 64 + lane)) = make_uint4(w[0], w[1], w[2], w[3]);
                });
                continue;
            }
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
                    // window rows r = 16 (4 g + jj) + c - 64 lie in 64-block g - 1
                    uint32_t* col = BUF + (64 * (g - 1) + c) * RS + swz_b(g - 1, v);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) col[16 * jj * RS] = pack2<CT>(xs[i].re[jj], xs[i].im[jj]);
                }
            });
        }
        __syncthreads();
        if constexpr (SPEC) continue;  // the next item's S0 writes BUF only after its barriers

        // ================= S2: inverse row DFTs (window columns) ==============================
        for (int r0 = 16 * wave; r0 < 16 * wave + 16; r0 += 4) {
            Operand<CT> opd[4];
            Tile xs[4];
            static_for<0, 4>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int r = r0 + i;
                Operand<CT> o;
                // columns v = c + 16 (4 g + jj) have v >> 6 = g: swz flips jj by t
                const int t = ((r >> 6) ^ g) & 3;
                const uint32_t* row = BUF + r * RS + c + 64 * g;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o.w[jj] = row[16 * (jj ^ t)];
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
                if (r >= Hs || scol >= Ws) continue;
                uint32_t w[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = BUF[r * RS + scol + i];
                const int64_t o0 = (b * a.C + ch) * IMGSZ + (int64_t)r * Ws + scol;
                uint4 y0, y1;
                y0.x = __byte_perm(w[0], w[1], 0x5410); y0.y = __byte_perm(w[2], w[3], 0x5410);
                y0.z = __byte_perm(w[4], w[5], 0x5410); y0.w = __byte_perm(w[6], w[7], 0x5410);
                y1.x = __byte_perm(w[0], w[1], 0x7632); y1.y = __byte_perm(w[2], w[3], 0x7632);
                y1.z = __byte_perm(w[4], w[5], 0x7632); y1.w = __byte_perm(w[6], w[7], 0x7632);
                // streamed with the non-temporal hint: nothing here reads y again
                st4_nt((uint32_t*)((uint16_t*)a.y + o0), y0);
                if (has1) st4_nt((uint32_t*)((uint16_t*)a.y + o0 + a.C * IMGSZ), y1);
            }
        }
        // the next item's S0 writes STG first and BUF only after a barrier
    }
}

// 2D filter spectrum of the kernel placed at grid rows 64 - Hs/2 + a, columns 64 - Ws/2 + e:
// K[u][v] = sum_{a,e} k[a][e] w^(u (a + dr) + v (e + dc)) / P^2 (w = exp(-2 pi i / 256)),
// computed as two explicit DFT-matrix passes in fp32 (one-off, not on the convolution path),
// stored in the order the column stage reads it: [channel][v][lane][jj], u = lane%16 +
// 16 (4 (lane/16) + jj).
template <int IO>
__global__ void __launch_bounds__(256) filter2d_kernel(const void* k, void* kf, float inv_p2, int Hs, int Ws) {
    __shared__ float2 T[S2D][32];
    __shared__ float2 W[P2D];
    const int ch = blockIdx.x, vb = blockIdx.y, tid = threadIdx.x;
    const int dr = 64 - Hs / 2, dc = 64 - Ws / 2;
    for (int e = tid; e < P2D; e += blockDim.x) {
        double s, cc;
        sincospi(-2.0 * e / P2D, &s, &cc);
        W[e] = make_float2((float)cc, (float)s);
    }
    __syncthreads();
    const uint16_t* kc = (const uint16_t*)k + (int64_t)ch * Hs * Ws;
    for (int idx = tid; idx < Hs * 32; idx += blockDim.x) {
        const int ar = idx / 32, vv = idx % 32, v = 32 * vb + vv;
        float re = 0.f, im = 0.f;
        for (int e = 0; e < Ws; ++e) {
            const float x = unpack_lo<IO>(kc[ar * Ws + e]);
            const float2 w = W[(v * (e + dc)) & (P2D - 1)];
            re += x * w.x;
            im += x * w.y;
        }
        T[ar][vv] = make_float2(re, im);
    }
    __syncthreads();
    for (int idx = tid; idx < P2D * 32; idx += blockDim.x) {
        const int vv = idx / P2D, u = idx % P2D, v = 32 * vb + vv;
        float re = 0.f, im = 0.f;
        for (int ar = 0; ar < Hs; ++ar) {
            const float2 t = T[ar][vv], w = W[(u * (ar + dr)) & (P2D - 1)];
            re += t.x * w.x - t.y * w.y;
            im += t.x * w.y + t.y * w.x;
        }
        const int pos = ((16 * (u >> 6) + (u & 15)) * 4) + ((u >> 4) & 3);
        ((uint32_t*)kf)[((int64_t)ch * P2D + v) * P2D + pos] = pack2<IO>(re * inv_p2, im * inv_p2);
    }
}

// The adjoint operator's spectrum, in the same stored order: (-1)^(u+v) conj(K[u][v]).  The
// forward reads the window at grid offset 64 of an image placed at offset 0; its adjoint places
// the output gradient at 64 and reads at 0, which is the same window read of a convolution with
// the conjugate spectrum shifted by 128 = P/2 in each axis, a sign (-1)^u (-1)^v.  The skip
// term, a delta at (64, 64), maps to itself, so D is unchanged.  Both factors flip sign bits
// only (exact).  One thread per stored (re, im) word; u's parity is the lane's parity in the
// stored order ([channel][v][lane][jj], u = lane % 16 + 16 (4 (lane / 16) + jj)).
__global__ void __launch_bounds__(256) adj2d_kernel(const uint32_t* kf, uint32_t* ka, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) {
        const int pos = (int)(i & (P2D - 1)), v = (int)((i >> 8) & (P2D - 1));
        const int odd = ((pos >> 2) ^ v) & 1;    // parity of u + v
        // even: conj (flip the imaginary sign); odd: -conj (flip the real sign)
        ka[i] = kf[i] ^ (odd ? 0x00008000u : 0x80000000u);
    }
}

// dk[c][a][e] = sum_b r[b*C + c][Hs-1-a][Ws-1-e] in fp32 (ascending b): the batch sum of the
// per-image correlations, each computed as a convolution with the rotated output gradient.
template <int IO>
__global__ void __launch_bounds__(256) dk2d_sum_kernel(const void* r, float* dk, int64_t B, int64_t C, int Hs,
                                                       int Ws) {
    const int64_t img = (int64_t)Hs * Ws, total = C * img;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t c = i / img, p = i - c * img;
        const int a = (int)(p / Ws), e = (int)(p - (int64_t)a * Ws);
        const int64_t src = (int64_t)(Hs - 1 - a) * Ws + (Ws - 1 - e);
        float acc = 0.f;
        for (int64_t b = 0; b < B; ++b) acc += unpack_lo<IO>(((const uint16_t*)r)[(b * C + c) * img + src]);
        dk[i] = acc;
    }
}

// dD[c] = sum_b sum_pixels dy u in fp32: one workgroup per channel, 8 elements per 16-byte load
// (Ws is a multiple of 8, so every image starts on a 16-byte boundary), fixed-order tree reduction.
template <int IO>
__global__ void __launch_bounds__(256) dd2d_kernel(const void* dy, const void* u, float* dD, int64_t B, int64_t C,
                                                   int64_t img) {
    const int64_t c = blockIdx.x, img8 = img / 8;
    float acc = 0.f;
    for (int64_t b = 0; b < B; ++b) {
        const uint4* pd = (const uint4*)((const uint16_t*)dy + (b * C + c) * img);
        const uint4* pu = (const uint4*)((const uint16_t*)u + (b * C + c) * img);
        for (int64_t p = threadIdx.x; p < img8; p += 256) {
            const uint4 wd = pd[p], wu = pu[p];
            const uint32_t d4[4] = {wd.x, wd.y, wd.z, wd.w}, u4[4] = {wu.x, wu.y, wu.z, wu.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = fmaf(unpack_lo<IO>(d4[i]), unpack_lo<IO>(u4[i]), acc);
                acc = fmaf(unpack_hi<IO>(d4[i]), unpack_hi<IO>(u4[i]), acc);
            }
        }
    }
    __shared__ float red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) dD[c] = red[0];
}

static unsigned grid2d_for(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

hipError_t launch_adj2d(const void* kf, void* ka, int64_t C, hipStream_t st) {
    const int64_t words = C * P2D * P2D;
    if (words <= 0) return hipSuccess;
    hipLaunchKernelGGL(adj2d_kernel, dim3(grid2d_for(words)), dim3(256), 0, st, (const uint32_t*)kf, (uint32_t*)ka,
                       words);
    return hipGetLastError();
}

hipError_t launch_dk2d_sum(int dtype, const void* r, float* dk, int64_t B, int64_t C, int Hs, int Ws, hipStream_t st) {
    const int64_t total = C * Hs * Ws;
    if (total <= 0) return hipSuccess;
    if (dtype == CT_F16)
        hipLaunchKernelGGL((dk2d_sum_kernel<CT_F16>), dim3(grid2d_for(total)), dim3(256), 0, st, r, dk, B, C, Hs, Ws);
    else
        hipLaunchKernelGGL((dk2d_sum_kernel<CT_BF16>), dim3(grid2d_for(total)), dim3(256), 0, st, r, dk, B, C, Hs, Ws);
    return hipGetLastError();
}

hipError_t launch_dd2d(int dtype, const void* dy, const void* u, float* dD, int64_t B, int64_t C, int64_t img,
                       hipStream_t st) {
    if (C <= 0) return hipSuccess;
    if (dtype == CT_F16)
        hipLaunchKernelGGL((dd2d_kernel<CT_F16>), dim3((unsigned)C), dim3(256), 0, st, dy, u, dD, B, C, img);
    else
        hipLaunchKernelGGL((dd2d_kernel<CT_BF16>), dim3((unsigned)C), dim3(256), 0, st, dy, u, dD, B, C, img);
    return hipGetLastError();
}

hipError_t launch_conv2d(int dtype, const Conv2DArgs& a, hipStream_t st) {
    if (a.filter) {
        dim3 grid((unsigned)a.C, P2D / 32);
        if (dtype == CT_F16)
            hipLaunchKernelGGL((filter2d_kernel<CT_F16>), grid, dim3(256), 0, st, a.u, (void*)a.kf, a.inv_p2, a.Hs, a.Ws);
        else
            hipLaunchKernelGGL((filter2d_kernel<CT_BF16>), grid, dim3(256), 0, st, a.u, (void*)a.kf, a.inv_p2, a.Hs, a.Ws);
        return hipGetLastError();
    }
    const int64_t nitems = (a.B + 1) / 2 * a.C;
    if (nitems <= 0) return hipSuccess;
    const int64_t nwg = nitems < a.cus ? nitems : a.cus;
    if (a.spec) {
        if (a.B != 1) return hipErrorInvalidValue;  // single images only
        if (dtype == CT_F16) hipLaunchKernelGGL((conv2d_kernel<CT_F16, true>), dim3((unsigned)nwg), dim3(512), 0, st, a);
        else hipLaunchKernelGGL((conv2d_kernel<CT_BF16, true>), dim3((unsigned)nwg), dim3(512), 0, st, a);
        return hipGetLastError();
    }
    if (dtype == CT_F16) hipLaunchKernelGGL((conv2d_kernel<CT_F16, false>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    else hipLaunchKernelGGL((conv2d_kernel<CT_BF16, false>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcv
