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
// runs over 16 columns of the block (the tile layout of lconv_device.h).  The w_P twiddle runs
// on the vector ALU between the two stages, and one LDS exchange moves the contracted digit
// from n1 to n2 (forward) or from k2 to k1 (inverse).  Global rows go straight between memory
// and tile registers: a lane's tiles hold consecutive columns, so one access instruction moves
// whole 128-byte row segments of 4 rows.
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

// K (1, 2, 4 or 8) consecutive 16-bit elements <-> fp32, and K consecutive 32-bit words (one
// access each; the index is a multiple of K)
template <int CT, int K>
__device__ __forceinline__ void ldh(const void* p, int64_t i, float* x) {
    const uint16_t* q = (const uint16_t*)p + i;
    if constexpr (K == 1) {
        x[0] = unpack_lo<CT>(*q);
    } else if constexpr (K == 2) {
        const uint32_t w = *(const uint32_t*)q;
        x[0] = unpack_lo<CT>(w); x[1] = unpack_hi<CT>(w);
    } else if constexpr (K == 4) {
        const uint2 w = *(const uint2*)q;
        x[0] = unpack_lo<CT>(w.x); x[1] = unpack_hi<CT>(w.x); x[2] = unpack_lo<CT>(w.y); x[3] = unpack_hi<CT>(w.y);
    } else {
        const uint4 w = *(const uint4*)q;
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = unpack_lo<CT>(ww[i]); x[2 * i + 1] = unpack_hi<CT>(ww[i]); }
    }
}
template <int CT, int K>
__device__ __forceinline__ void sth(void* p, int64_t i, const float* x) {
    uint16_t* q = (uint16_t*)p + i;
    if constexpr (K == 1) {
        *q = (uint16_t)(pack2<CT>(x[0], 0.f) & 0xffffu);
    } else if constexpr (K == 2) {
        *(uint32_t*)q = pack2<CT>(x[0], x[1]);
    } else if constexpr (K == 4) {
        *(uint2*)q = make_uint2(pack2<CT>(x[0], x[1]), pack2<CT>(x[2], x[3]));
    } else {
        *(uint4*)q = make_uint4(pack2<CT>(x[0], x[1]), pack2<CT>(x[2], x[3]), pack2<CT>(x[4], x[5]), pack2<CT>(x[6], x[7]));
    }
}
// sth with the non-temporal hint, for the final output, where 16 lanes cover whole 128-byte
// lines (K >= 4).  With narrower slices two workgroups write the halves of one line, which the
// L2 merges for ordinary stores but not for streamed ones (measured: 36% more bytes written).
template <int CT, int K>
__device__ __forceinline__ void sth_nt(void* p, int64_t i, const float* x) {
    if constexpr (K < 4) {
        sth<CT, K>(p, i, x);
    } else {
        uint32_t* q = (uint32_t*)((uint16_t*)p + i);
#pragma unroll
        for (int j = 0; j < K / 2; ++j) __builtin_nontemporal_store(pack2<CT>(x[2 * j], x[2 * j + 1]), q + j);
    }
}
template <int K>
__device__ __forceinline__ void ldw(const uint32_t* p, int64_t i, uint32_t* w) {
    if constexpr (K == 1) {
        w[0] = p[i];
    } else if constexpr (K == 2) {
        const uint2 t = *(const uint2*)(p + i);
        w[0] = t.x; w[1] = t.y;
    } else {
#pragma unroll
        for (int h = 0; h < K / 4; ++h) {
            const uint4 t = *(const uint4*)(p + i + 4 * h);
            w[4 * h] = t.x; w[4 * h + 1] = t.y; w[4 * h + 2] = t.z; w[4 * h + 3] = t.w;
        }
    }
}
template <int K>
__device__ __forceinline__ void stw(uint32_t* p, int64_t i, const uint32_t* w) {
    if constexpr (K == 1) *(p + i) = w[0];
    else if constexpr (K == 2) *(uint2*)(p + i) = make_uint2(w[0], w[1]);
    else {
#pragma unroll
        for (int h = 0; h < K / 4; ++h) *(uint4*)(p + i + 4 * h) = make_uint4(w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]);
    }
}

// Column placement: tile g of the NCG tiles of a stage unit holds, in its L index x, global
// column NCG x + g of the block, so a lane's NCG tiles cover NCG consecutive columns and every
// global access moves NCG elements at once (whole 128-byte lines per row and instruction).  In
// LDS the same value sits at slot 16 g + x.

// PAIR (sequences of one real row, half rows kept): the workgroup transforms sequences s and
// s + 1 as one complex signal x_s + i x_{s+1} and splits the result in the second stage.
template <int CT, int P, bool PAIR>
__global__ void __launch_bounds__(512, 4) colmx_fwd_kernel(const ColArgs a) {
    using C = Cm<P>;
    constexpr int R = C::R, H = C::H, RB = C::RB, HB = C::HB, NCG = C::NCG;
    __shared__ uint32_t Y[C::CB * C::YC];
    const int lane = threadIdx.x & 63, g = lane >> 4, x = lane & 15;
    const int wave = PAIR ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
    const int64_t s = PAIR ? 2 * (int64_t)blockIdx.y : blockIdx.y, n_lo0 = block_col0<P>();
    const bool hasB = PAIR && s + 1 < a.nseq;
    const int64_t col0 = n_lo0 + NCG * x;  // this lane's first column
    int64_t row0, row1;
    seq_rows(a, a.seq0 + s, row0, row1);
    if constexpr (PAIR) {  // row1: the second sequence's row (each sequence is one real row)
        int64_t rb0, rb1;
        seq_rows(a, a.seq0 + (hasB ? s + 1 : s), rb0, rb1);
        row1 = hasB ? rb0 : -1;
    }
    const float2* twc = (const float2*)a.tw_col;
    // Scalar bases (this block's first column of each input row) and 32-bit lane offsets: the
    // loads take the scalar-base address form, with no 64-bit arithmetic per element.
    const uint16_t* const ub0 = (const uint16_t*)a.u + row0 + n_lo0;
    const uint16_t* const ub1 = (const uint16_t*)a.u + (row1 >= 0 ? row1 : row0) + n_lo0;
    const uint16_t* const qb0 = (const uint16_t*)a.q + row0 + n_lo0;
    const uint16_t* const qb1 = (const uint16_t*)a.q + (row1 >= 0 ? row1 : row0) + n_lo0;
    const uint32_t lane_off = NCG * x;
    // columns of this block below N, as a 32-bit bound on the lane offsets
    const uint32_t nlim = (uint32_t)(a.N - n_lo0 < 0 ? 0 : (a.N - n_lo0 > 0xffffffffLL ? 0xffffffffLL : a.N - n_lo0));

    // Stage 1, per n2 (two per wave), NCG tiles: radix R over n1 < H (gated pairs packed as
    // complex x_b + i x_{b+1}), times w_P^{n2 k1}, into the exchange.
    // The first-stage blocks stay in registers when they are few (P <= 512); at P = 1024
    // (eight blocks) they are read where they are used, from the cache.
    constexpr bool KEEP_F1 = RB * HB <= 4;
    MatImg<CT> f1[KEEP_F1 ? RB : 1][KEEP_F1 ? HB : 1];
    auto f1img = [&](int rb, int kc) LCV_INLINE { return load_img<CT>(a.img, C::G.f1 + rb * HB + kc, lane); };
    if constexpr (KEEP_F1) {
        static_for<0, RB>([&](auto rb) LCV_INLINE {
            static_for<0, HB>([&](auto kc) LCV_INLINE {
                f1[rb][kc] = f1img(decltype(rb)::value, decltype(kc)::value);
            });
        });
    }
    // All loads of the stage first (raw words: NCG 16-bit columns per access), then the
    // arithmetic, so one memory latency covers both n2 of the wave.
    // (P = 1024 has two K chunks per n2: its n2 go one at a time, which keeps it in 128 VGPRs)
    constexpr int RW = (NCG + 1) / 2;  // 32-bit words per access
    constexpr int NB = HB == 1 ? 2 : 1;  // n2 values whose loads are issued together
    uint32_t ru[NB][HB][4][RW], rq[NB][HB][4][RW], ru1[NB][HB][4][RW], rq1[NB][HB][4][RW];
    bool okv[NB][HB][4];
    auto ldraw = [&](const void* p, int64_t i, uint32_t* w) LCV_INLINE {
        const uint16_t* h = (const uint16_t*)p + i;
        if constexpr (NCG == 1) w[0] = *h;
        else if constexpr (NCG == 2) w[0] = *(const uint32_t*)h;
        else { const uint2 t = *(const uint2*)h; w[0] = t.x; w[1] = t.y; }
    };
    auto raw_f = [&](const uint32_t* w, int q) LCV_INLINE {
        return (q & 1) ? unpack_hi<CT>(w[q >> 1]) : unpack_lo<CT>(w[q >> 1]);
    };
    static_for<0, 2 / NB>([&](auto gg) LCV_INLINE {
        constexpr int gi = decltype(gg)::value;
        static_for<0, NB>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            const int n2 = wave + 8 * (NB * gi + i);
            static_for<0, HB>([&](auto kk) LCV_INLINE {
                constexpr int kc = decltype(kk)::value;
                static_for<0, 4>([&](auto jj) LCV_INLINE {
                    constexpr int j = decltype(jj)::value;
                    const int n1 = 16 * kc + 4 * g + j;
                    const uint32_t off = (uint32_t)kRow * (16 * n1 + n2) + lane_off;
                    // N is a multiple of 8: all NCG columns alike
                    const bool ok = n1 < H && off < nlim;
                    const int64_t e = ok ? off : lane_off;  // a valid element of the same rows
                    okv[i][kc][j] = ok;
                    ldraw(ub0, e, ru[i][kc][j]);
                    if (a.q) ldraw(qb0, e, rq[i][kc][j]);
                    if (row1 >= 0) {
                        ldraw(ub1, e, ru1[i][kc][j]);
                        if (a.q) ldraw(qb1, e, rq1[i][kc][j]);
                    }
                });
            });
        });
        static_for<0, NB>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            const int n2 = wave + 8 * (NB * gi + i);
            Operand<CT> op[NCG][HB];
            static_for<0, HB>([&](auto kk) LCV_INLINE {
                constexpr int kc = decltype(kk)::value;
                static_for<0, 4>([&](auto jj) LCV_INLINE {
                    constexpr int j = decltype(jj)::value;
                    static_for<0, NCG>([&](auto qq) LCV_INLINE {
                        constexpr int q = decltype(qq)::value;
                        float re = raw_f(ru[i][kc][j], q), im = 0.f;
                        if (a.q) re *= raw_f(rq[i][kc][j], q);
                        if (row1 >= 0) {
                            im = raw_f(ru1[i][kc][j], q);
                            if (a.q) im *= raw_f(rq1[i][kc][j], q);
                        }
                        op[q][kc].w[j] = okv[i][kc][j] ? pack2<CT>(re, im) : 0u;
                    });
                });
            });
            // w_P^{n2 k1} for k1 = 16 rb + 4 g + j: a table value per rb times powers of w_P^{n2}
            const float2 wstep = twc[n2];
            static_for<0, RB>([&](auto r) LCV_INLINE {
                constexpr int rb = decltype(r)::value;
                float2 tw[4];
                tw[0] = twc[n2 * (16 * rb + 4 * g)];  // < P
#pragma unroll
                for (int j = 1; j < 4; ++j) tw[j] = cmulf(tw[j - 1], wstep);
                static_for<0, NCG>([&](auto qq) LCV_INLINE {
                    constexpr int q = decltype(qq)::value;
                    const int cs = 16 * q + x;
                    f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                    static_for<0, HB>([&](auto kk) LCV_INLINE {
                        constexpr int kc = decltype(kk)::value;
                        if constexpr (KEEP_F1) stage_keep_acc<CT>(f1[rb][kc], op[q][kc], re, im);
                        else stage_keep_acc<CT>(f1img(rb, kc), op[q][kc], re, im);
                    });
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k1 = 16 * rb + 4 * g + j;
                        float xr = re[j], xi = im[j];
                        cmul(xr, xi, tw[j].x, tw[j].y);
                        Y[yaddr<P>(cs, k1, n2)] = pack2<CT>(xr, xi);
                    }
                });
            });
        });
    });
    __syncthreads();

    const MatImg<CT> f16 = load_img<CT>(a.img, C::G.f16, lane);
    const int64_t mask = a.M - 1;
    uint32_t* const wsb = (uint32_t*)a.ws + s * a.rows * kRow + n_lo0;  // this block's row 0
    if constexpr (PAIR) {
        // Stage 2 for z = x_A + i x_B.  Rows k of the two real transforms follow from rows k and
        // P - k of Z (Hermitian split): X_A[k] = (Z[k] + conj Z[P-k]) / 2 and
        // X_B[k] = (Z[k] - conj Z[P-k]) / 2i; only rows k <= P/2 are kept.  A slot takes digits
        // k1a and k1b = R - k1a: the 16-point DFT of k1a (tile rows k2 = 4 g + j) and the
        // row-reversed one of k1b (rows 15 - k2) leave Z[k] and Z[P - k] in one lane.  Lanes
        // g < 2 keep the rows of k1a, lanes g >= 2 those of k1b.  The self-paired digits: k1 = 0
        // takes its partner from the conjugate DFT (rows (16 - k2) mod 16; written as k1b = R),
        // k1 = R/2 from the reversed one; each keeps its rows k <= P/2 only.
        const MatImg<CT> f16r = load_img<CT>(a.img, C::G.f16r, lane);
        uint32_t* const wsbB = wsb + a.rows * kRow;  // B's row 0 (used only with hasB)
        const bool lo = g < 2;
        const float sg = lo ? 1.f : -1.f;
        // w_M^{n_lo k} of a kept row k = e - / + R j: per column, the step in j
        float2 wjs[NCG];
        static_for<0, NCG>([&](auto qq) LCV_INLINE {
            constexpr int q = decltype(qq)::value;
            const float2 w = tw_m(a.tw_lo, a.tw_hi, ((col0 + q) * R) & mask);
            wjs[q] = lo ? w : make_float2(w.x, -w.y);
        });
        auto slot = [&](int k1a, int k1b, const MatImg<CT>& mb, int nkeep) LCV_INLINE {
            // this lane's kept rows: e + R j (g < 2) or e - R j (g >= 2)
            const int e = lo ? k1a + 4 * g * R : k1b + R * (15 - 4 * g);
            uint32_t oa[4][NCG], ob[4][NCG];
            static_for<0, NCG>([&](auto qq) LCV_INLINE {
                constexpr int q = decltype(qq)::value;
                const int cs = 16 * q + x;
                Operand<CT> opa, opb;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    opa.w[j] = Y[yaddr<P>(cs, k1a, 4 * g + j)];
                    opb.w[j] = Y[yaddr<P>(cs, k1b & (R - 1), 4 * g + j)];
                }
                const Tile ta = stage_keep<CT>(f16, opa), tb = stage_keep<CT>(mb, opb);
                // the 1/2 of the split rides on the twiddle
                float2 w = tw_m(a.tw_lo, a.tw_hi, ((col0 + q) * e) & mask);
                w.x *= 0.5f;
                w.y *= 0.5f;
                // with own row a = ta, partner b = tb: X_A = a + conj b, X_B = -i (a - conj b);
                // swapping a and b (lanes g >= 2) conjugates both
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float ar = ta.re[j] + tb.re[j], ai = sg * (ta.im[j] - tb.im[j]);
                    float br = ta.im[j] + tb.im[j], bi = sg * (tb.re[j] - ta.re[j]);
                    cmul(ar, ai, w.x, w.y);
                    cmul(br, bi, w.x, w.y);
                    oa[j][q] = pack2<CT>(ar, ai);
                    ob[j][q] = pack2<CT>(br, bi);
                    w = cmulf(w, wjs[q]);
                }
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (lo || 4 * g + j < nkeep) {
                    const uint32_t kh = lo ? e + R * j : e - R * j;
                    stw<NCG>(wsb, (int64_t)(kh * (uint32_t)kRow + lane_off), oa[j]);
                    if (hasB) stw<NCG>(wsbB, (int64_t)(kh * (uint32_t)kRow + lane_off), ob[j]);
                }
            }
        };
        // digit pairs of this wave: k1a = w + 16 i (w = 1, 2, 3), 16 - w + 16 i (w = 5, 6, 7),
        // 4 + 8 i (w = 4), 8 + 8 i (w = 0, which also takes the self-paired 0 and R/2)
        const int kb0 = wave == 0 ? 8 : wave == 4 ? 4 : wave < 4 ? wave : 16 - wave;
        const int ks = (wave & 3) == 0 ? 8 : 16, cnt = wave == 0 ? R / 16 - 1 : R / 16;
        for (int i = 0; i < cnt; ++i) slot(kb0 + ks * i, R - kb0 - ks * i, f16r, 16);
        if (wave == 0) {
            const MatImg<CT> i16 = load_img<CT>(a.img, C::G.i16, lane);  // rows (16 - k2) mod 16
            slot(0, R, i16, 9);
            slot(R / 2, R / 2, f16r, 8);
        }
    } else {
        // Stage 2, per k1 (R/8 per wave), NCG tiles: 16-point DFT over n2, the four-step twiddle
        // w_M^{n_lo k_hi}, store rows k_hi = k1 + R k2 of the workspace.
        // w_M^{n_lo k_hi} for k_hi = k1 + R (4 g + j), k1 = wave + 8 i: per column, a base for
        // i = 0, a step for i, and a step for j (products of fp32 table values; at most 11 steps)
        float2 wb[NCG], wi[NCG], wj[NCG];
        static_for<0, NCG>([&](auto qq) LCV_INLINE {
            constexpr int q = decltype(qq)::value;
            const int64_t n_lo = col0 + q;
            wb[q] = tw_m(a.tw_lo, a.tw_hi, (n_lo * (wave + 4 * g * R)) & mask);
            wi[q] = tw_m(a.tw_lo, a.tw_hi, (n_lo * 8) & mask);
            wj[q] = tw_m(a.tw_lo, a.tw_hi, (n_lo * R) & mask);
        });
        static_for<0, R / 8>([&](auto ii) LCV_INLINE {
            const int k1 = wave + 8 * decltype(ii)::value;
            uint32_t out[4][NCG];
            static_for<0, NCG>([&](auto qq) LCV_INLINE {
                constexpr int q = decltype(qq)::value;
                const int cs = 16 * q + x;
                Operand<CT> op;
#pragma unroll
                for (int j = 0; j < 4; ++j) op.w[j] = Y[yaddr<P>(cs, k1, 4 * g + j)];
                Tile t = stage_keep<CT>(f16, op);  // rows k2 = 4 g + j
                float2 w = wb[q];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float xr = t.re[j], xi = t.im[j];
                    cmul(xr, xi, w.x, w.y);
                    w = cmulf(w, wj[q]);
                    out[j][q] = pack2<CT>(xr, xi);
                }
                wb[q] = cmulf(wb[q], wi[q]);
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kh = k1 + R * (4 * g + j);
                if (kh < a.rows) stw<NCG>(wsb, (int64_t)((uint32_t)kh * (uint32_t)kRow + lane_off), out[j]);
            }
        });
    }
}

// PAIR (half rows, one real row per sequence): a block takes two sequences A, B and runs one
// complex inverse on V_A + i V_B; the real part of the result is A's output and the imaginary
// part B's (both are real), so the transform and its twiddles are shared by the two.
template <int CT, int P, bool PAIR>
__global__ void __launch_bounds__(512, 4) colmx_inv_kernel(const ColArgs a) {
    using C = Cm<P>;
    constexpr int R = C::R, H = C::H, RB = C::RB, HB = C::HB, NCG = C::NCG;
    __shared__ uint32_t Z[C::CB * C::ZC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, x = lane & 15;
    const int64_t s = PAIR ? 2 * (int64_t)blockIdx.y : (int64_t)blockIdx.y, n_lo0 = block_col0<P>();
    const bool hasB = PAIR && s + 1 < a.nseq;  // an odd count's last block has A only
    const int64_t col0 = n_lo0 + NCG * x;
    int64_t row0, row1;
    seq_rows(a, a.seq0 + s, row0, row1);
    if constexpr (PAIR) {  // row1: B's row (each sequence is one real row)
        int64_t rb0, rb1;
        seq_rows(a, a.seq0 + (hasB ? s + 1 : s), rb0, rb1);
        row1 = hasB ? rb0 : -1;
    }
    const float2* twc = (const float2*)a.tw_col;
    const int64_t mask = a.M - 1;
    // scalar bases and 32-bit lane offsets (as in the forward pass)
    const uint32_t* const wsb = (const uint32_t*)a.ws + s * a.rows * kRow + n_lo0;
    const uint32_t* const wsbB = hasB ? wsb + a.rows * kRow : wsb;  // PAIR: B's rows (A's if none)
    const int64_t r1 = row1 >= 0 ? row1 : row0;
    uint16_t* const yb0 = (uint16_t*)a.y + row0 + n_lo0;
    uint16_t* const yb1 = (uint16_t*)a.y + r1 + n_lo0;
    const uint16_t* const vb0 = (const uint16_t*)a.v + row0 + n_lo0;
    const uint16_t* const vb1 = (const uint16_t*)a.v + r1 + n_lo0;
    const uint32_t lane_off = NCG * x;
    const uint32_t nlim = (uint32_t)(a.N - n_lo0 < 0 ? 0 : (a.N - n_lo0 > 0xffffffffLL ? 0xffffffffLL : a.N - n_lo0));

    // Stage 1, per k1 (R/8 per wave), NCG tiles: rows k_hi = k1 + R k2 of the workspace, times
    // conj(w_M^{n_lo k_hi}), 16-point inverse DFT over k2, times conj(w_P^{n2 k1}), into the
    // exchange.
    const MatImg<CT> i16 = load_img<CT>(a.img, C::G.i16, lane);
    // conj(w_M^{n_lo k_hi}) factors as in the forward pass: base, step for i, step for j
    float2 wb[NCG], wi[NCG], wj[NCG];
    static_for<0, NCG>([&](auto qq) LCV_INLINE {
        constexpr int q = decltype(qq)::value;
        const int64_t n_lo = col0 + q;
        wb[q] = tw_m(a.tw_lo, a.tw_hi, (n_lo * (wave + 4 * g * R)) & mask);
        wi[q] = tw_m(a.tw_lo, a.tw_hi, (n_lo * 8) & mask);
        wj[q] = tw_m(a.tw_lo, a.tw_hi, (n_lo * R) & mask);
    });
    // Rows k_hi >= a.rows are not stored (one real row per sequence): the column spectrum V of a
    // real column is conjugate-symmetric, V[P - k] = conj V[k], and with V = conj(w_M^{n_lo k})
    // times the stored value, row k reads as w_8192^{n_lo} conj(stored row P - k).
    const bool half = a.rows < P;
    float2 wrow[NCG];  // w_8192^{n_lo}
    static_for<0, NCG>([&](auto qq) LCV_INLINE {
        constexpr int q = decltype(qq)::value;
        wrow[q] = half ? tw_m(a.tw_lo, a.tw_hi, ((col0 + q) * P) & mask) : make_float2(1.f, 0.f);
    });
    // one k1: the twiddled, packed operand of column tile q from the raw rows zw (PAIR: and zwB)
    auto stage1 = [&](int k1, const uint32_t (*zw)[NCG], const uint32_t (*zwB)[NCG]) LCV_INLINE {
        // conj(w_P^{n2 k1}) for n2 = 4 g + j
        const float2 p1 = twc[k1];
        float2 tp[4];
        tp[0] = twc[4 * g * k1];  // < P
#pragma unroll
        for (int j = 1; j < 4; ++j) tp[j] = cmulf(tp[j - 1], p1);
        static_for<0, NCG>([&](auto qq) LCV_INLINE {
            constexpr int q = decltype(qq)::value;
            const int cs = 16 * q + x;
            float2 w = wb[q];
            Operand<CT> op;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float zr = unpack_lo<CT>(zw[j][q]), zi = unpack_hi<CT>(zw[j][q]);
                const bool mirrored = k1 + R * (4 * g + j) >= a.rows;
                if constexpr (PAIR) {
                    // Z = V_A + i V_B; a mirrored row is w_8192^{n_lo} conj(stored A + i conj stored B)
                    const float br = hasB ? unpack_lo<CT>(zwB[j][q]) : 0.f;
                    const float bi = hasB ? unpack_hi<CT>(zwB[j][q]) : 0.f;
                    if (mirrored) {
                        const float mr = zr + bi, mi = br - zi;
                        zr = mr * wrow[q].x - mi * wrow[q].y;
                        zi = mr * wrow[q].y + mi * wrow[q].x;
                    } else {
                        const float mr = zr - bi, mi = zi + br;
                        zr = mr;
                        zi = mi;
                    }
                } else if (mirrored) {  // mirrored row: w_8192^{n_lo} conj(z)
                    const float mr = zr, mi = -zi;
                    zr = mr * wrow[q].x - mi * wrow[q].y;
                    zi = mr * wrow[q].y + mi * wrow[q].x;
                }
                cmulc(zr, zi, w.x, w.y);
                w = cmulf(w, wj[q]);
                op.w[j] = pack2<CT>(zr, zi);
            }
            wb[q] = cmulf(wb[q], wi[q]);
            Tile t = stage_keep<CT>(i16, op);  // rows n2 = 4 g + j
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n2 = 4 * g + j;
                float zr = t.re[j], zi = t.im[j];
                cmulc(zr, zi, tp[j].x, tp[j].y);
                Z[zaddr<P>(cs, n2, k1)] = pack2<CT>(zr, zi);
            }
        });
    };
    auto ldrows = [&](const uint32_t* base, int k1, uint32_t (*dst)[NCG]) LCV_INLINE {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kh = k1 + R * (4 * g + j), kr = kh < a.rows ? kh : P - kh;
            ldw<NCG>(base, (int64_t)((uint32_t)kr * (uint32_t)kRow + lane_off), dst[j]);
        }
    };
    if constexpr (!PAIR) {
        // all rows' loads first, then the arithmetic
        uint32_t in[R / 8][4][NCG];
        static_for<0, R / 8>([&](auto ii) LCV_INLINE {
            ldrows(wsb, wave + 8 * decltype(ii)::value, in[decltype(ii)::value]);
        });
        static_for<0, R / 8>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            stage1(wave + 8 * i, in[i], in[i]);
        });
    } else {
        // two sequences: the rows of k1 + 8 load while k1 is computed (double buffer)
        uint32_t inA[2][4][NCG], inB[2][4][NCG];
        ldrows(wsb, wave, inA[0]);
        ldrows(wsbB, wave, inB[0]);
        static_for<0, R / 8>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            if constexpr (i + 1 < R / 8) {
                ldrows(wsb, wave + 8 * (i + 1), inA[(i + 1) & 1]);
                ldrows(wsbB, wave + 8 * (i + 1), inB[(i + 1) & 1]);
            }
            stage1(wave + 8 * i, inA[i & 1], inB[i & 1]);
        });
    }
    __syncthreads();

    // Stage 2, per n2 (two per wave), NCG tiles: inverse radix R over k1 for the kept rows
    // n1 < H, post-gate, store rows n_hi = 16 n1 + n2 (and n < N) of the output pair.
    MatImg<CT> i2[HB][RB];
    static_for<0, HB>([&](auto rb) LCV_INLINE {
        static_for<0, RB>([&](auto kc) LCV_INLINE {
            i2[rb][kc] = load_img<CT>(a.img, C::G.i2 + decltype(rb)::value * RB + decltype(kc)::value, lane);
        });
    });
    static_for<0, 2>([&](auto ii) LCV_INLINE {
        const int n2 = wave + 8 * decltype(ii)::value;
        static_for<0, HB>([&](auto r) LCV_INLINE {
            constexpr int rb = decltype(r)::value;
            Tile acc[NCG];
            static_for<0, NCG>([&](auto qq) LCV_INLINE {
                constexpr int q = decltype(qq)::value;
                const int cs = 16 * q + x;
                f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                static_for<0, RB>([&](auto kk) LCV_INLINE {
                    constexpr int kc = decltype(kk)::value;
                    Operand<CT> op;
#pragma unroll
                    for (int j = 0; j < 4; ++j) op.w[j] = Z[zaddr<P>(cs, n2, 16 * kc + 4 * g + j)];
                    stage_keep_acc<CT>(i2[rb][kc], op, re, im);
                });
                acc[q] = Tile{re, im};
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n1 = 16 * rb + 4 * g + j;
                const uint32_t off = (uint32_t)kRow * (16 * n1 + n2) + lane_off;
                const bool ok = n1 < H && off < nlim;
                const int64_t e = ok ? off : lane_off;
                float yr[NCG], yi[NCG], t[NCG];
                static_for<0, NCG>([&](auto qq) LCV_INLINE {
                    constexpr int q = decltype(qq)::value;
                    yr[q] = acc[q].re[j];
                    yi[q] = acc[q].im[j];
                });
                if (a.v) {
                    ldh<CT, NCG>(vb0, e, t);
#pragma unroll
                    for (int q = 0; q < NCG; ++q) yr[q] *= t[q];
                    if (row1 >= 0) {
                        ldh<CT, NCG>(vb1, e, t);
#pragma unroll
                        for (int q = 0; q < NCG; ++q) yi[q] *= t[q];
                    }
                }
                if (ok) {
                    sth_nt<CT, NCG>(yb0, e, yr);
                    if (row1 >= 0) sth_nt<CT, NCG>(yb1, e, yi);
                }
            }
        });
    });
}

// ---- short columns, P = 16 R with R = 1, 2, 4, 8 (M1 = 16 .. 128): registers only -------------
//
// The same factorization with a first digit of at most 8 values: its DFT (radix R over n1,
// R/2 nonzero inputs forward, R/2 kept outputs inverse) runs on the vector ALU with constant
// coefficients, and the 16-point DFT over n2 on the matrix cores.  A lane's operand already
// holds the four n2 = 4 g + j of its columns, so no data crosses lanes and nothing goes
// through LDS: every wave works alone on 16 NCG columns of one sequence, NCG consecutive
// columns per lane (2 to 16 bytes per row and access).

// exp(-2 pi i e / R) for R <= 8 (constants after unrolling)
__device__ __forceinline__ float2 w_small(int e, int R) {
    constexpr float c = 0.70710678118654752f;
    const float2 t[8] = {{1.f, 0.f}, {c, -c}, {0.f, -1.f}, {-c, -c}, {-1.f, 0.f}, {-c, c}, {0.f, 1.f}, {c, c}};
    return t[((e % R + R) % R) * (8 / R)];
}

template <int P>
struct Cr {
    static constexpr ColMxGrid G = colmx_grid(P);
    static constexpr int R = P / 16, H = R > 1 ? R / 2 : 1;  // n1 values in, n1 values kept
    static constexpr int NCG = 4 / H;                         // columns per lane: 4, 4, 2, 1
    static constexpr int COLS = 16 * NCG;                     // columns per wave
};

template <int CT, int P>
__global__ void __launch_bounds__(256, 4) colreg_fwd_kernel(const ColArgs a) {
    using C = Cr<P>;
    constexpr int R = C::R, H = C::H, NCG = C::NCG, RW = (NCG + 1) / 2;
    const int lane = threadIdx.x & 63, g = lane >> 4, x = lane & 15;
    // wave of the sequence (readfirstlane: the compiler keeps what depends on it in scalars)
    const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t s = blockIdx.y;
    const int64_t cw0 = wid * C::COLS;          // the wave's first column
    const int64_t col0 = cw0 + NCG * x;
    int64_t row0, row1;
    seq_rows(a, a.seq0 + s, row0, row1);
    const float2* twc = (const float2*)a.tw_col;
    const int64_t mask = a.M - 1;
    // scalar bases and 32-bit lane offsets: no 64-bit arithmetic per element
    const uint16_t* const ub0 = (const uint16_t*)a.u + row0 + cw0;
    const uint16_t* const ub1 = (const uint16_t*)a.u + (row1 >= 0 ? row1 : row0) + cw0;
    const uint16_t* const qb0 = (const uint16_t*)a.q + row0 + cw0;
    const uint16_t* const qb1 = (const uint16_t*)a.q + (row1 >= 0 ? row1 : row0) + cw0;
    const uint32_t lane_off = NCG * x;
    const uint32_t nlim = (uint32_t)(a.N - cw0 < 0 ? 0 : (a.N - cw0 > 0xffffffffLL ? 0xffffffffLL : a.N - cw0));

    // gated input pairs x[16 n1 + 4 g + j] of this lane's columns, packed in the compute type
    // (R = 1: only rows 4 g + j < 8 are nonzero)
    uint32_t xin[H][4][NCG];
    {
        uint32_t ru[H][4][RW], rq[H][4][RW], ru1[H][4][RW], rq1[H][4][RW];
        bool okv[H][4];
        auto ldraw = [&](const void* p, int64_t i, uint32_t* w) LCV_INLINE {
            const uint16_t* h = (const uint16_t*)p + i;
            if constexpr (NCG == 2) w[0] = *(const uint32_t*)h;
            else if constexpr (NCG == 4) { const uint2 t = *(const uint2*)h; w[0] = t.x; w[1] = t.y; }
            else { const uint4 t = *(const uint4*)h; w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w; }
        };
        static_for<0, H>([&](auto nn) LCV_INLINE {
            constexpr int n1 = decltype(nn)::value;
            static_for<0, 4>([&](auto jj) LCV_INLINE {
                constexpr int j = decltype(jj)::value;
                const int nh = 16 * n1 + 4 * g + j;
                const uint32_t off = (uint32_t)kRow * nh + lane_off;
                const bool ok = (R > 1 || nh < 8) && off < nlim;
                const int64_t e = ok ? off : lane_off;
                okv[n1][j] = ok;
                ldraw(ub0, e, ru[n1][j]);
                if (a.q) ldraw(qb0, e, rq[n1][j]);
                if (row1 >= 0) {
                    ldraw(ub1, e, ru1[n1][j]);
                    if (a.q) ldraw(qb1, e, rq1[n1][j]);
                }
            });
        });
        auto raw_f = [&](const uint32_t* w, int q) LCV_INLINE {
            return (q & 1) ? unpack_hi<CT>(w[q >> 1]) : unpack_lo<CT>(w[q >> 1]);
        };
        static_for<0, H>([&](auto nn) LCV_INLINE {
            constexpr int n1 = decltype(nn)::value;
            static_for<0, 4>([&](auto jj) LCV_INLINE {
                constexpr int j = decltype(jj)::value;
                static_for<0, NCG>([&](auto qq) LCV_INLINE {
                    constexpr int q = decltype(qq)::value;
                    float re = raw_f(ru[n1][j], q), im = 0.f;
                    if (a.q) re *= raw_f(rq[n1][j], q);
                    if (row1 >= 0) {
                        im = raw_f(ru1[n1][j], q);
                        if (a.q) im *= raw_f(rq1[n1][j], q);
                    }
                    xin[n1][j][q] = okv[n1][j] ? pack2<CT>(re, im) : 0u;
                });
            });
        });
    }

    const MatImg<CT> f16 = load_img<CT>(a.img, C::G.f16, lane);
    uint32_t* const wsb = (uint32_t*)a.ws + s * a.rows * kRow + cw0;  // the wave's columns, row 0
    // four-step twiddle w_M^{n_lo k_hi}, n_lo = col0 + q, k_hi = k1 + R (4 g + j):
    // w_M^{col0 k_hi} w_M^{q k_hi}, stepped along j by w_M^{col0 R} and w_M^{R}
    // Per-k1 factors advance from k1 to k1 + 1 by one product each (at most 7 steps), so the
    // tables are read once:  w_P^{4 g k1}, w_P^{k1}, w_M^{col0 (k1 + 4 g R)}, w_M^{k1 + 4 g R}.
    const float2 wcR = tw_m(a.tw_lo, a.tw_hi, (col0 * R) & mask);
    const float2 w1R = ((const float2*)a.tw_lo)[R];
    const float2 tb1 = twc[4 * g], ts1 = twc[1 % P];
    const float2 wb1 = tw_m(a.tw_lo, a.tw_hi, col0 & mask), sb1 = ((const float2*)a.tw_lo)[1];
    float2 tbk = make_float2(1.f, 0.f), tsk = make_float2(1.f, 0.f);
    float2 wbk = tw_m(a.tw_lo, a.tw_hi, (col0 * 4 * g * R) & mask);
    float2 sbk = ((const float2*)a.tw_lo)[4 * g * R];
    static_for<0, R>([&](auto kk) LCV_INLINE {
        constexpr int k1 = decltype(kk)::value;
        // first digit: y[j][q] = w_P^{n2 k1} sum_{n1 < H} w_R^{n1 k1} x[n1][j][q], n2 = 4 g + j
        Operand<CT> op[NCG];
        const float2 ts = tsk;
        float2 tw = tbk;
        static_for<0, 4>([&](auto jj) LCV_INLINE {
            constexpr int j = decltype(jj)::value;
            static_for<0, NCG>([&](auto qq) LCV_INLINE {
                constexpr int q = decltype(qq)::value;
                float yr = 0.f, yi = 0.f;
                static_for<0, H>([&](auto nn) LCV_INLINE {
                    constexpr int n1 = decltype(nn)::value;
                    const float xr = unpack_lo<CT>(xin[n1][j][q]), xi = unpack_hi<CT>(xin[n1][j][q]);
                    if constexpr (R == 1 || (n1 * k1) % R == 0) {
                        yr += xr; yi += xi;
                    } else {
                        const float2 w = w_small(n1 * k1, R);
                        yr += xr * w.x - xi * w.y;
                        yi += xr * w.y + xi * w.x;
                    }
                });
                if constexpr (k1 > 0) cmul(yr, yi, tw.x, tw.y);
                op[q].w[j] = pack2<CT>(yr, yi);
            });
            tw = cmulf(tw, ts);
        });
        // 16-point DFT over n2, rows k2 = 4 g + j; twiddle; store rows k_hi
        const float2 wb = wbk, sb = sbk;
        tbk = cmulf(tbk, tb1);
        tsk = cmulf(tsk, ts1);
        wbk = cmulf(wbk, wb1);
        sbk = cmulf(sbk, sb1);
        uint32_t out[4][NCG];
        static_for<0, NCG>([&](auto qq) LCV_INLINE {
            constexpr int q = decltype(qq)::value;
            Tile t = stage_keep<CT>(f16, op[q]);
            float2 w = wb, sj = sb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // w_M^{(col0 + q) k_hi} = w_M^{col0 k_hi} (w_M^{k_hi})^q
                float2 wq = w;
#pragma unroll
                for (int r = 0; r < q; ++r) wq = cmulf(wq, sj);
                float xr = t.re[j], xi = t.im[j];
                cmul(xr, xi, wq.x, wq.y);
                out[j][q] = pack2<CT>(xr, xi);
                w = cmulf(w, wcR);
                sj = cmulf(sj, w1R);
            }
        });
#pragma unroll
        for (int j = 0; j < 4; ++j)
            stw<NCG>(wsb, (int64_t)((uint32_t)(k1 + R * (4 * g + j)) * (uint32_t)kRow + lane_off), out[j]);
    });
}

template <int CT, int P>
__global__ void __launch_bounds__(256, 4) colreg_inv_kernel(const ColArgs a) {
    using C = Cr<P>;
    constexpr int R = C::R, H = C::H, NCG = C::NCG;
    const int lane = threadIdx.x & 63, g = lane >> 4, x = lane & 15;
    const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t s = blockIdx.y;
    const int64_t cw0 = wid * C::COLS;          // the wave's first column
    const int64_t col0 = cw0 + NCG * x;
    int64_t row0, row1;
    seq_rows(a, a.seq0 + s, row0, row1);
    const float2* twc = (const float2*)a.tw_col;
    const int64_t mask = a.M - 1;
    // scalar bases and 32-bit lane offsets (as in the forward pass)
    const uint32_t* const wsb = (const uint32_t*)a.ws + s * a.rows * kRow + cw0;
    const int64_t r1 = row1 >= 0 ? row1 : row0;
    uint16_t* const yb0 = (uint16_t*)a.y + row0 + cw0;
    uint16_t* const yb1 = (uint16_t*)a.y + r1 + cw0;
    const uint16_t* const vb0 = (const uint16_t*)a.v + row0 + cw0;
    const uint16_t* const vb1 = (const uint16_t*)a.v + r1 + cw0;
    const uint32_t lane_off = NCG * x;
    const uint32_t nlim = (uint32_t)(a.N - cw0 < 0 ? 0 : (a.N - cw0 > 0xffffffffLL ? 0xffffffffLL : a.N - cw0));
    const MatImg<CT> i16 = load_img<CT>(a.img, C::G.i16, lane);

    // y[n1][j][q] for rows n_hi = 16 n1 + 4 g + j < P / 2
    float yr[H][4][NCG], yi[H][4][NCG];
    const float2 wcR = tw_m(a.tw_lo, a.tw_hi, (col0 * R) & mask);
    const float2 w1R = ((const float2*)a.tw_lo)[R];
    // per-k1 factors stepped from k1 to k1 + 1, as in the forward pass
    const float2 tb1 = twc[4 * g], ts1 = twc[1 % P];
    const float2 wb1 = tw_m(a.tw_lo, a.tw_hi, col0 & mask), sb1 = ((const float2*)a.tw_lo)[1];
    float2 tbk = make_float2(1.f, 0.f), tsk = make_float2(1.f, 0.f);
    float2 wbk = tw_m(a.tw_lo, a.tw_hi, (col0 * 4 * g * R) & mask);
    float2 sbk = ((const float2*)a.tw_lo)[4 * g * R];
    uint32_t in[2][4][NCG];  // workspace rows of k1 and k1 + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) ldw<NCG>(wsb, (int64_t)((uint32_t)(R * (4 * g + j)) * (uint32_t)kRow + lane_off), in[0][j]);
    static_for<0, R>([&](auto kk) LCV_INLINE {
        constexpr int k1 = decltype(kk)::value, b = k1 & 1;
        if constexpr (k1 + 1 < R) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ldw<NCG>(wsb, (int64_t)((uint32_t)(k1 + 1 + R * (4 * g + j)) * (uint32_t)kRow + lane_off), in[1 - b][j]);
        }
        // conj(w_M^{n_lo k_hi}), stepped as in the forward pass
        const float2 wb = wbk, sb = sbk, tb = tbk, ts = tsk;
        tbk = cmulf(tbk, tb1);
        tsk = cmulf(tsk, ts1);
        wbk = cmulf(wbk, wb1);
        sbk = cmulf(sbk, sb1);
        Operand<CT> op[NCG];
        {
            float2 w = wb, sj = sb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float2 wq = w;
                static_for<0, NCG>([&](auto qq) LCV_INLINE {
                    constexpr int q = decltype(qq)::value;
                    float zr = unpack_lo<CT>(in[b][j][q]), zi = unpack_hi<CT>(in[b][j][q]);
                    cmulc(zr, zi, wq.x, wq.y);
                    op[q].w[j] = pack2<CT>(zr, zi);
                    wq = cmulf(wq, sj);
                });
                w = cmulf(w, wcR);
                sj = cmulf(sj, w1R);
            }
        }
        // 16-point inverse DFT over k2 (rows n2 = 4 g + j), conj(w_P^{n2 k1}), then the first
        // digit: y[n1] += w_R^{-n1 k1} z for the kept n1 < H
        static_for<0, NCG>([&](auto qq) LCV_INLINE {
            constexpr int q = decltype(qq)::value;
            Tile t = stage_keep<CT>(i16, op[q]);
            float2 tw = tb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float zr = t.re[j], zi = t.im[j];
                if constexpr (k1 > 0) cmulc(zr, zi, tw.x, tw.y);
                tw = cmulf(tw, ts);
                static_for<0, H>([&](auto nn) LCV_INLINE {
                    constexpr int n1 = decltype(nn)::value;
                    float ar = zr, ai = zi;
                    if constexpr (R > 1 && (n1 * k1) % R != 0) {
                        const float2 w = w_small(-n1 * k1, R);
                        ar = zr * w.x - zi * w.y;
                        ai = zr * w.y + zi * w.x;
                    }
                    if constexpr (k1 == 0) {
                        yr[n1][j][q] = ar;
                        yi[n1][j][q] = ai;
                    } else {
                        yr[n1][j][q] += ar;
                        yi[n1][j][q] += ai;
                    }
                });
            }
        });
    });
    // gate and store rows n_hi = 16 n1 + 4 g + j (R = 1: only 4 g + j < 8)
    static_for<0, H>([&](auto nn) LCV_INLINE {
        constexpr int n1 = decltype(nn)::value;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nh = 16 * n1 + 4 * g + j;
            const uint32_t off = (uint32_t)kRow * nh + lane_off;
            const bool ok = (R > 1 || nh < 8) && off < nlim;
            const int64_t e = ok ? off : lane_off;
            float vr[NCG], vi[NCG], t[NCG];
#pragma unroll
            for (int q = 0; q < NCG; ++q) { vr[q] = yr[n1][j][q]; vi[q] = yi[n1][j][q]; }
            if (a.v) {
                ldh<CT, NCG>(vb0, e, t);
#pragma unroll
                for (int q = 0; q < NCG; ++q) vr[q] *= t[q];
                if (row1 >= 0) {
                    ldh<CT, NCG>(vb1, e, t);
#pragma unroll
                    for (int q = 0; q < NCG; ++q) vi[q] *= t[q];
                }
            }
            if (ok) {
                sth_nt<CT, NCG>(yb0, e, vr);
                if (row1 >= 0) sth_nt<CT, NCG>(yb1, e, vi);
            }
        }
    });
}

template <int CT, int P>
hipError_t launch_r(bool fwd, const ColArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)(kRow / (4 * Cr<P>::COLS)), (unsigned)a.nseq);
    if (fwd) hipLaunchKernelGGL((colreg_fwd_kernel<CT, P>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((colreg_inv_kernel<CT, P>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int CT, int P>
hipError_t launch_t(bool fwd, const ColArgs& a, hipStream_t st) {
    static_assert(kRow / Cm<P>::CB % (8 * Cm<P>::S) == 0, "the XCD order needs whole groups");
    const dim3 grid((unsigned)(kRow / Cm<P>::CB), (unsigned)a.nseq);
    const dim3 gp((unsigned)(kRow / Cm<P>::CB), (unsigned)((a.nseq + 1) / 2));  // sequence pairs
    if (fwd && a.rows < P) hipLaunchKernelGGL((colmx_fwd_kernel<CT, P, true>), gp, dim3(512), 0, st, a);
    else if (fwd) hipLaunchKernelGGL((colmx_fwd_kernel<CT, P, false>), grid, dim3(512), 0, st, a);
    else if (P >= 512 && a.rows < P) {  // half rows: sequences in pairs (P = 256's wider tiles would spill)
        hipLaunchKernelGGL((colmx_inv_kernel<CT, P, true>), gp, dim3(512), 0, st, a);
    } else {
        hipLaunchKernelGGL((colmx_inv_kernel<CT, P, false>), grid, dim3(512), 0, st, a);
    }
    return hipGetLastError();
}

template <int CT>
hipError_t launch_ct(bool fwd, const ColArgs& a, hipStream_t st) {
    switch (a.M1) {
    case 16: return launch_r<CT, 16>(fwd, a, st);
    case 32: return launch_r<CT, 32>(fwd, a, st);
    case 64: return launch_r<CT, 64>(fwd, a, st);
    case 128: return launch_r<CT, 128>(fwd, a, st);
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
    // half rows: single real rows only (no second row in any sequence), matrix-core lengths only
    if (a.rows != a.M1 && (a.rows != a.M1 / 2 + 1 || a.M1 < 256 || a.B != 1)) return hipErrorInvalidValue;
    if (dtype == CT_F16) return launch_ct<CT_F16>(fwd, a, st);
    if (dtype == CT_BF16) return launch_ct<CT_BF16>(fwd, a, st);
    return hipErrorInvalidValue;
}

}  // namespace lcv
