// fused1d_kernels.h -- the fused causal FFT convolution for transform lengths M = 256 R <= 8192:
// the kernel templates and their launch templates.  Each mode is instantiated in its own
// translation unit (fused1d_conv.hip, fused1d_adj.hip, fused1d_part.hip, fused1d_sparse.hip,
// fused1d.hip), so the modes compile in parallel.
//
// One workgroup (8 waves) transforms 32 tiles of 256 points at a time: one (pair of) sequence
// rows when R = 32, or 32 / R of them for shorter transforms.  Digits:
//     n = 256 n1 + 16 n2 + n3,     f = k1 + R k2 + 16 R k3.
// Forward (zero-padded input: n1 < R/2 only):
//   F1  radix-R over n1, matrix-core blocks, columns (n2, n3)              LDS V -> LDS XY
//   F2  radix-16 over n2 with w_{16R}^{n2 k1} folded into the block         registers
//   T   w_256^{n3 k2} (the only twiddle that needs the vector ALU)         registers
//   F3  radix-16 over n3 with w_M^{n3 k1} folded into the block            registers
// Pointwise product with the filter spectrum (D folded in: (K + D) / M), then the mirror
// image of the forward chain, and I3 computes only n1 < R/2: the causal truncation
// (Caracal abstract on the "RubiConv" page).  Two real rows b, b+1 with the same filter ride
// in one complex sequence x_b + i x_{b+1}: the filter is real, so the real and imaginary
// parts of the result are the two convolutions.
//
// The chain follows the fusion the pages describe -- FFT, pointwise spectral product and
// inverse FFT with no intermediate off-chip traffic ("FlashConv" page, Mechanism; FlashFFTConv
// abstract) -- and the block-matrix form of the FFT (same passages).  Block sizes, the
// register-resident tiles and the twiddle folding are this implementation's own.
#pragma once
#include <type_traits>

#include "fused_io.h"
#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

// MODE: conv / filter / row / row-forward / adjoint / partial.  GQ, GV: pre-gate and post-gate
// present (conv, adjoint, partial).  The adjoint runs the convolution chain on dy (pre-gated by v)
// with the conjugate spectrum, which turns the causal sum into the correlation sum over later
// positions, and writes two gated copies of the result: du = q dx and dq = u dx.
// The partial mode (a filter of at most M/2 taps on a sequence of any length) takes one block of
// C = M/2 output positions per item: the window [jC - C, jC + C) of the input fills the whole
// transform, and the upper half of the circular result is exactly the block's linear
// convolution (the lower half, where the window wraps, is not computed).
// The sparse mode is the convolution with the filter spectrum kept only on the frequency blocks
// (tiles, f mod R = k1) whose bit is set in a.keep: a wave whose tiles are all dropped skips its
// register chain and leaves zero tiles, and D x is added in the time domain (a dropped tile
// still carries D X), from the x values V holds for the lane's own slot.
template <int R, int CT, int IO, int MODE, bool GQ, bool GV>
__global__ void __launch_bounds__(512) fused1d_kernel(const Fused1DArgs a) {
    constexpr int P = 32 / R;                  // sequences per workgroup iteration
    constexpr int M = 256 * R;
    constexpr int C = M / 2;                   // partial mode: output positions per item
    constexpr bool ADJ = MODE == MODE_ADJ;
    constexpr bool PART = MODE == MODE_PART;
    constexpr bool SPARSE = MODE == MODE_SPARSE;
    constexpr bool SAVE = MODE == MODE_SAVE;
    // learned Butterfly: factor blocks from the caller (a.tables), one real row per transform
    // (its result is complex: the real part is kept), D x added in the time domain
    constexpr bool LBF = MODE == MODE_LBF;
    constexpr bool DTIME = SPARSE || LBF;            // D x added in the time domain
    constexpr bool CONV = MODE == MODE_CONV || ADJ || SPARSE || SAVE || LBF;  // batch-row input and output, half input
    constexpr bool BATCH = CONV || PART;             // batch rows, gates, filter per channel
    constexpr bool HALF_IN = (CONV || MODE == MODE_FILTER);
    constexpr bool HALF_OUT = BATCH;
    constexpr bool INV = (BATCH || MODE == MODE_ROW);
    constexpr int NIN = HALF_IN ? R / 2 : R;   // nonzero n1 rows
    constexpr int NOUT = HALF_OUT ? R / 2 : R; // n1 rows produced
    constexpr int OUT0 = PART ? R / 2 : 0;     // first n1 row produced
    constexpr int KCF = (R + 15) / 16;         // table grid (full variant)
    constexpr int KC1 = (NIN + 15) / 16;
    constexpr int RB1 = (R + 15) / 16;
    constexpr int KC3 = (R + 15) / 16;
    constexpr int RB3 = (NOUT + 15) / 16;
    constexpr int RB3_0 = OUT0 / 16;           // first I3 row block of the table used
    constexpr int EW = CT == CT_F32 ? 2 : 1;   // LDS words per complex element
    constexpr int SV = 260;                    // V: row stride (elements) per n1 row
    constexpr int ST = 324, SR = 20;           // XY: tile stride, row stride inside a tile
    constexpr int SO = 260;                    // O: row stride (complex fp32)
    constexpr int V_W = P * NIN * SV * EW;
    constexpr int XY_W = 32 * ST * EW;
    // fp32 row and partial passes: O (same element size as V) aliases V; both are used
    // wave-locally, and O then keeps V's rows per sequence so that a wave's O rows lie in its
    // own V columns
    constexpr bool O_ALIAS = ((MODE == MODE_ROW || PART) && CT == CT_F32);
    constexpr int OSEQ = O_ALIAS ? NIN : NOUT; // O rows per sequence
    constexpr int O_W = (INV && !O_ALIAS) ? P * NOUT * SO * 2 : 0;
    constexpr bool RES = (CT != CT_F32);       // matrix images resident in registers
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
    // The radix-R blocks (F1, I3) are shared by all waves: on the convolution path they live in
    // LDS (copied once), which keeps the per-tile blocks in registers without spills.
    constexpr bool IMG_LDS = RES && (BATCH || MODE == MODE_ROW);
    constexpr int IMGS_W = IMG_LDS ? (T_F2 - T_F1) / 4 : 0;
    constexpr int IOW = IO == CT_F32 ? 2 : 1;  // uint4 per 8 io elements
    // One sequence per iteration (R = 32) and 16-bit spectra: the filter spectrum of the
    // current channel stays in LDS and is reloaded only when the channel changes (consecutive
    // items are the batch pairs of one channel).
    constexpr bool KF_LDS = BATCH && R == 32 && IO != CT_F32;
    constexpr int KF_W = KF_LDS ? 32 * 64 * 4 : 0;

    __shared__ __attribute__((aligned(16))) uint32_t lds[V_W + XY_W + O_W + IMGS_W + KF_W];
    uint32_t* V = lds;
    uint32_t* XY = lds + V_W;
    float* O = (float*)(O_ALIAS ? lds : lds + V_W + XY_W);
    uint32_t* IMGS = lds + V_W + XY_W + O_W;
    uint4* KFL = (uint4*)(lds + V_W + XY_W + O_W + IMGS_W);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const char* tab = (const char*)a.tables;

    // ---- loop-invariant registers: twiddles and matrix images ------------------------------
    f32x4 twr, twi;
    {
        const float4* tp = (const float4*)(tab + T_TW) + lane * 2;
        float4 t0 = tp[0], t1 = tp[1];
        twr = f32x4{t0.x, t0.z, t1.x, t1.z};
        twi = f32x4{t0.y, t0.w, t1.y, t1.w};
    }
    MatImg<CT> mf2[4], mf3[4], mi1[4], mi2[4], mf1[RB1][KC1], mi3[RB3][KC3];
    if constexpr (RES) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k1 = (wave * 4 + i) % R;
            mf2[i] = load_img<CT>(tab + T_F2, k1, lane);
            mf3[i] = load_img<CT>(tab + T_F3, k1, lane);
            if constexpr (INV) {
                mi1[i] = load_img<CT>(tab + T_I1, k1, lane);
                mi2[i] = load_img<CT>(tab + T_I2, k1, lane);
            }
        }
        if constexpr (IMG_LDS) {
            for (int w = tid; w < IMGS_W / 4; w += 512) ((uint4*)IMGS)[w] = ((const uint4*)(tab + T_F1))[w];
            __syncthreads();  // every wave reads all of them
        } else {
#pragma unroll
            for (int rb = 0; rb < RB1; ++rb)
#pragma unroll
                for (int kc = 0; kc < KC1; ++kc) mf1[rb][kc] = load_img<CT>(tab + T_F1, rb * KCF + kc, lane);
            if constexpr (INV) {
#pragma unroll
                for (int rb = 0; rb < RB3; ++rb)
#pragma unroll
                    for (int kc = 0; kc < KC3; ++kc)
                        mi3[rb][kc] = load_img<CT>(tab + T_I3, (RB3_0 + rb) * KCF + kc, lane);
            }
        }
    }
    auto F1 = [&](int rb, int kc) LCV_INLINE {
        if constexpr (IMG_LDS) return load_img_lds<CT>(IMGS, rb * KCF + kc, lane);
        else return RES ? mf1[rb][kc] : load_img<CT>(tab + T_F1, rb * KCF + kc, lane);
    };
    auto I3 = [&](int rb, int kc) LCV_INLINE {  // rb counts from the first row block produced
        if constexpr (IMG_LDS) return load_img_lds<CT>(IMGS + (T_I3 - T_F1) / 4, (RB3_0 + rb) * KCF + kc, lane);
        else return RES ? mi3[rb][kc] : load_img<CT>(tab + T_I3, (RB3_0 + rb) * KCF + kc, lane);
    };
    auto F2 = [&](int i) LCV_INLINE { return RES ? mf2[i] : load_img<CT>(tab + T_F2, (wave * 4 + i) % R, lane); };
    auto F3 = [&](int i) LCV_INLINE { return RES ? mf3[i] : load_img<CT>(tab + T_F3, (wave * 4 + i) % R, lane); };
    auto I1 = [&](int i) LCV_INLINE { return RES ? mi1[i] : load_img<CT>(tab + T_I1, (wave * 4 + i) % R, lane); };
    auto I2 = [&](int i) LCV_INLINE { return RES ? mi2[i] : load_img<CT>(tab + T_I2, (wave * 4 + i) % R, lane); };

    // sparse: bit i set when this wave's tile i is a kept frequency block (wave-uniform)
    uint32_t wave_keep = 0xfu;
    if constexpr (SPARSE) {
        wave_keep = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) wave_keep |= ((a.keep >> ((wave * 4 + i) % R)) & 1u) << i;
    }

    // ---- work decomposition ---------------------------------------------------------------
    const uint32_t Bp = (uint32_t)(LBF ? a.B : (a.B + 1) / 2);  // pairs (LBF: rows) per channel
    const int64_t first = (int64_t)blockIdx.x * a.per_wg;
    const int64_t last = first + a.per_wg < a.nitems ? first + a.per_wg : a.nitems;
    const int64_t HN = a.H * a.N;
    const int m1s = a.M1 > 1 ? __builtin_ctzll((unsigned long long)a.M1) : 0;  // M1 is a power of 2
    // CONV item -> (channel h, first batch row b); 32-bit: item counts stay below 2^32
    auto decode = [&](int64_t item, int64_t& h, int64_t& b) LCV_INLINE {
        const uint32_t it = (uint32_t)item, hh = it / Bp;
        h = hh;
        b = (LBF ? 1 : 2) * (int64_t)(it - hh * Bp);
    };
    // PART: the sequences of a channel are its (batch row b, block j) windows, s = b nch + j; an
    // item is a pair of consecutive sequences (s0, s0 + 1) of one channel, so two blocks of one
    // row share a transform when the batch is odd or 1.  item -> (channel h, first sequence s0).
    const uint32_t nch = (uint32_t)(PART ? a.nchunk : 1);
    const uint32_t nseq = (uint32_t)(PART ? a.B * a.nchunk : 1);   // sequences per channel
    const uint32_t sp = (nseq + 1) / 2;                              // sequence pairs per channel
    auto decode_part = [&](int64_t item, int64_t& h, int64_t& s0) LCV_INLINE {
        const uint32_t it = (uint32_t)item, hh = it / sp;
        h = hh;
        s0 = 2 * (int64_t)(it - hh * sp);
    };
    // channel of a CONV or PART item
    auto channel_of = [&](int64_t item) LCV_INLINE {
        int64_t h, b;
        if constexpr (PART) decode_part(item, h, b);
        else decode(item, h, b);
        return h;
    };
    // ROW/ROWFWD item -> workspace row (local sequence * M1 + k_hi).  ROW items run k_hi-major
    // (item = k_hi * sequences + local sequence): the batch pairs of one channel, consecutive
    // sequences, then read the same spectrum row one after another on one workgroup.
    const uint32_t nsq = (uint32_t)(a.nitems >> m1s);
    auto ws_row = [&](int64_t item) LCV_INLINE -> int64_t {
        if constexpr (MODE == MODE_ROW) {
            const uint32_t it = (uint32_t)item, kh = it / nsq, sl = it - kh * nsq;
            return ((int64_t)sl << m1s) + kh;
        } else {
            return item;
        }
    };
    // ROW/ROWFWD item -> (channel h, row k_hi)
    auto decode_row = [&](int64_t item, int64_t& h, int64_t& khi) LCV_INLINE {
        const int64_t r = ws_row(item);
        const int64_t s = a.seq0 + (r >> m1s);
        khi = r & (a.M1 - 1);
        h = (int64_t)((uint32_t)s / (uint32_t)a.seq_per_h);
    };

    // Slots of P0 / P4: 8 consecutive elements of one sequence row.  A wave's slots are the
    // columns of its own radix-R blocks (blocks wave*BPW .. +BPW-1, every row n1), so the input
    // a wave packs into V is exactly what its F1 reads, and the output it stores is exactly
    // what its I3 wrote to O: no barrier is needed around P0 and P4.  Slot ci of the wave:
    // row n1 = ci / (2 BPW), block wave*BPW + (ci / 2) % BPW, half ci % 2 of the block.
    auto slot = [&](int ci, int& p, int& n0) LCV_INLINE {
        const int n1 = ci / (2 * BPW), blk = wave * BPW + (ci >> 1) % BPW;
        p = blk >> 4;
        n0 = 256 * n1 + 16 * (blk & 15) + 8 * (ci & 1);
    };
    // Half-length input (one slot per lane): sequence p_io of the iteration, elements n0_io..+8.
    int p_io, n0_io;
    slot(lane, p_io, n0_io);
    // Element offsets of the slot's two rows, clamped into range so that every load can be
    // issued unconditionally (out-of-range slots are masked where the data is used).  With no
    // branches around memory instructions the compiler's wait counts stay exact, which keeps
    // the software pipeline below intact.
    // For R >= 4 the blocks of a wave lie in one sequence, so the row arithmetic is
    // wave-uniform: readfirstlane moves it to the scalar unit.
    auto io_offsets = [&](int64_t item, int64_t& o0, int64_t& o1, bool& ok0, bool& ok1) LCV_INLINE {
        ok0 = item < last && n0_io < a.N;
        int64_t itc = item < last ? item : last - 1;
        if constexpr (R >= 4) itc = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)itc);
        const int64_t n0c = n0_io < a.N ? n0_io : a.N - 8;
        if constexpr (CONV) {
            int64_t h, b;
            decode(itc, h, b);
            const int64_t row0 = (b * a.H + h) * a.N;
            const int64_t row1 = !LBF && b + 1 < a.B ? row0 + HN : row0;
            o0 = row0 + n0c;
            o1 = row1 + n0c;
            ok1 = ok0 && !LBF && b + 1 < a.B;
        } else {
            o0 = itc * a.N + n0c;
            o1 = o0;
            ok1 = false;
        }
    };
    // PART: for each sequence (b, j) of the item's pair, the slot's window half `half` (0: the
    // previous block, 1: block j) is position (j - 1 + half) C + n0_io of row b; outside [0, N),
    // or past the channel's last sequence, it reads as zero and is never stored.  The two
    // sequences can lie in different rows at different positions: ok0 and ok1 are independent.
    auto part_offsets = [&](int64_t item, int half, int64_t& o0, int64_t& o1, bool& ok0, bool& ok1) LCV_INLINE {
        int64_t itc = item < last ? item : last - 1;
        if constexpr (R >= 4) itc = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)itc);
        int64_t h, s0;
        decode_part(itc, h, s0);
        auto one = [&](int64_t sq, int64_t& o, bool& ok) LCV_INLINE {
            const bool valid = sq < (int64_t)nseq;
            const uint32_t sc = (uint32_t)(valid ? sq : s0), b = sc / nch, j = sc - b * nch;
            const int64_t pos = ((int64_t)j - 1 + half) * C + n0_io;
            // chunk-local (a.local): the previous block reads as zero, so the result is block j's
            // own causal convolution
            ok = item < last && valid && pos >= 0 && pos < a.N && (half == 1 || !a.local);
            const int64_t posc = pos < 0 ? 0 : (pos < a.N ? pos : a.N - 8);
            o = ((int64_t)b * a.H + h) * a.N + posc;
        };
        one(s0, o0, ok0);
        one(s0 + 1, o1, ok1);
    };
    // Software pipeline: u, q of the NEXT iteration and v of this one are in flight while the
    // transforms run, so HBM latency overlaps the work.  PART holds both window halves
    // (index 2 half + row).
    constexpr int NRAW = PART ? 4 : 2;
    uint4 ru[NRAW][IOW], rq[NRAW][IOW], rv[2][IOW];
    auto issue_in = [&](int64_t it_base) LCV_INLINE {
        if constexpr (PART) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                int64_t o0, o1;
                bool k0, k1;
                part_offsets(it_base + p_io, half, o0, o1, k0, k1);
                load_raw<IO>(a.u, o0, ru[2 * half]);
                load_raw<IO>(a.u, o1, ru[2 * half + 1]);
                if constexpr (GQ) {
                    load_raw<IO>(a.q, o0, rq[2 * half]);
                    load_raw<IO>(a.q, o1, rq[2 * half + 1]);
                }
            }
            return;
        }
        int64_t o0, o1;
        bool k0, k1;
        io_offsets(it_base + p_io, o0, o1, k0, k1);
        load_raw<IO>(a.u, o0, ru[0]);
        if constexpr (CONV) {
            if constexpr (!LBF) load_raw<IO>(a.u, o1, ru[1]);
            if constexpr (GQ) {
                load_raw<IO>(a.q, o0, rq[0]);
                if constexpr (!LBF) load_raw<IO>(a.q, o1, rq[1]);
            }
        }
    };
    if constexpr (HALF_IN || PART) issue_in(first);
    int64_t kf_h = -1;   // channel whose spectrum KFL holds (wave-uniform)

    // One iteration.  FULL: every slot is in range (no stores need guarding).
    auto body = [&](const int64_t it0, auto full_tag) LCV_INLINE {
        constexpr bool FULL = decltype(full_tag)::value;
        // phases are kept apart: the compiler does not move work across the barriers
        __builtin_amdgcn_sched_barrier(0);
        // ================= P0: inputs -> V =================================================
        if constexpr (HALF_IN) {
            int64_t o0, o1;
            bool ok0, ok1;
            io_offsets(it0 + p_io, o0, o1, ok0, ok1);
            float xr[8], xi[8];
            unpack_raw<IO>(ru[0], xr);
            if constexpr (LBF) {
                if constexpr (GQ) {
                    float t[8];
                    unpack_raw<IO>(rq[0], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xr[i] *= t[i];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) xi[i] = 0.f;
            } else if constexpr (CONV) {
                unpack_raw<IO>(ru[1], xi);
                if constexpr (GQ) {
                    float t[8];
                    unpack_raw<IO>(rq[0], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xr[i] *= t[i];
                    unpack_raw<IO>(rq[1], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xi[i] *= t[i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) xi[i] = 0.f;
            }
            // Full iterations need no masks: every slot is in range, and the second row of an
            // odd batch's last pair duplicates the first (same results, same address).
            if constexpr (!FULL) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    xr[i] = ok0 ? xr[i] : 0.f;
                    xi[i] = ok1 ? xi[i] : 0.f;
                }
            }
            uint32_t* dst = V + ((p_io * NIN + (n0_io >> 8)) * SV + (n0_io & 255)) * EW;
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
        } else if constexpr (PART) {
            // both window halves of the slot: rows n1 < R/2 (previous block), then n1 >= R/2
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                int64_t o0, o1;
                bool ok0, ok1;
                part_offsets(it0 + p_io, half, o0, o1, ok0, ok1);
                float xr[8], xi[8];
                unpack_raw<IO>(ru[2 * half], xr);
                unpack_raw<IO>(ru[2 * half + 1], xi);
                if constexpr (GQ) {
                    float t[8];
                    unpack_raw<IO>(rq[2 * half], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xr[i] *= t[i];
                    unpack_raw<IO>(rq[2 * half + 1], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xi[i] *= t[i];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    xr[i] = ok0 ? xr[i] : 0.f;
                    xi[i] = ok1 ? xi[i] : 0.f;
                }
                const int n0 = n0_io + half * C;
                uint32_t* dst = V + ((p_io * NIN + (n0 >> 8)) * SV + (n0 & 255)) * EW;
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
            }
        } else {  // ROW / ROWFWD: one complex row of 8192 from the workspace (P == 1)
            const uint32_t* src = (const uint32_t*)a.u + ws_row(it0) * (int64_t)M * EW;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                int pp, n0;
                slot(lane + 64 * r, pp, n0);
                uint32_t* dst = V + ((n0 >> 8) * SV + (n0 & 255)) * EW;
#pragma unroll
                for (int i = 0; i < 2 * EW; ++i) ((uint4*)dst)[i] = ((const uint4*)(src + (int64_t)n0 * EW))[i];
            }
        }

        // Loads issued now: the filter spectrum of this wave's tiles and D (P2), then the
        // post-gate v (P4).  The next iteration's u, q follow after F1, so that the loads of
        // one iteration do not all queue at once.
        uint4 rk[4][IOW];
        uint32_t dk[4];
        if constexpr (KF_LDS) {
            // Each wave reads back only the spectrum slices it stores itself (its own four
            // tiles), so no barrier is needed; the loads are waited for inside the branch,
            // which is taken once per channel.
            const int64_t item = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(it0 < last ? it0 : last - 1));
            const int64_t h = channel_of(item);
            if (h != kf_h) {
                // D is folded in here, (K + D) / M, rounded once to the spectrum's type
                const uint4* src = (const uint4*)((const uint32_t*)a.kf + h * M) + wave * 4 * 64 + lane;
                const uint4 t0 = src[0], t1 = src[64], t2 = src[128], t3 = src[192];
                // (sparse: no fold, D x is added in the time domain)
                const float d = DTIME ? 0.f : raw1_to_f32<IO>(load1_raw<IO>(a.D, h)) * a.inv_m;
                auto fold = [&](uint32_t w) LCV_INLINE { return pack2<IO>(unpack_lo<IO>(w) + d, unpack_hi<IO>(w)); };
                auto fold4 = [&](uint4 t) LCV_INLINE { return make_uint4(fold(t.x), fold(t.y), fold(t.z), fold(t.w)); };
                KFL[(wave * 4 + 0) * 64 + lane] = fold4(t0);
                KFL[(wave * 4 + 1) * 64 + lane] = fold4(t1);
                KFL[(wave * 4 + 2) * 64 + lane] = fold4(t2);
                KFL[(wave * 4 + 3) * 64 + lane] = fold4(t3);
                kf_h = h;
            }
        } else if constexpr (INV) {
            // the 4 tiles of a wave belong to one sequence when R >= 4 (two when R == 2)
            constexpr int NSEQ_W = R >= 4 ? 1 : 2;
            int64_t bases[2] = {0, 0};
            uint32_t ds[2] = {0, 0};
#pragma unroll
            for (int s = 0; s < NSEQ_W; ++s) {
                int64_t item = it0 + (wave * 4 + 2 * s) / R;
                item = item < last ? item : last - 1;
                int64_t h;
                if constexpr (BATCH) {
                    h = channel_of(item);
                    bases[s] = h * M;
                } else {
                    int64_t khi;
                    decode_row(item, h, khi);
                    bases[s] = h * a.M + khi * M;
                }
                ds[s] = load1_raw<IO>(a.D, h);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = NSEQ_W == 1 ? 0 : i / 2, k1 = (wave * 4 + i) % R;
                dk[i] = ds[s];
                load_raw_c4<IO>(a.kf, bases[s] + ((int64_t)k1 * 64 + lane) * 4, rk[i]);
            }
        }
        if constexpr (BATCH && GV) {
            int64_t o0, o1;
            bool k0, k1;
            if constexpr (PART) part_offsets(it0 + p_io, 1, o0, o1, k0, k1);  // the block's outputs
            else io_offsets(it0 + p_io, o0, o1, k0, k1);
            load_raw<IO>(a.v, o0, rv[0]);
            if constexpr (!LBF) load_raw<IO>(a.v, o1, rv[1]);
        }
        // P1 reads only the V slots this wave wrote (its own blocks): no barrier.
        __builtin_amdgcn_sched_barrier(0);

        // ================= P1: F1 (radix R over n1), V -> XY =================================
        // Chunks of CH1 column blocks: all LDS reads of a chunk are issued before its matrix
        // products and all writes after them (a write to XY may not be reordered before a read
        // of V, so interleaving them would serialise the chunk on LDS latency).
        {
            constexpr int CH1 = (BPW < 2 || NIN > 16) ? 1 : 2;  // full-length input: one block at a time
            MatImg<CT> img1[RB1][KC1];
            static_for<0, RB1>([&](auto rr) LCV_INLINE {
                static_for<0, KC1>([&](auto kk) LCV_INLINE {
                    img1[decltype(rr)::value][decltype(kk)::value] = F1(decltype(rr)::value, decltype(kk)::value);
                });
            });
#pragma unroll 1
            for (int b0 = 0; b0 < BPW; b0 += CH1) {
                Operand<CT> din[CH1][KC1];
                static_for<0, CH1>([&](auto cc) LCV_INLINE {
                    constexpr int ci = decltype(cc)::value;
                    const int blk = wave * BPW + b0 + ci, p = blk >> 4, b = blk & 15;
                    static_for<0, KC1>([&](auto kk) LCV_INLINE {
                        constexpr int kc = decltype(kk)::value;
                        din[ci][kc] = lds_operand<CT>(V, [&](int j) {
                            const int n1 = 16 * kc + 4 * g + j;
                            return n1 < NIN ? (p * NIN + n1) * SV + 16 * b + c : -1;
                        });
                    });
                });
                Tile acc[CH1][RB1];
                static_for<0, CH1>([&](auto cc) LCV_INLINE {
                    constexpr int ci = decltype(cc)::value;
                    static_for<0, RB1>([&](auto rr) LCV_INLINE {
                        constexpr int rb = decltype(rr)::value;
                        acc[ci][rb].re = f32x4{0.f, 0.f, 0.f, 0.f};
                        acc[ci][rb].im = f32x4{0.f, 0.f, 0.f, 0.f};
                        static_for<0, KC1>([&](auto kk) LCV_INLINE {
                            constexpr int kc = decltype(kk)::value;
                            stage_keep_acc<CT>(img1[rb][kc], din[ci][kc], acc[ci][rb].re, acc[ci][rb].im);
                        });
                    });
                });
                static_for<0, CH1>([&](auto cc) LCV_INLINE {
                    constexpr int ci = decltype(cc)::value;
                    const int blk = wave * BPW + b0 + ci, p = blk >> 4, b = blk & 15;
                    static_for<0, RB1>([&](auto rr) LCV_INLINE {
                        constexpr int rb = decltype(rr)::value;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int k1 = 16 * rb + 4 * g + j;
                            if (k1 < R) lds_put<CT>(XY, (p * R + k1) * ST + b * SR + c, acc[ci][rb].re[j], acc[ci][rb].im[j]);
                        }
                    });
                });
            }
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);

        // ================= P2: F2, twiddle, F3, product, I1, twiddle, I2 (registers) =========
        // The wave's four tiles form two independent groups of two.  The stages of the two
        // groups are skewed by one: the matrix products of one group are issued next to the
        // vector work (twiddles, spectral product, packing) of the other, so both units stay
        // busy inside one wave.  A scheduling fence between steps keeps the skew.
        Operand<CT> opd[4];
        Tile xs[4];
        auto ld_op = [&](auto grp) LCV_INLINE {
            constexpr int i0 = 2 * decltype(grp)::value;
            static_for<i0, i0 + 2>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int t = wave * 4 + i;
                opd[i] = lds_operand<CT>(XY, [&](int j) { return t * ST + (4 * g + j) * SR + c; });
            });
        };
        // matrix stage st (1: F2, 2: F3, 3: I1, 4: I2) of a group
        auto mstage = [&](auto grp, auto stg) LCV_INLINE {
            constexpr int i0 = 2 * decltype(grp)::value, st = decltype(stg)::value;
            // raised priority while issuing: the products start as early as possible and run
            // under the other wave's vector work
            __builtin_amdgcn_s_setprio(1);
            static_for<i0, i0 + 2>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                if constexpr (st == 1) xs[i] = stage_swap<CT>(F2(i), opd[i]);       // (L = k2, K = n3)
                else if constexpr (st == 2) xs[i] = stage_keep<CT>(F3(i), opd[i]);  // (L = k2, K = k3)
                else if constexpr (st == 3) xs[i] = stage_swap<CT>(I1(i), opd[i]);  // (L = n3, K = k2)
                else xs[i] = stage_keep<CT>(I2(i), opd[i]);                         // (L = n3, K = n2)
            });
            __builtin_amdgcn_s_setprio(0);
        };
        // vector step after matrix stage st of a group
        auto vstep = [&](auto grp, auto stg) LCV_INLINE {
            constexpr int i0 = 2 * decltype(grp)::value, st = decltype(stg)::value;
            static_for<i0, i0 + 2>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int t = wave * 4 + i;
                if constexpr (st == 1) {
                    cmul4(xs[i], twr, twi);
                    opd[i] = to_operand<CT>(xs[i]);
                } else if constexpr (st == 2 && INV) {
                    f32x4 kr, ki;
                    if constexpr (KF_LDS) {
                        const uint4 kw = KFL[t * 64 + lane];  // (K + D) / M
                        unpack_raw_c4v<IO>(&kw, kr, ki);
                    } else {
                        unpack_raw_c4v<IO>(rk[i], kr, ki);
                        if constexpr (!DTIME) kr += raw1_to_f32<IO>(dk[i]) * a.inv_m;  // (K + D) / M
                    }
                    if constexpr (SPARSE) {  // a dropped block of a partly kept wave
                        const bool kept = (wave_keep >> i) & 1u;
                        kr = kept ? kr : f32x4{0.f, 0.f, 0.f, 0.f};
                        ki = kept ? ki : f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                    if constexpr (ADJ) cmulc4(xs[i], kr, ki);  // D is real: conj(K + D) = conj(K) + D
                    else cmul4(xs[i], kr, ki);
                    opd[i] = to_operand<CT>(xs[i]);
                } else if constexpr (st == 2) {
                    // spectrum in transform order, scaled by 1/M
                    const int p = t / R, k1 = t % R;
                    const int64_t item = it0 + p;
                    if (FULL || item < last) {
                        int64_t base;
                        if constexpr (MODE == MODE_FILTER) {
                            base = item * M;
                        } else if (a.wrows) {  // wrows rows per sequence (rows past them not formed)
                            const uint32_t sl = (uint32_t)item / (uint32_t)a.wrows;
                            const int64_t khi = (int64_t)((uint32_t)item - sl * (uint32_t)a.wrows);
                            base = (a.seq0 + sl) * a.M + khi * M;
                        } else {
                            const int64_t h = a.seq0 + (item >> m1s), khi = item & (a.M1 - 1);
                            base = h * a.M + khi * M;
                        }
                        store_c4v<IO>(a.y, base + ((int64_t)k1 * 64 + lane) * 4, xs[i].re * a.inv_m,
                                      xs[i].im * a.inv_m);
                    }
                } else if constexpr (st == 3) {
                    cmulc4(xs[i], twr, twi);
                    opd[i] = to_operand<CT>(xs[i]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        lds_put<CT>(XY, t * ST + (4 * g + j) * SR + c, xs[i].re[j], xs[i].im[j]);
                }
            });
        };
        using G0 = std::integral_constant<int, 0>;
        using G1 = std::integral_constant<int, 1>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        using S3 = std::integral_constant<int, 3>;
        using S4 = std::integral_constant<int, 4>;
        // one matrix product, then a share of the vector work, repeated: the two waves of a SIMD
        // leave each barrier in step, and fine interleaving lets one wave's products run under
        // the other's vector instructions
        auto interleave = [&](auto nv) LCV_INLINE {
            static_for<0, 4>([&](auto) LCV_INLINE {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, decltype(nv)::value, 0);
            });
        };
        auto chain = [&]() LCV_INLINE {
            ld_op(G0{});
            ld_op(G1{});
            mstage(G0{}, S1{});
            __builtin_amdgcn_sched_barrier(0);
            mstage(G1{}, S1{}); vstep(G0{}, S1{});
            interleave(std::integral_constant<int, 10>{});
            __builtin_amdgcn_sched_barrier(0);
            mstage(G0{}, S2{}); vstep(G1{}, S1{});
            interleave(std::integral_constant<int, 10>{});
            __builtin_amdgcn_sched_barrier(0);
            mstage(G1{}, S2{}); vstep(G0{}, S2{});
            interleave(std::integral_constant<int, 14>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (INV) {
                mstage(G0{}, S3{}); vstep(G1{}, S2{});
                interleave(std::integral_constant<int, 14>{});
                __builtin_amdgcn_sched_barrier(0);
                mstage(G1{}, S3{}); vstep(G0{}, S3{});
                interleave(std::integral_constant<int, 10>{});
                // the next iteration's u, q go out here (consumed in its P0): late enough to keep
                // their registers out of the busiest part of this phase
                if constexpr (HALF_IN || PART) issue_in(it0 + P);  // clamped: harmless past the end
                __builtin_amdgcn_sched_barrier(0);
                mstage(G0{}, S4{}); vstep(G1{}, S3{});
                interleave(std::integral_constant<int, 10>{});
                __builtin_amdgcn_sched_barrier(0);
                mstage(G1{}, S4{}); vstep(G0{}, S4{});
                interleave(std::integral_constant<int, 4>{});
                __builtin_amdgcn_sched_barrier(0);
                vstep(G1{}, S4{});
            } else {
                vstep(G1{}, S2{});
                if constexpr (HALF_IN) issue_in(it0 + P);
            }
        };
        // (fp32 runs the chain unconditionally: dropped blocks still multiply by zero, but a
        // branch around this chain, whose blocks come from global memory in fp32, sends the
        // compiler's scheduler into a very long search)
        if constexpr (SPARSE && CT != CT_F32) {
            if (wave_keep != 0) {
                chain();
            } else {
                // every tile of this wave is a dropped block: zero tiles for I3
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = wave * 4 + i;
#pragma unroll
                    for (int j = 0; j < 4; ++j) lds_put<CT>(XY, t * ST + (4 * g + j) * SR + c, 0.f, 0.f);
                }
                issue_in(it0 + P);
            }
        } else {
            chain();
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (INV) {
            // adjoint with gates: u for dq = u dx, loaded here (the transform registers are free)
            uint4 re2[2][IOW];
            if constexpr (ADJ && GV) {
                int64_t o0, o1;
                bool k0, k1;
                io_offsets(it0 + p_io, o0, o1, k0, k1);
                load_raw<IO>(a.e2, o0, re2[0]);
                load_raw<IO>(a.e2, o1, re2[1]);
            }
            // ================= P3: I3 (inverse radix R over k1, n1 < NOUT), XY -> O ============
            // Same chunked read / multiply / write order as P1.
            {
                constexpr int CH3 = (BPW < 2 || NOUT > 16) ? 1 : 2;
                MatImg<CT> img3[RB3][KC3];
                static_for<0, RB3>([&](auto rr) LCV_INLINE {
                    static_for<0, KC3>([&](auto kk) LCV_INLINE {
                        img3[decltype(rr)::value][decltype(kk)::value] = I3(decltype(rr)::value, decltype(kk)::value);
                    });
                });
#pragma unroll 1
                for (int b0 = 0; b0 < BPW; b0 += CH3) {
                    Operand<CT> din[CH3][KC3];
                    static_for<0, CH3>([&](auto cc) LCV_INLINE {
                        constexpr int ci = decltype(cc)::value;
                        const int blk = wave * BPW + b0 + ci, p = blk >> 4, b = blk & 15;
                        static_for<0, KC3>([&](auto kk) LCV_INLINE {
                            constexpr int kc = decltype(kk)::value;
                            din[ci][kc] = lds_operand<CT>(XY, [&](int j) {
                                const int k1 = 16 * kc + 4 * g + j;
                                return k1 < R ? (p * R + k1) * ST + b * SR + c : -1;
                            });
                        });
                    });
                    Tile acc[CH3][RB3];
                    static_for<0, CH3>([&](auto cc) LCV_INLINE {
                        constexpr int ci = decltype(cc)::value;
                        static_for<0, RB3>([&](auto rr) LCV_INLINE {
                            constexpr int rb = decltype(rr)::value;
                            acc[ci][rb].re = f32x4{0.f, 0.f, 0.f, 0.f};
                            acc[ci][rb].im = f32x4{0.f, 0.f, 0.f, 0.f};
                            static_for<0, KC3>([&](auto kk) LCV_INLINE {
                                constexpr int kc = decltype(kk)::value;
                                stage_keep_acc<CT>(img3[rb][kc], din[ci][kc], acc[ci][rb].re, acc[ci][rb].im);
                            });
                        });
                    });
                    static_for<0, CH3>([&](auto cc) LCV_INLINE {
                        constexpr int ci = decltype(cc)::value;
                        const int blk = wave * BPW + b0 + ci, p = blk >> 4, b = blk & 15;
                        static_for<0, RB3>([&](auto rr) LCV_INLINE {
                            constexpr int rb = decltype(rr)::value;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                // output row: transform row n1 = 16 (RB3_0 + rb) + 4g + j, minus OUT0
                                const int o = 16 * (RB3_0 + rb) + 4 * g + j - OUT0;
                                if (o >= 0 && o < NOUT)
                                    *(float2*)(O + 2 * ((p * OSEQ + o) * SO + 16 * b + c)) =
                                        make_float2(acc[ci][rb].re[j], acc[ci][rb].im[j]);
                            }
                        });
                    });
                }
            }
            // P4 reads only the O slots this wave wrote (its own blocks): no barrier.
            __builtin_amdgcn_sched_barrier(0);

            // ================= P4: epilogue ==================================================
            if constexpr (BATCH) {
                int64_t o0, o1;
                bool ok0, ok1;
                if constexpr (PART) part_offsets(it0 + p_io, 1, o0, o1, ok0, ok1);  // block outputs
                else io_offsets(it0 + p_io, o0, o1, ok0, ok1);
                const float4* src = (const float4*)(O + 2 * ((p_io * OSEQ + (n0_io >> 8)) * SO + (n0_io & 255)));
                float yr[8], yi[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float4 w = src[i];
                    yr[2 * i] = w.x; yi[2 * i] = w.y; yr[2 * i + 1] = w.z; yi[2 * i + 1] = w.w;
                }
                if constexpr (DTIME) {
                    // + D x, from the slot's packed pair in V (written by this lane in P0)
                    const int64_t hc = channel_of(it0 + p_io < last ? it0 + p_io : last - 1);
                    const float d = raw1_to_f32<IO>(load1_raw<IO>(a.D, hc));
                    const uint32_t* xv = V + ((p_io * NIN + (n0_io >> 8)) * SV + (n0_io & 255)) * EW;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        float xr_, xi_;
                        if constexpr (CT == CT_F32) {
                            const float2 e = ((const float2*)xv)[i];
                            xr_ = e.x;
                            xi_ = e.y;
                        } else {
                            xr_ = unpack_lo<CT>(xv[i]);
                            xi_ = unpack_hi<CT>(xv[i]);
                        }
                        yr[i] += d * xr_;
                        yi[i] += d * xi_;
                    }
                }
                if constexpr (ADJ && GV) {
                    // dq = u dx (second output), before dx is gated into du below
                    float t[8], zr[8], zi[8];
                    unpack_raw<IO>(re2[0], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) zr[i] = yr[i] * t[i];
                    unpack_raw<IO>(re2[1], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) zi[i] = yi[i] * t[i];
                    if constexpr (!FULL) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) zi[i] = o1 != o0 ? zi[i] : zr[i];
                    }
                    if (FULL || ok0) {
                        store8_nt<IO>(a.y2, o0, zr);
                        store8_nt<IO>(a.y2, o1, zi);
                    }
                }
                if constexpr (SAVE) {
                    // the pre-gate output c, masked like y below
                    float ci[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) ci[i] = FULL || o1 != o0 ? yi[i] : yr[i];
                    if (FULL || ok0) {
                        store8_nt<IO>(a.y2, o0, yr);
                        store8_nt<IO>(a.y2, o1, ci);
                    }
                }
                if constexpr (GV) {
                    float t[8];
                    unpack_raw<IO>(rv[0], t);
#pragma unroll
                    for (int i = 0; i < 8; ++i) yr[i] *= t[i];
                    if constexpr (!LBF) {
                        unpack_raw<IO>(rv[1], t);
#pragma unroll
                        for (int i = 0; i < 8; ++i) yi[i] *= t[i];
                    }
                }
                if constexpr (LBF) {
                    // one real row: the real part of the result
                    if (FULL || ok0) store8_nt<IO>(a.y, o0, yr);
                } else if constexpr (PART) {
                    // the two sequences are stored independently (different rows or blocks)
                    if (ok0) store8_nt<IO>(a.y, o0, yr);
                    if (ok1) store8_nt<IO>(a.y, o1, yi);
                } else {
                    // odd B, partial iteration: the masked second row must not overwrite the first
                    if constexpr (!FULL) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) yi[i] = o1 != o0 ? yi[i] : yr[i];
                    }
                    if (FULL || ok0) {
                        store8_nt<IO>(a.y, o0, yr);
                        store8_nt<IO>(a.y, o1, yi);
                    }
                }
            } else {  // ROW: complex row back to the workspace, in compute type
                uint32_t* dstrow = (uint32_t*)a.y + ws_row(it0) * (int64_t)M * EW;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    int pp, n0;
                    slot(lane + 64 * r, pp, n0);
                    const float4* src = (const float4*)(O + 2 * ((n0 >> 8) * SO + (n0 & 255)));  // P == 1
                    float w[16];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float4 s = src[i];
                        w[4 * i] = s.x; w[4 * i + 1] = s.y; w[4 * i + 2] = s.z; w[4 * i + 3] = s.w;
                    }
                    if constexpr (CT == CT_F32) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            ((float4*)(dstrow + (int64_t)n0 * 2))[i] =
                                make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
                    } else {
                        uint4 q0, q1;
                        q0.x = pack2<CT>(w[0], w[1]);   q0.y = pack2<CT>(w[2], w[3]);
                        q0.z = pack2<CT>(w[4], w[5]);   q0.w = pack2<CT>(w[6], w[7]);
                        q1.x = pack2<CT>(w[8], w[9]);   q1.y = pack2<CT>(w[10], w[11]);
                        q1.z = pack2<CT>(w[12], w[13]); q1.w = pack2<CT>(w[14], w[15]);
                        ((uint4*)(dstrow + n0))[0] = q0;
                        ((uint4*)(dstrow + n0))[1] = q1;
                    }
                }
            }
        }
    };

    // Full iterations (every slot in range) run without store guards; a partial last
    // iteration, or a length that does not fill the half transform, takes the guarded body.
    const bool whole_rows = !PART && (!HALF_IN || a.N == M / 2);
    int64_t it0 = first;
    if (whole_rows) {
        for (; it0 + P <= last; it0 += P) body(it0, std::integral_constant<bool, true>{});
    }
    for (; it0 < last; it0 += P) body(it0, std::integral_constant<bool, false>{});
}

// ------------------------------------------------------------------------------------------
// Pipelined kernel for M = 8192 (R = 32), 16-bit types, whole rows (N = 4096), convolution.
//
// Same transform chain as fused1d_kernel, arranged so that the vector/matrix-heavy register
// chain (P2) of one iteration runs beside the LDS- and memory-heavy wave-local work of its
// neighbours: segment k holds P2(k) and W(k) = { P3, P4 of k-1; P0, P1 of k+1 }, with one
// barrier per segment.  XY is double-buffered (iteration parity).  Waves 0-3 run P2 first and
// waves 4-7 run W first, so each SIMD (which hosts waves w and w+4) pairs the two kinds of work.
// O is kept in the compute type and shares V's space (both are used wave-locally); the filter
// spectrum has two LDS copies so the next channel's can be loaded while the current one is read.
// ADJ: the adjoint chain (conjugate spectrum; outputs du = q dx and dq = u dx), as in
// fused1d_kernel.
// ROW: the row pass of the multi-pass path (the MODE_ROW chain of fused1d_kernel): an item is one
// complex 8192-point row of the workspace, transformed in full (F1 over all 32 n1, I3 back to
// all 32 rows), multiplied by its slice of the spectrum (registers, loaded one item ahead) and
// written back in place.  Items run k_hi-major over the chunk, so that the batch pairs of one
// channel meet the same spectrum row back to back.
// ------------------------------------------------------------------------------------------
template <int CT, bool GQ, bool GV, bool ADJ, bool SAVE = false, bool ROW = false>
__global__ void __launch_bounds__(512) conv8k_kernel(const Fused1DArgs a) {
    constexpr int R = 32, M = 8192, KCF = 2;
    constexpr int IMG = ImgBytes<CT>::value;
    constexpr int T_F1 = 0, T_I3 = T_F1 + IMG * 2 * KCF, T_F2 = T_I3 + IMG * KCF * KCF;
    constexpr int T_F3 = T_F2 + IMG * R, T_I1 = T_F3 + IMG * R, T_I2 = T_I1 + IMG * R, T_TW = T_I2 + IMG * R;
    constexpr int ST = 260;                      // XY tile stride (words)
    constexpr int SV = 260;                      // V / O row stride (words, one complex per word)
    constexpr int NR = ROW ? 32 : 16;            // rows n1 of the V / O slots
    constexpr int NIM = ROW ? 8 : 4;             // F1 and I3 block images kept in LDS
    constexpr int NKF = ROW ? 0 : 2;             // LDS copies of the spectrum (ROW: registers)
    constexpr int XY_W = 32 * ST, V_W = NR * SV, IM_W = NIM * IMG / 4, KF_W = 32 * 64 * 4;
    __shared__ __attribute__((aligned(16))) uint32_t lds[2 * XY_W + V_W + IM_W + NKF * KF_W];
    uint32_t* const XYb = lds;                   // two buffers of XY_W
    uint32_t* const V = lds + 2 * XY_W;          // input slots (P0 -> P1) and output slots (P3 -> P4)
    uint32_t* const IMS = V + V_W;               // F1 (rb = 0, 1) and I3 (kc = 0, 1) images
    uint4* const KFL = (uint4*)(IMS + IM_W);     // two copies of (K + D) / M, 32 tiles x 64 lanes

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const char* tab = (const char*)a.tables;
    const int64_t first = (int64_t)blockIdx.x * a.per_wg;
    const int64_t last = first + a.per_wg < a.nitems ? first + a.per_wg : a.nitems;
    if (first >= last) return;

    // Tile element (row r, column col) of tile t.  Rows 4g + j of one instruction land in four
    // different bank groups (the XOR on row / 4); tiles 4g + j of one instruction do too (the
    // stride 260 = 4 mod 64 words).
    auto xy_addr = [&](int t, int r, int col) LCV_INLINE { return t * ST + ((16 * r + col) ^ (((r >> 2) & 3) << 4)); };

    // ---- loop-invariant registers and LDS ---------------------------------------------------
    f32x4 twr, twi;
    {
        const float4* tp = (const float4*)(tab + T_TW) + lane * 2;
        float4 t0 = tp[0], t1 = tp[1];
        twr = f32x4{t0.x, t0.z, t1.x, t1.z};
        twi = f32x4{t0.y, t0.w, t1.y, t1.w};
    }
    MatImg<CT> mf2[4], mf3[4], mi1[4], mi2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k1 = wave * 4 + i;
        mf2[i] = load_img<CT>(tab + T_F2, k1, lane);
        mf3[i] = load_img<CT>(tab + T_F3, k1, lane);
        mi1[i] = load_img<CT>(tab + T_I1, k1, lane);
        mi2[i] = load_img<CT>(tab + T_I2, k1, lane);
    }
    {
        // F1 blocks (rb, kc) are table images rb KCF + kc, I3 blocks (rb, kc) likewise.  CONV:
        // F1 (0, 0), (1, 0) (inputs n1 < 16) and I3 (0, 0), (0, 1) (outputs n1 < 16).  ROW: all
        // four of each, F1 (rb, kc) at rb KCF + kc and I3 (rb, kc) at 4 + rb KCF + kc.
        // (offsets computed, not read from a local array: a dynamically indexed array would be
        // placed in LDS)
        auto src_of = [&](int img) LCV_INLINE {
            if constexpr (ROW) return img < 4 ? T_F1 + IMG * img : T_I3 + IMG * (img - 4);
            else return img < 2 ? T_F1 + IMG * KCF * img : T_I3 + IMG * (img - 2);
        };
        for (int w = tid; w < IM_W / 4; w += 512) {
            const int img = w / (IMG / 16), off = w % (IMG / 16);
            ((uint4*)IMS)[w] = ((const uint4*)(tab + src_of(img)))[off];
        }
        __syncthreads();  // every wave reads all four
    }

    // ---- items and addresses --------------------------------------------------------------
    const uint32_t Bp = (uint32_t)((a.B + 1) / 2);
    // element strides between batch rows and between channels ([B][H][N] unless set)
    const int64_t sB = a.sb ? a.sb : a.H * a.N, sH = a.sh ? a.sh : a.N;
    auto channel = [&](int64_t item) LCV_INLINE {
        return (int64_t)((uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)item) / Bp);
    };
    // ROW: item -> workspace row (local sequence * wr + k_hi), item = k_hi * sequences + local
    // sequence: the batch pairs of one channel (consecutive sequences) read the same spectrum
    // row back to back.  (Visiting rows k_hi and M1 - k_hi together, which read one stored row
    // through the spectrum's conjugate symmetry, measured slower.)
    // The workspace holds wr rows per sequence: M1, or M1/2 + 1 when each sequence is one real row
    // (the rest follow by conjugate symmetry and are never formed).
    const uint32_t wr = ROW ? (uint32_t)(a.wrows ? a.wrows : a.M1) : 1u;
    const uint32_t nsq = ROW ? (uint32_t)(a.nitems / wr) : 1u;
    auto row_of = [&](int64_t item, uint32_t& sl, uint32_t& kh) LCV_INLINE {
        item = item < last ? item : last - 1;
        const uint32_t it = __builtin_amdgcn_readfirstlane((uint32_t)item);
        kh = it / nsq;
        sl = it - kh * nsq;
    };
    auto ws_row = [&](int64_t item) LCV_INLINE -> int64_t {
        uint32_t sl, kh;
        row_of(item, sl, kh);
        return (int64_t)sl * wr + kh;
    };
    // this lane's slot: row n1 = lane / 4, columns 32 wave + 8 (lane % 4) .. +8 (the wave's blocks)
    const int s_n1 = lane >> 2, s_col = 32 * wave + 8 * (lane & 3);
    const int64_t s_n0 = 256 * s_n1 + s_col;
    // element offsets of the slot in the item's two batch rows (an odd batch's last pair
    // repeats its row: same data in, same results out to the same address)
    auto offsets = [&](int64_t item, int64_t& o0, int64_t& o1) LCV_INLINE {
        item = item < last ? item : last - 1;
        const uint32_t it = __builtin_amdgcn_readfirstlane((uint32_t)item), hh = it / Bp;
        const int64_t b = 2 * (int64_t)(it - hh * Bp);
        const int64_t row0 = b * sB + hh * sH;
        o0 = row0 + s_n0;
        o1 = (b + 1 < a.B ? row0 + sB : row0) + s_n0;
    };
    uint4 ru[2], rq[2], rv[2], re2[2];
    uint4 rw0, rw1, rw2, rw3;  // ROW: this lane's slot of the row, rows n1 = s_n1 and s_n1 + 16
    uint4 rk[4];         // ROW: the spectrum slice of this wave's four tiles, one item ahead
    float rkd = 0.f;     // ROW: D[h] / M of that item
    auto issue_row = [&](int64_t item) LCV_INLINE {
        const uint4* src = (const uint4*)((const uint32_t*)a.u + ws_row(item) * M + s_n0);
        rw0 = src[0];
        rw1 = src[1];
        rw2 = src[16 * 256 / 4];
        rw3 = src[16 * 256 / 4 + 1];
    };
    auto issue_kf_row = [&](int64_t item) LCV_INLINE {
        uint32_t sl, kh;
        row_of(item, sl, kh);
        const int64_t h = (int64_t)((uint32_t)(a.seq0 + sl) / (uint32_t)a.seq_per_h);
        const uint4* src = (const uint4*)((const uint32_t*)a.kf + h * a.M + (int64_t)kh * M);
        static_for<0, 4>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            rk[i] = src[(wave * 4 + i) * 64 + lane];
        });
        rkd = raw1_to_f32<CT>(load1_raw<CT>(a.D, h)) * a.inv_m;
    };
    auto issue_uq = [&](int64_t item) LCV_INLINE {
        if constexpr (ROW) {
            issue_row(item);
            return;
        }
        int64_t o0, o1;
        offsets(item, o0, o1);
        load_raw<CT>(a.u, o0, &ru[0]);
        load_raw<CT>(a.u, o1, &ru[1]);
        if constexpr (GQ) {
            load_raw<CT>(a.q, o0, &rq[0]);
            load_raw<CT>(a.q, o1, &rq[1]);
        }
    };
    auto issue_v = [&](int64_t item) LCV_INLINE {
        if constexpr (GV) {
            int64_t o0, o1;
            offsets(item, o0, o1);
            load_raw<CT>(a.v, o0, &rv[0]);
            load_raw<CT>(a.v, o1, &rv[1]);
        }
    };
    // adjoint with gates: u for dq = u dx, issued just before the item's P3
    auto issue_e2 = [&](int64_t item) LCV_INLINE {
        if constexpr (ADJ && GV) {
            int64_t o0, o1;
            offsets(item, o0, o1);
            load_raw<CT>(a.e2, o0, &re2[0]);
            load_raw<CT>(a.e2, o1, &re2[1]);
        }
    };
    // (K + D) / M of channel h into copy kb, this wave's tiles only (read back by this wave)
    // The filter is real, so its spectrum is Hermitian, K[M - f] = conj(K[f]): with
    // f = k1 + 32 k2 + 512 k3 held at tile k1, lane 16 g + k2, value j (k3 = 4 g + j), tile
    // 32 - k1 (k1 = 1 .. 15) is tile k1 read at lane 63 - l with the four values reversed and
    // conjugated.  Only tiles 0 .. 16 are read from memory (the loads stay unconditional: a
    // mirrored tile selects its source address and then its values).
    auto load_kf = [&](int64_t h, int kb) LCV_INLINE {
        const uint4* base = (const uint4*)((const uint32_t*)a.kf + h * M);
        uint4 t[4];
        static_for<0, 4>([&](auto ii) LCV_INLINE {
            constexpr int i = decltype(ii)::value;
            const int k1 = wave * 4 + i;
            const bool mir = k1 > 16;
            const uint4 m = base[(mir ? 32 - k1 : k1) * 64 + (mir ? 63 - lane : lane)];
            constexpr uint32_t S = 0x80000000u;   // sign of the imaginary half
            t[i] = mir ? make_uint4(m.w ^ S, m.z ^ S, m.y ^ S, m.x ^ S) : m;
        });
        const float d = raw1_to_f32<CT>(load1_raw<CT>(a.D, h)) * a.inv_m;
        auto fold = [&](uint32_t w) LCV_INLINE { return pack2<CT>(unpack_lo<CT>(w) + d, unpack_hi<CT>(w)); };
        auto fold4 = [&](uint4 v) LCV_INLINE { return make_uint4(fold(v.x), fold(v.y), fold(v.z), fold(v.w)); };
        uint4* dst = KFL + kb * (KF_W / 4) + wave * 4 * 64 + lane;
        dst[0] = fold4(t[0]);
        dst[64] = fold4(t[1]);
        dst[128] = fold4(t[2]);
        dst[192] = fold4(t[3]);
    };

    // ---- phases ------------------------------------------------------------------------------
    // P0: gate and pack this lane's slot of the item into V
    auto P0 = [&]() LCV_INLINE {
        if constexpr (ROW) {
            uint4* d0 = (uint4*)(V + s_n1 * SV + s_col);
            uint4* d1 = (uint4*)(V + (s_n1 + 16) * SV + s_col);
            d0[0] = rw0;
            d0[1] = rw1;
            d1[0] = rw2;
            d1[1] = rw3;
            return;
        }
        float xr[8], xi[8];
        unpack_raw<CT>(&ru[0], xr);
        unpack_raw<CT>(&ru[1], xi);
        if constexpr (GQ) {
            float t[8];
            unpack_raw<CT>(&rq[0], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[i] *= t[i];
            unpack_raw<CT>(&rq[1], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) xi[i] *= t[i];
        }
        uint4 w0, w1;
        w0.x = pack2<CT>(xr[0], xi[0]); w0.y = pack2<CT>(xr[1], xi[1]);
        w0.z = pack2<CT>(xr[2], xi[2]); w0.w = pack2<CT>(xr[3], xi[3]);
        w1.x = pack2<CT>(xr[4], xi[4]); w1.y = pack2<CT>(xr[5], xi[5]);
        w1.z = pack2<CT>(xr[6], xi[6]); w1.w = pack2<CT>(xr[7], xi[7]);
        uint4* dst = (uint4*)(V + s_n1 * SV + s_col);
        dst[0] = w0;
        dst[1] = w1;
    };
    // P1: F1 (radix 32 over n1 < 16) on this wave's two column blocks, V -> XY
    auto P1 = [&](uint32_t* XY) LCV_INLINE {
        if constexpr (ROW) {  // all 32 rows n1: two K chunks per output block
            Operand<CT> din[2][2];
            static_for<0, 2>([&](auto bb) LCV_INLINE {
                constexpr int bi = decltype(bb)::value;
                const int b = 2 * wave + bi;
                static_for<0, 2>([&](auto kk) LCV_INLINE {
                    constexpr int kc = decltype(kk)::value;
                    din[bi][kc] = lds_operand<CT>(V, [&](int j) { return (16 * kc + 4 * g + j) * SV + 16 * b + c; });
                });
            });
            static_for<0, 2>([&](auto rr) LCV_INLINE {
                constexpr int rb = decltype(rr)::value;
                const MatImg<CT> f0 = load_img_lds<CT>(IMS, 2 * rb, lane), f1 = load_img_lds<CT>(IMS, 2 * rb + 1, lane);
                static_for<0, 2>([&](auto bb) LCV_INLINE {
                    constexpr int bi = decltype(bb)::value;
                    const int b = 2 * wave + bi;
                    f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                    stage_keep_acc<CT>(f0, din[bi][0], re, im);
                    stage_keep_acc<CT>(f1, din[bi][1], re, im);
#pragma unroll
                    for (int j = 0; j < 4; ++j) lds_put<CT>(XY, xy_addr(16 * rb + 4 * g + j, b, c), re[j], im[j]);
                });
            });
            return;
        }
        const MatImg<CT> f0 = load_img_lds<CT>(IMS, 0, lane), f1 = load_img_lds<CT>(IMS, 1, lane);
        Operand<CT> din[2];
        static_for<0, 2>([&](auto bb) LCV_INLINE {
            constexpr int bi = decltype(bb)::value;
            const int b = 2 * wave + bi;
            din[bi] = lds_operand<CT>(V, [&](int j) { return (4 * g + j) * SV + 16 * b + c; });
        });
        Tile acc[2][2];
        static_for<0, 2>([&](auto bb) LCV_INLINE {
            constexpr int bi = decltype(bb)::value;
            acc[bi][0] = stage_keep<CT>(f0, din[bi]);
            acc[bi][1] = stage_keep<CT>(f1, din[bi]);
        });
        static_for<0, 2>([&](auto bb) LCV_INLINE {
            constexpr int bi = decltype(bb)::value;
            const int b = 2 * wave + bi;
            static_for<0, 2>([&](auto rr) LCV_INLINE {
                constexpr int rb = decltype(rr)::value;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lds_put<CT>(XY, xy_addr(16 * rb + 4 * g + j, b, c), acc[bi][rb].re[j], acc[bi][rb].im[j]);
            });
        });
    };
    // P2: F2, twiddle, F3, product, I1, twiddle, I2 on this wave's four tiles (registers).
    // Two groups of two tiles, one stage apart; inside a step one product, then a share of
    // the vector work, repeated.
    auto P2 = [&](uint32_t* XY, const uint4* kfl) LCV_INLINE {
        Operand<CT> opd[4];
        Tile xs[4];
        auto ld_op = [&](auto grp) LCV_INLINE {
            constexpr int i0 = 2 * decltype(grp)::value;
            static_for<i0, i0 + 2>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int t = wave * 4 + i;
                opd[i] = lds_operand<CT>(XY, [&](int j) { return xy_addr(t, 4 * g + j, c); });
            });
        };
        auto mstage = [&](auto grp, auto stg) LCV_INLINE {
            constexpr int i0 = 2 * decltype(grp)::value, st = decltype(stg)::value;
            __builtin_amdgcn_s_setprio(1);
            static_for<i0, i0 + 2>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                if constexpr (st == 1) xs[i] = stage_swap<CT>(mf2[i], opd[i]);       // (L = k2, K = n3)
                else if constexpr (st == 2) xs[i] = stage_keep<CT>(mf3[i], opd[i]);  // (L = k2, K = k3)
                else if constexpr (st == 3) xs[i] = stage_swap<CT>(mi1[i], opd[i]);  // (L = n3, K = k2)
                else xs[i] = stage_keep<CT>(mi2[i], opd[i]);                         // (L = n3, K = n2)
            });
            __builtin_amdgcn_s_setprio(0);
        };
        auto vstep = [&](auto grp, auto stg) LCV_INLINE {
            constexpr int i0 = 2 * decltype(grp)::value, st = decltype(stg)::value;
            static_for<i0, i0 + 2>([&](auto ii) LCV_INLINE {
                constexpr int i = decltype(ii)::value;
                const int t = wave * 4 + i;
                if constexpr (st == 1) {
                    cmul4(xs[i], twr, twi);
                    opd[i] = to_operand<CT>(xs[i]);
                } else if constexpr (st == 2) {
                    f32x4 kr, ki;
                    if constexpr (ROW) {
                        unpack_raw_c4v<CT>(&rk[i], kr, ki);
                        kr += rkd;  // (K + D) / M
                    } else {
                        const uint4 kw = kfl[t * 64 + lane];  // (K + D) / M
                        unpack_raw_c4v<CT>(&kw, kr, ki);
                    }
                    if constexpr (ADJ) cmulc4(xs[i], kr, ki);
                    else cmul4(xs[i], kr, ki);
                    opd[i] = to_operand<CT>(xs[i]);
                } else if constexpr (st == 3) {
                    cmulc4(xs[i], twr, twi);
                    opd[i] = to_operand<CT>(xs[i]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) lds_put<CT>(XY, xy_addr(t, 4 * g + j, c), xs[i].re[j], xs[i].im[j]);
                }
            });
        };
        auto interleave = [&](auto nv) LCV_INLINE {
            static_for<0, 4>([&](auto) LCV_INLINE {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, decltype(nv)::value, 0);
            });
        };
        using G0 = std::integral_constant<int, 0>;
        using G1 = std::integral_constant<int, 1>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        using S3 = std::integral_constant<int, 3>;
        using S4 = std::integral_constant<int, 4>;
        ld_op(G0{});
        ld_op(G1{});
        mstage(G0{}, S1{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G1{}, S1{}); vstep(G0{}, S1{}); interleave(std::integral_constant<int, 10>{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G0{}, S2{}); vstep(G1{}, S1{}); interleave(std::integral_constant<int, 10>{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G1{}, S2{}); vstep(G0{}, S2{}); interleave(std::integral_constant<int, 14>{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G0{}, S3{}); vstep(G1{}, S2{}); interleave(std::integral_constant<int, 14>{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G1{}, S3{}); vstep(G0{}, S3{}); interleave(std::integral_constant<int, 10>{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G0{}, S4{}); vstep(G1{}, S3{}); interleave(std::integral_constant<int, 10>{});
        __builtin_amdgcn_sched_barrier(0);
        mstage(G1{}, S4{}); vstep(G0{}, S4{}); interleave(std::integral_constant<int, 4>{});
        __builtin_amdgcn_sched_barrier(0);
        vstep(G1{}, S4{});
    };
    // P3: I3 (inverse radix 32, rows n1 < 16) on this wave's two column blocks, XY -> O (in V)
    auto P3 = [&](const uint32_t* XY) LCV_INLINE {
        constexpr int IB = ROW ? 4 : 2;  // first I3 image in LDS
        const MatImg<CT> i0 = load_img_lds<CT>(IMS, IB, lane), i1 = load_img_lds<CT>(IMS, IB + 1, lane);
        Operand<CT> din[2][2];
        static_for<0, 2>([&](auto bb) LCV_INLINE {
            constexpr int bi = decltype(bb)::value;
            const int b = 2 * wave + bi;
            static_for<0, 2>([&](auto kk) LCV_INLINE {
                constexpr int kc = decltype(kk)::value;
                din[bi][kc] = lds_operand<CT>(XY, [&](int j) { return xy_addr(16 * kc + 4 * g + j, b, c); });
            });
        });
        Tile acc[2];
        static_for<0, 2>([&](auto bb) LCV_INLINE {
            constexpr int bi = decltype(bb)::value;
            acc[bi].re = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[bi].im = f32x4{0.f, 0.f, 0.f, 0.f};
            stage_keep_acc<CT>(i0, din[bi][0], acc[bi].re, acc[bi].im);
            stage_keep_acc<CT>(i1, din[bi][1], acc[bi].re, acc[bi].im);
        });
        static_for<0, 2>([&](auto bb) LCV_INLINE {
            constexpr int bi = decltype(bb)::value;
            const int b = 2 * wave + bi;
#pragma unroll
            for (int j = 0; j < 4; ++j) V[(4 * g + j) * SV + 16 * b + c] = pack2<CT>(acc[bi].re[j], acc[bi].im[j]);
        });
        if constexpr (ROW) {  // rows n1 = 16 .. 31 as well
            const MatImg<CT> i2 = load_img_lds<CT>(IMS, IB + 2, lane), i3 = load_img_lds<CT>(IMS, IB + 3, lane);
            static_for<0, 2>([&](auto bb) LCV_INLINE {
                constexpr int bi = decltype(bb)::value;
                const int b = 2 * wave + bi;
                f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
                stage_keep_acc<CT>(i2, din[bi][0], re, im);
                stage_keep_acc<CT>(i3, din[bi][1], re, im);
#pragma unroll
                for (int j = 0; j < 4; ++j) V[(16 + 4 * g + j) * SV + 16 * b + c] = pack2<CT>(re[j], im[j]);
            });
        }
    };
    // P4: post-gate and store this lane's slot of the item
    auto P4 = [&](int64_t item) LCV_INLINE {
        if constexpr (ROW) {  // back to the workspace row, in place
            uint4* dst = (uint4*)((uint32_t*)a.y + ws_row(item) * M + s_n0);
            const uint4* s0 = (const uint4*)(V + s_n1 * SV + s_col);
            const uint4* s1 = (const uint4*)(V + (s_n1 + 16) * SV + s_col);
            const uint4 w0 = s0[0], w1 = s0[1], w2 = s1[0], w3 = s1[1];
            dst[0] = w0;
            dst[1] = w1;
            dst[16 * 256 / 4] = w2;
            dst[16 * 256 / 4 + 1] = w3;
            return;
        }
        int64_t o0, o1;
        offsets(item, o0, o1);
        const uint4* src = (const uint4*)(V + s_n1 * SV + s_col);
        const uint4 w0 = src[0], w1 = src[1];
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float yr[8], yi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            yr[i] = unpack_lo<CT>(w[i]);
            yi[i] = unpack_hi<CT>(w[i]);
        }
        if constexpr (ADJ && GV) {
            float t[8], zr[8], zi[8];
            unpack_raw<CT>(&re2[0], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) zr[i] = yr[i] * t[i];
            unpack_raw<CT>(&re2[1], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) zi[i] = yi[i] * t[i];
            store8_nt<CT>(a.y2, o0, zr);
            store8_nt<CT>(a.y2, o1, zi);
        }
        if constexpr (SAVE) {   // the pre-gate output c
            store8_nt<CT>(a.y2, o0, yr);
            store8_nt<CT>(a.y2, o1, yi);
        }
        if constexpr (GV) {
            float t[8];
            unpack_raw<CT>(&rv[0], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) yr[i] *= t[i];
            unpack_raw<CT>(&rv[1], t);
#pragma unroll
            for (int i = 0; i < 8; ++i) yi[i] *= t[i];
        }
        store8_nt<CT>(a.y, o0, yr);  // streamed past the caches: nothing here reads y again
        store8_nt<CT>(a.y, o1, yi);
    };

    // ---- pipeline ------------------------------------------------------------------------------
    // Each wave group runs its own copy of the item loop (P2 first for waves 0-3, W first for
    // waves 4-7), with the first and last items peeled off: the steady loop has no branch around
    // a memory instruction but the rare spectrum reload, so the compiler's vmcnt waits count the
    // loads issued one item ahead instead of draining them.
    int64_t kf_h = ROW ? 0 : channel(first);  // (ROW items carry no batch count)
    int kb = 0;
    if constexpr (ROW) issue_kf_row(first);
    else load_kf(kf_h, 0);
    issue_uq(first);
    P0();
    issue_uq(first + 1);
    P1(XYb);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    // W(k): P3, P4 of k - 1; the next channel's spectrum; P0, P1 of k + 1 (guarded: the first
    // and last items; unguarded: first < k < last - 1)
    auto W = [&](int64_t k, uint32_t* XYo, int& kb_next, auto guarded) LCV_INLINE {
        constexpr bool GU = decltype(guarded)::value;
        if (!GU || k > first) {
            issue_e2(k - 1);
            P3(XYo);
            P4(k - 1);
        }
        if (!ROW && (!GU || k + 1 < last)) {
            const int64_t hn = channel(k + 1);
            if (hn != kf_h) {
                kb_next = 1 - kb;
                load_kf(hn, kb_next);
                kf_h = hn;
            }
        }
        issue_v(k);
        if (!GU || k + 1 < last) {
            P0();
            issue_uq(k + 2);
            P1(XYo);
        }
    };
    auto iteration = [&](int64_t k, auto p2_first, auto guarded) LCV_INLINE {
        const int xb = (int)((k - first) & 1);
        uint32_t* const XYk = XYb + xb * XY_W;
        uint32_t* const XYo = XYb + (1 - xb) * XY_W;
        int kb_next = kb;
        if constexpr (decltype(p2_first)::value) {
            P2(XYk, KFL + kb * (KF_W / 4));
            if constexpr (ROW) issue_kf_row(k + 1);  // clamped past the end
            __builtin_amdgcn_sched_barrier(0);
            W(k, XYo, kb_next, guarded);
        } else {
            W(k, XYo, kb_next, guarded);
            __builtin_amdgcn_sched_barrier(0);
            P2(XYk, KFL + kb * (KF_W / 4));
            if constexpr (ROW) issue_kf_row(k + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        kb = kb_next;
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto p2_first) LCV_INLINE {
        iteration(first, p2_first, Yes{});
        int64_t k = first + 1;
        for (; k < last - 1; ++k) iteration(k, p2_first, No{});
        if (k < last) iteration(k, p2_first, Yes{});
    };
    if (wave < 4) run(Yes{});
    else run(No{});
    issue_e2(last - 1);
    P3(XYb + ((last - 1 - first) & 1) * XY_W);
    P4(last - 1);
}

// ------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------

template <int R, int CT, int IO, int MODE, bool GQ, bool GV>
static hipError_t launch_t(const Fused1DArgs& a0, int cus, hipStream_t st) {
    Fused1DArgs a = a0;
    constexpr int P = 32 / R;
    if (a.nitems <= 0) return hipSuccess;
    const int64_t groups = (a.nitems + P - 1) / P;
    int64_t nwg = groups < cus ? groups : cus;
    const int64_t gpw = (groups + nwg - 1) / nwg;
    a.per_wg = gpw * P;
    nwg = (a.nitems + a.per_wg - 1) / a.per_wg;
    hipLaunchKernelGGL((fused1d_kernel<R, CT, IO, MODE, GQ, GV>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    return hipGetLastError();
}

template <int CT, bool GQ, bool GV, bool ADJ, bool SAVE, bool ROW = false>
static hipError_t launch_8k(const Fused1DArgs& a0, int cus, hipStream_t st) {
    Fused1DArgs a = a0;
    if (a.nitems <= 0) return hipSuccess;
    int64_t nwg = a.nitems < cus ? a.nitems : cus;
    a.per_wg = (a.nitems + nwg - 1) / nwg;
    nwg = (a.nitems + a.per_wg - 1) / a.per_wg;
    hipLaunchKernelGGL((conv8k_kernel<CT, GQ, GV, ADJ, SAVE, ROW>), dim3((unsigned)nwg), dim3(512), 0, st, a);
    return hipGetLastError();
}

template <int R, int T, int MODE>
static hipError_t launch_conv(bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t st) {
    constexpr bool ADJ = MODE == MODE_ADJ;
    if constexpr (R == 32 && T != CT_F32) {
        if (a.N == 4096) {  // whole rows: the pipelined kernel (the only one with row strides)
            constexpr bool SAVE = MODE == MODE_SAVE;
            if (gq && gv) return launch_8k<T, true, true, ADJ, SAVE>(a, cus, st);
            if (gq) return launch_8k<T, true, false, ADJ, SAVE>(a, cus, st);
            if (gv) return launch_8k<T, false, true, ADJ, SAVE>(a, cus, st);
            return launch_8k<T, false, false, ADJ, SAVE>(a, cus, st);
        }
    }
    if (a.sb != 0 || a.sh != 0) return hipErrorInvalidValue;
    if (gq && gv) return launch_t<R, T, T, MODE, true, true>(a, cus, st);
    if (gq) return launch_t<R, T, T, MODE, true, false>(a, cus, st);
    if (gv) return launch_t<R, T, T, MODE, false, true>(a, cus, st);
    return launch_t<R, T, T, MODE, false, false>(a, cus, st);
}

template <int R, int T>
static hipError_t launch_sparse(bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t st) {
    if (gq && gv) return launch_t<R, T, T, MODE_SPARSE, true, true>(a, cus, st);
    if (gq) return launch_t<R, T, T, MODE_SPARSE, true, false>(a, cus, st);
    if (gv) return launch_t<R, T, T, MODE_SPARSE, false, true>(a, cus, st);
    return launch_t<R, T, T, MODE_SPARSE, false, false>(a, cus, st);
}

template <int R, int T>
static hipError_t launch_lbf(bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t st) {
    if (gq && gv) return launch_t<R, T, T, MODE_LBF, true, true>(a, cus, st);
    if (gq) return launch_t<R, T, T, MODE_LBF, true, false>(a, cus, st);
    if (gv) return launch_t<R, T, T, MODE_LBF, false, true>(a, cus, st);
    return launch_t<R, T, T, MODE_LBF, false, false>(a, cus, st);
}

template <int R, int T>
static hipError_t launch_part(bool gq, bool gv, const Fused1DArgs& a, int cus, hipStream_t st) {
    if (gq && gv) return launch_t<R, T, T, MODE_PART, true, true>(a, cus, st);
    if (gq) return launch_t<R, T, T, MODE_PART, true, false>(a, cus, st);
    if (gv) return launch_t<R, T, T, MODE_PART, false, true>(a, cus, st);
    return launch_t<R, T, T, MODE_PART, false, false>(a, cus, st);
}

// Calls f(std::integral_constant<int, R>) for the supported R.
template <typename F>
static hipError_t for_r(int R, F&& f) {
    switch (R) {
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    default: return hipErrorInvalidValue;
    }
}

}  // namespace lcv
