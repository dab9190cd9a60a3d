// coldft.h -- batched complex DFTs of power-of-two length on fp32 columns in LDS, and the 8-wide
// global I/O helpers the column passes use (io elements and compute-type complex workspace).
// Self-sorting radix-8/4/2 passes (Stockham order: natural order out, no bit reversal); each
// thread does whole small DFTs in registers.
#pragma once
#include <type_traits>

#include "lconv_device.h"

namespace lcv {

namespace {

__device__ __forceinline__ float2 cmulf(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cmulcf(float2 a, float2 b) {  // a * conj(b)
    return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}

// exp(-2 pi i r / M) from the two-level table (r reduced mod M by the caller)
__device__ __forceinline__ float2 tw_m(const float* lo, const float* hi, int64_t r) {
    float2 a = ((const float2*)lo)[r & 2047];
    float2 b = ((const float2*)hi)[r >> 11];
    return cmulf(a, b);
}

// (sequence -> rows) of a column pass's sequence gs: the pair of batch rows (b, b+1) of one
// channel (row1 = -1 past the last row), or one filter channel
template <typename A>
__device__ __forceinline__ void seq_rows(const A& a, int64_t gs, int64_t& row0, int64_t& row1) {
    if (a.filter) {
        row0 = gs * a.N;
        row1 = -1;
    } else {
        const int64_t h = gs / a.seq_per_h, b = 2 * (gs % a.seq_per_h);
        row0 = (b * a.H + h) * a.N;
        row1 = b + 1 < a.B ? row0 + a.H * a.N : -1;
    }
}

// In-register DFT of length RAD (1, 2, 4 or 8); sign -1 forward, +1 inverse.
template <int RAD, bool INV>
__device__ __forceinline__ void dft_small(float2* v) {
    auto bfly = [](float2& a, float2& b) LCV_INLINE {
        const float2 t = b;
        b = make_float2(a.x - t.x, a.y - t.y);
        a = make_float2(a.x + t.x, a.y + t.y);
    };
    // multiply by -i (forward) or +i (inverse)
    auto rot = [](float2 a) LCV_INLINE { return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x); };
    if constexpr (RAD == 1) {
    } else if constexpr (RAD == 2) {
        bfly(v[0], v[1]);
    } else if constexpr (RAD == 4) {
        bfly(v[0], v[2]);
        bfly(v[1], v[3]);
        v[3] = rot(v[3]);
        bfly(v[0], v[1]);
        bfly(v[2], v[3]);
        const float2 t = v[1];  // outputs in order 0, 2, 1, 3 -> natural
        v[1] = v[2];
        v[2] = t;
    } else {
        // radix 8 = decimation in frequency: 4 butterflies (stride 4), twiddles w8^k, then two
        // radix-4 DFTs on the even and odd halves
        const float h = 0.70710678118654752f;
        bfly(v[0], v[4]);
        bfly(v[1], v[5]);
        bfly(v[2], v[6]);
        bfly(v[3], v[7]);
        // v[4..7] *= w8^{0,1,2,3}  (w8 = exp(-+ 2 pi i / 8))
        v[5] = INV ? make_float2(h * (v[5].x - v[5].y), h * (v[5].x + v[5].y))
                   : make_float2(h * (v[5].x + v[5].y), h * (v[5].y - v[5].x));
        v[6] = rot(v[6]);
        v[7] = INV ? make_float2(-h * (v[7].x + v[7].y), h * (v[7].x - v[7].y))
                   : make_float2(h * (v[7].y - v[7].x), -h * (v[7].x + v[7].y));
        float2 e[4] = {v[0], v[1], v[2], v[3]}, o[4] = {v[4], v[5], v[6], v[7]};
        dft_small<4, INV>(e);
        dft_small<4, INV>(o);
        // DIF: outputs 2k from the first half, 2k+1 from the second
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = e[k];
            v[2 * k + 1] = o[k];
        }
    }
}

// One self-sorting pass of radix RAD over the columns of buf (column-major, column stride ld) that
// belong to this wave: columns wave + nw * i, the same set in every pass, so no column moves
// between waves and no barrier is needed between passes.  Sub-transform length before the
// pass: ns.  FIRST: the second half of the input is zero.  A column's L / RAD butterfly groups
// are spread over the lanes: several of the wave's columns per round when there are fewer
// groups than lanes, or ROUNDS = groups / 64 groups per lane when there are more.  The pass is
// in place: all of a column's LDS reads (every round) precede its writes in the wave's own
// instruction order, and columns do not interact.  Not inlined: each (radix, rounds) variant
// keeps its own register budget instead of raising the calling kernel's to the largest one.
template <int RAD, bool INV, bool FIRST, int ROUNDS>
__device__ __attribute__((noinline)) void stockham_pass_wave(float2* buf, int L, int ld, int CB, int ns,
                                                   const float* tw_col, int m1, int wave, int nw, int lane) {
    const int groups = L / RAD;
    const int cpr = groups >= 64 ? 1 : 64 / groups;  // this wave's columns per round
    const int sub = groups >= 64 ? 0 : lane / groups;
    const int tmul = m1 / (ns * RAD);
    for (int idx = sub; wave + nw * idx < CB; idx += cpr) {
        const int c = wave + nw * idx;
        float2 v[ROUNDS][RAD];
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const int j = groups >= 64 ? lane + 64 * r : lane % groups;
            const int tstep = tmul * (j % ns);
#pragma unroll
            for (int q = 0; q < RAD; ++q) {
                float2 x = make_float2(0.f, 0.f);
                if (!FIRST || q < RAD / 2) x = buf[c * ld + j + q * groups];
                if (q > 0 && ns > 1) {
                    const float2 w = ((const float2*)tw_col)[(tstep * q) & (m1 - 1)];
                    x = INV ? cmulcf(x, w) : cmulf(x, w);
                }
                v[r][q] = x;
            }
        }
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) dft_small<RAD, INV>(v[r]);
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const int j = groups >= 64 ? lane + 64 * r : lane % groups;
            const int k = j % ns, b0 = (j / ns) * ns * RAD + k;
#pragma unroll
            for (int q = 0; q < RAD; ++q) buf[c * ld + b0 + q * ns] = v[r][q];
        }
    }
}

// Full column DFT of length L = M1 (power of two, 32..1024) over the CB columns of buf; each
// wave transforms its own columns.  Callers bracket it with block barriers.
template <int kThreads, bool INV>
__device__ void column_dft(float2* buf, int L, int ld, int CB, const float* tw_col, int m1) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kThreads / 64;
    int ns = 1;
    bool first = !INV;  // forward: the input's second half is zero
    // one pass of radix RAD, with the rounds its group count needs (L <= 1024)
    auto pass = [&](auto rad) {
        constexpr int RAD = decltype(rad)::value;
        const int rounds = L / RAD <= 64 ? 1 : L / RAD / 64;
        auto go = [&](auto rr) {
            constexpr int RR = decltype(rr)::value;
            if (first) stockham_pass_wave<RAD, INV, true, RR>(buf, L, ld, CB, ns, tw_col, m1, wave, nw, lane);
            else stockham_pass_wave<RAD, INV, false, RR>(buf, L, ld, CB, ns, tw_col, m1, wave, nw, lane);
        };
        constexpr int MAXR = 1024 / RAD / 64;  // rounds a length of at most 1024 can need
        if (rounds == 1 || MAXR < 2) go(std::integral_constant<int, 1>{});
        else if (rounds == 2 || MAXR < 4) go(std::integral_constant<int, (MAXR < 2 ? 1 : 2)>{});
        else if (rounds == 4 || MAXR < 8) go(std::integral_constant<int, (MAXR < 4 ? 1 : 4)>{});
        else go(std::integral_constant<int, (MAXR < 8 ? 1 : 8)>{});
        ns *= RAD;
        first = false;
    };
    while (ns < L) {
        const int rem = L / ns;
        if (rem >= 8) pass(std::integral_constant<int, 8>{});
        else if (rem == 4) pass(std::integral_constant<int, 4>{});
        else pass(std::integral_constant<int, 2>{});
    }
    __syncthreads();
}

// 8 consecutive io elements -> fp32 (raw 16-byte words for 16-bit types, 32 bytes for fp32)
template <int IO>
__device__ __forceinline__ void ld8(const void* p, int64_t i, float* x) {
    if constexpr (IO == CT_F32) {
        const float4 a = ((const float4*)((const float*)p + i))[0], b = ((const float4*)((const float*)p + i))[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        const uint4 w = *(const uint4*)((const uint16_t*)p + i);
        x[0] = unpack_lo<IO>(w.x); x[1] = unpack_hi<IO>(w.x); x[2] = unpack_lo<IO>(w.y); x[3] = unpack_hi<IO>(w.y);
        x[4] = unpack_lo<IO>(w.z); x[5] = unpack_hi<IO>(w.z); x[6] = unpack_lo<IO>(w.w); x[7] = unpack_hi<IO>(w.w);
    }
}
template <int IO>
__device__ __forceinline__ void st8(void* p, int64_t i, const float* x) {
    if constexpr (IO == CT_F32) {
        ((float4*)((float*)p + i))[0] = make_float4(x[0], x[1], x[2], x[3]);
        ((float4*)((float*)p + i))[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else {
        uint4 w;
        w.x = pack2<IO>(x[0], x[1]); w.y = pack2<IO>(x[2], x[3]);
        w.z = pack2<IO>(x[4], x[5]); w.w = pack2<IO>(x[6], x[7]);
        *(uint4*)((uint16_t*)p + i) = w;
    }
}
// 8 consecutive workspace complex values (type CT) <-> fp32
template <int CT>
__device__ __forceinline__ void ws_ld8(const void* p, int64_t i, float2* z) {
    if constexpr (CT == CT_F32) {
        const float4* s = (const float4*)((const float2*)p + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 a = s[k];
            z[2 * k] = make_float2(a.x, a.y);
            z[2 * k + 1] = make_float2(a.z, a.w);
        }
    } else {
        const uint4* s = (const uint4*)((const uint32_t*)p + i);
        const uint4 a = s[0], b = s[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) z[k] = make_float2(unpack_lo<CT>(w[k]), unpack_hi<CT>(w[k]));
    }
}
template <int CT>
__device__ __forceinline__ void ws_st8(void* p, int64_t i, const float2* z) {
    if constexpr (CT == CT_F32) {
        float4* d = (float4*)((float2*)p + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) d[k] = make_float4(z[2 * k].x, z[2 * k].y, z[2 * k + 1].x, z[2 * k + 1].y);
    } else {
        uint4 a, b;
        a.x = pack2<CT>(z[0].x, z[0].y); a.y = pack2<CT>(z[1].x, z[1].y);
        a.z = pack2<CT>(z[2].x, z[2].y); a.w = pack2<CT>(z[3].x, z[3].y);
        b.x = pack2<CT>(z[4].x, z[4].y); b.y = pack2<CT>(z[5].x, z[5].y);
        b.z = pack2<CT>(z[6].x, z[6].y); b.w = pack2<CT>(z[7].x, z[7].y);
        uint4* d = (uint4*)((uint32_t*)p + i);
        d[0] = a;
        d[1] = b;
    }
}

}  // namespace

}  // namespace lcv
