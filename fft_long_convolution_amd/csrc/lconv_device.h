// lconv_device.h -- gfx950 device building blocks for the factored FFT convolution.
//
// A length-16 complex DFT (or a twiddle-folded variant of it) is applied to 16 columns at once
// as a real matrix product on the matrix cores: with z = zr + i zi and a complex 16x16
// matrix G,  Re(G z) = Gr zr - Gi zi  and  Im(G z) = Gi zr + Gr zi.  Stacking (zr, zi) along
// the contraction axis (K = 32 reals) gives two v_mfma_f32_16x16x32_{bf16,f16} per 16 columns
// (one for the real rows, one for the imaginary rows), or 2 x 8 v_mfma_f32_16x16x4_f32 for
// fp32 operands.  This is the "FFT as matrix multiplications on matrix units" idea of the
// FlashFFTConv abstract and the FlashConv page (Mechanism), laid out for 64-wide waves.
//
// Register layout of one 16 x 16 complex TILE (the unit every stage works on):
//   lane l = 16 g + x  (g = l / 16 in 0..3, x = l % 16)
//   the lane holds 4 complex values: "L index" x, "K index" 4 g + j for j = 0..3.
// As an MFMA operand a tile supplies 8 K-slots per lane: slot 2j is Re, slot 2j+1 is Im of
// K index 4g+j.  Whatever physical K order the hardware uses, A and B slots pair up the same
// way, so the product sums exactly over (K index, re/im).
// A 16x16 MFMA output puts row 4g+j, column x into lane 16g+x, register j.  Hence:
//   * data as B operand (matrix as A): output rows = G's output index -> K position,
//     the data's L index stays in L                            ("keep")
//   * data as A operand (matrix as B): the data's L index moves to the K position, the
//     output index of G lands in L                              ("swap")
// and the output of one stage is directly the operand of the next: no lane movement.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.h"

// Kernel-local lambdas must inline: an out-of-line call would move the register arrays they
// capture into memory (which the compiler then places in LDS).
#define LCV_INLINE __attribute__((always_inline))

namespace lcv {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

// ---- scalar conversions ------------------------------------------------------------------

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// (lo, hi) -> packed 2 x 16-bit, round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32)
template <int CT> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
// One packed convert.  (Inline asm is not an option here: the compiler does not track the
// matrix-core result hazard for an asm instruction that reads those registers.)
template <> __device__ __forceinline__ uint32_t pack2<CT_BF16>(float lo, float hi) {
    f32x2 t = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<CT_F16>(float lo, float hi) {
    f32x2 t = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(t, f16x2));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).  Arrays indexed by
// these constants are split into registers from the start; a #pragma-unrolled loop index is
// still a variable when the optimiser first sees the arrays, which can leave them in memory.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
template <int CT> __device__ __forceinline__ float unpack_lo(uint32_t w) {
    return CT == CT_BF16 ? bf16lo_to_f32(w) : f16lo_to_f32(w);
}
template <int CT> __device__ __forceinline__ float unpack_hi(uint32_t w) {
    return CT == CT_BF16 ? bf16hi_to_f32(w) : f16hi_to_f32(w);
}

// 16 bytes stored with the non-temporal hint (one streamed vector store)
__device__ __forceinline__ void st4_nt(uint32_t* p, uint4 v) {
    __builtin_nontemporal_store(v.x, p);
    __builtin_nontemporal_store(v.y, p + 1);
    __builtin_nontemporal_store(v.z, p + 2);
    __builtin_nontemporal_store(v.w, p + 3);
}

// ---- tiles and operands ------------------------------------------------------------------

// fp32 tile: 4 complex values per lane (the MFMA accumulators of the re and im products).
// Kept as two 4-vectors, never as float arrays: element updates then stay register values
// instead of memory the optimiser may leave in place.
struct Tile {
    f32x4 re, im;
};

// Operand image of a tile (or of a matrix): 8 K-slots per lane.
template <int CT> struct Operand;
template <> struct Operand<CT_F32> {
    float s[8];
};
template <> struct Operand<CT_F16> {
    uint32_t w[4];  // w[j] = (Re, Im) of K index 4g+j, packed fp16
};
template <> struct Operand<CT_BF16> {
    uint32_t w[4];  // packed bf16
};

// A complex matrix image: the operand feeding the real-output product and the one feeding
// the imaginary-output product.
template <int CT> struct MatImg {
    Operand<CT> re, im;
};

template <int CT> __device__ __forceinline__ Operand<CT> to_operand(const Tile& t) {
    Operand<CT> o;
    if constexpr (CT == CT_F32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { o.s[2 * j] = t.re[j]; o.s[2 * j + 1] = t.im[j]; }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) o.w[j] = pack2<CT>(t.re[j], t.im[j]);
    }
    return o;
}

template <int CT> __device__ __forceinline__ Tile from_operand(const Operand<CT>& o) {
    Tile t;
    if constexpr (CT == CT_F32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { t.re[j] = o.s[2 * j]; t.im[j] = o.s[2 * j + 1]; }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) { t.re[j] = unpack_lo<CT>(o.w[j]); t.im[j] = unpack_hi<CT>(o.w[j]); }
    }
    return t;
}

template <int CT> __device__ __forceinline__ Operand<CT> zero_operand() {
    Operand<CT> o;
    if constexpr (CT == CT_F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o.s[i] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o.w[i] = 0u;
    }
    return o;
}

// acc += A x B for one K-chunk of 32 reals (16 complex).
template <int CT>
__device__ __forceinline__ f32x4 mma(const Operand<CT>& a, const Operand<CT>& b, f32x4 acc) {
    if constexpr (CT == CT_BF16) {
        u32x4 av = {a.w[0], a.w[1], a.w[2], a.w[3]};
        u32x4 bv = {b.w[0], b.w[1], b.w[2], b.w[3]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    } else if constexpr (CT == CT_F16) {
        u32x4 av = {a.w[0], a.w[1], a.w[2], a.w[3]};
        u32x4 bv = {b.w[0], b.w[1], b.w[2], b.w[3]};
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                      __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.s[i], b.s[i], acc, 0, 0, 0);
        return acc;
    }
}

// Complex stage, data as B (matrix as A): output index -> K position, L kept.
template <int CT>
__device__ __forceinline__ void stage_keep_acc(const MatImg<CT>& m, const Operand<CT>& d, f32x4& re,
                                               f32x4& im) {
    re = mma<CT>(m.re, d, re);
    im = mma<CT>(m.im, d, im);
}
// Complex stage, data as A (matrix as B): the data's L index -> K position, output -> L.
template <int CT>
__device__ __forceinline__ void stage_swap_acc(const MatImg<CT>& m, const Operand<CT>& d, f32x4& re,
                                               f32x4& im) {
    re = mma<CT>(d, m.re, re);
    im = mma<CT>(d, m.im, im);
}

__device__ __forceinline__ Tile tile_from_acc(const f32x4& re, const f32x4& im) { return Tile{re, im}; }

template <int CT>
__device__ __forceinline__ Tile stage_keep(const MatImg<CT>& m, const Operand<CT>& d) {
    f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
    stage_keep_acc<CT>(m, d, re, im);
    return tile_from_acc(re, im);
}
template <int CT>
__device__ __forceinline__ Tile stage_swap(const MatImg<CT>& m, const Operand<CT>& d) {
    f32x4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
    stage_swap_acc<CT>(m, d, re, im);
    return tile_from_acc(re, im);
}

// (a + ib) *= (c + id)
__device__ __forceinline__ void cmul(float& a, float& b, float c, float d) {
    float r = a * c - b * d;
    float i = a * d + b * c;
    a = r;
    b = i;
}
// (a + ib) *= conj(c + id)
__device__ __forceinline__ void cmulc(float& a, float& b, float c, float d) {
    float r = a * c + b * d;
    float i = b * c - a * d;
    a = r;
    b = i;
}
// Tile-wide complex products: x *= (c + id), x *= conj(c + id), elementwise over the 4 values.
__device__ __forceinline__ void cmul4(Tile& x, const f32x4 c, const f32x4 d) {
    const f32x4 r = x.re * c - x.im * d;
    const f32x4 i = x.re * d + x.im * c;
    x.re = r;
    x.im = i;
}
__device__ __forceinline__ void cmulc4(Tile& x, const f32x4 c, const f32x4 d) {
    const f32x4 r = x.re * c + x.im * d;
    const f32x4 i = x.im * c - x.re * d;
    x.re = r;
    x.im = i;
}

// ---- matrix images in global memory --------------------------------------------------------
// One image = 64 lanes x (8 re-slots + 8 im-slots) of the compute type, lane-major.
template <int CT> struct ImgBytes {
    static constexpr int value = (CT == CT_F32 ? 4 : 2) * 16 * 64;
};

template <int CT>
__device__ __forceinline__ MatImg<CT> load_img(const void* base, int idx, int lane) {
    MatImg<CT> m;
    if constexpr (CT == CT_F32) {
        const float4* p = (const float4*)((const char*)base + (size_t)idx * ImgBytes<CT>::value) + lane * 4;
        float4 a = p[0], b = p[1], c = p[2], d = p[3];
        m.re.s[0] = a.x; m.re.s[1] = a.y; m.re.s[2] = a.z; m.re.s[3] = a.w;
        m.re.s[4] = b.x; m.re.s[5] = b.y; m.re.s[6] = b.z; m.re.s[7] = b.w;
        m.im.s[0] = c.x; m.im.s[1] = c.y; m.im.s[2] = c.z; m.im.s[3] = c.w;
        m.im.s[4] = d.x; m.im.s[5] = d.y; m.im.s[6] = d.z; m.im.s[7] = d.w;
    } else {
        const uint4* p = (const uint4*)((const char*)base + (size_t)idx * ImgBytes<CT>::value) + lane * 2;
        uint4 a = p[0], b = p[1];
        m.re.w[0] = a.x; m.re.w[1] = a.y; m.re.w[2] = a.z; m.re.w[3] = a.w;
        m.im.w[0] = b.x; m.im.w[1] = b.y; m.im.w[2] = b.z; m.im.w[3] = b.w;
    }
    return m;
}

// The same image layout, read from LDS (16-bit compute types only).
template <int CT>
__device__ __forceinline__ MatImg<CT> load_img_lds(const uint32_t* base, int idx, int lane) {
    static_assert(CT != CT_F32, "LDS images are used for 16-bit operands");
    MatImg<CT> m;
    const uint4* p = (const uint4*)(base + idx * (ImgBytes<CT>::value / 4)) + lane * 2;
    uint4 a = p[0], b = p[1];
    m.re.w[0] = a.x; m.re.w[1] = a.y; m.re.w[2] = a.z; m.re.w[3] = a.w;
    m.im.w[0] = b.x; m.im.w[1] = b.y; m.im.w[2] = b.z; m.im.w[3] = b.w;
    return m;
}

}  // namespace lcv
