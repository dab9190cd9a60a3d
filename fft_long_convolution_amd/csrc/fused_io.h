// fused_io.h -- device-side load / store / LDS helpers shared by the fused 1D kernels
// (element I/O in fp32, fp16 or bf16; complex spectra; compute-type LDS elements).
#pragma once
#include "lconv_device.h"

namespace lcv {

namespace {

template <int IO>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
    if constexpr (IO == CT_F32) {
        return ((const float*)base)[i];
    } else {
        uint32_t w = ((const uint16_t*)base)[i];
        return unpack_lo<IO>(w);
    }
}

template <int IO>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* x) {
    if constexpr (IO == CT_F32) {
        const float4* p = (const float4*)((const float*)base + off);
        float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        uint4 w = *(const uint4*)((const uint16_t*)base + off);
        x[0] = unpack_lo<IO>(w.x); x[1] = unpack_hi<IO>(w.x);
        x[2] = unpack_lo<IO>(w.y); x[3] = unpack_hi<IO>(w.y);
        x[4] = unpack_lo<IO>(w.z); x[5] = unpack_hi<IO>(w.z);
        x[6] = unpack_lo<IO>(w.w); x[7] = unpack_hi<IO>(w.w);
    }
}

template <int IO>
__device__ __forceinline__ void store8(void* base, int64_t off, const float* x) {
    if constexpr (IO == CT_F32) {
        float4* p = (float4*)((float*)base + off);
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else {
        uint4 w;
        w.x = pack2<IO>(x[0], x[1]);
        w.y = pack2<IO>(x[2], x[3]);
        w.z = pack2<IO>(x[4], x[5]);
        w.w = pack2<IO>(x[6], x[7]);
        *(uint4*)((uint16_t*)base + off) = w;
    }
}

// 8 consecutive elements as raw bits (1 uint4 for 16-bit types, 2 for fp32) and their unpacking.
// store8 with the non-temporal hint: a streamed output that nothing in the call reads again
template <int IO>
__device__ __forceinline__ void store8_nt(void* base, int64_t off, const float* x) {
    if constexpr (IO == CT_F32) {
        uint32_t* p = (uint32_t*)((float*)base + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(__float_as_uint(x[i]), p + i);
    } else {
        uint32_t* p = (uint32_t*)((uint16_t*)base + off);
        __builtin_nontemporal_store(pack2<IO>(x[0], x[1]), p);
        __builtin_nontemporal_store(pack2<IO>(x[2], x[3]), p + 1);
        __builtin_nontemporal_store(pack2<IO>(x[4], x[5]), p + 2);
        __builtin_nontemporal_store(pack2<IO>(x[6], x[7]), p + 3);
    }
}

template <int IO>
__device__ __forceinline__ void load_raw(const void* base, int64_t off, uint4* r) {
    if constexpr (IO == CT_F32) {
        const uint4* p = (const uint4*)((const float*)base + off);
        r[0] = p[0];
        r[1] = p[1];
    } else {
        r[0] = *(const uint4*)((const uint16_t*)base + off);
    }
}
template <int IO>
__device__ __forceinline__ void unpack_raw(const uint4* r, float* x) {
    if constexpr (IO == CT_F32) {
        x[0] = __uint_as_float(r[0].x); x[1] = __uint_as_float(r[0].y);
        x[2] = __uint_as_float(r[0].z); x[3] = __uint_as_float(r[0].w);
        x[4] = __uint_as_float(r[1].x); x[5] = __uint_as_float(r[1].y);
        x[6] = __uint_as_float(r[1].z); x[7] = __uint_as_float(r[1].w);
    } else {
        x[0] = unpack_lo<IO>(r[0].x); x[1] = unpack_hi<IO>(r[0].x);
        x[2] = unpack_lo<IO>(r[0].y); x[3] = unpack_hi<IO>(r[0].y);
        x[4] = unpack_lo<IO>(r[0].z); x[5] = unpack_hi<IO>(r[0].z);
        x[6] = unpack_lo<IO>(r[0].w); x[7] = unpack_hi<IO>(r[0].w);
    }
}
// 4 consecutive complex values (raw bits) of a spectrum stored in type IO.
template <int IO>
__device__ __forceinline__ void load_raw_c4(const void* base, int64_t off, uint4* r) {
    if constexpr (IO == CT_F32) {
        const uint4* p = (const uint4*)((const float*)base + 2 * off);
        r[0] = p[0];
        r[1] = p[1];
    } else {
        r[0] = *(const uint4*)((const uint32_t*)base + off);
    }
}
template <int IO>
__device__ __forceinline__ void unpack_raw_c4(const uint4* r, float* re, float* im) {
    if constexpr (IO == CT_F32) {
        re[0] = __uint_as_float(r[0].x); im[0] = __uint_as_float(r[0].y);
        re[1] = __uint_as_float(r[0].z); im[1] = __uint_as_float(r[0].w);
        re[2] = __uint_as_float(r[1].x); im[2] = __uint_as_float(r[1].y);
        re[3] = __uint_as_float(r[1].z); im[3] = __uint_as_float(r[1].w);
    } else {
        re[0] = unpack_lo<IO>(r[0].x); im[0] = unpack_hi<IO>(r[0].x);
        re[1] = unpack_lo<IO>(r[0].y); im[1] = unpack_hi<IO>(r[0].y);
        re[2] = unpack_lo<IO>(r[0].z); im[2] = unpack_hi<IO>(r[0].z);
        re[3] = unpack_lo<IO>(r[0].w); im[3] = unpack_hi<IO>(r[0].w);
    }
}

template <int IO>
__device__ __forceinline__ void unpack_raw_c4v(const uint4* r, f32x4& re, f32x4& im) {
    float a[4], b[4];
    unpack_raw_c4<IO>(r, a, b);
    re = f32x4{a[0], a[1], a[2], a[3]};
    im = f32x4{b[0], b[1], b[2], b[3]};
}

// 4 consecutive complex values of a spectrum stored in type IO -> fp32.
template <int IO>
__device__ __forceinline__ void load_c4(const void* base, int64_t off, float* re, float* im) {
    if constexpr (IO == CT_F32) {
        const float4* p = (const float4*)((const float*)base + 2 * off);
        float4 a = p[0], b = p[1];
        re[0] = a.x; im[0] = a.y; re[1] = a.z; im[1] = a.w;
        re[2] = b.x; im[2] = b.y; re[3] = b.z; im[3] = b.w;
    } else {
        uint4 w = *(const uint4*)((const uint32_t*)base + off);
        re[0] = unpack_lo<IO>(w.x); im[0] = unpack_hi<IO>(w.x);
        re[1] = unpack_lo<IO>(w.y); im[1] = unpack_hi<IO>(w.y);
        re[2] = unpack_lo<IO>(w.z); im[2] = unpack_hi<IO>(w.z);
        re[3] = unpack_lo<IO>(w.w); im[3] = unpack_hi<IO>(w.w);
    }
}

template <int IO>
__device__ __forceinline__ void store_c4v(void* base, int64_t off, const f32x4 re, const f32x4 im) {
    if constexpr (IO == CT_F32) {
        float4* p = (float4*)((float*)base + 2 * off);
        p[0] = make_float4(re[0], im[0], re[1], im[1]);
        p[1] = make_float4(re[2], im[2], re[3], im[3]);
    } else {
        uint4 w;
        w.x = pack2<IO>(re[0], im[0]);
        w.y = pack2<IO>(re[1], im[1]);
        w.z = pack2<IO>(re[2], im[2]);
        w.w = pack2<IO>(re[3], im[3]);
        *(uint4*)((uint32_t*)base + off) = w;
    }
}

// LDS complex element in compute type: one packed word (16-bit) or two floats.
template <int CT>
__device__ __forceinline__ void lds_put(uint32_t* base, int idx, float re, float im) {
    if constexpr (CT == CT_F32) {
        *(float2*)(base + 2 * idx) = make_float2(re, im);
    } else {
        base[idx] = pack2<CT>(re, im);
    }
}

// Read a tile operand: element (K index 4g + j, L index c) at base + idx(j).
template <int CT, typename F>
__device__ __forceinline__ Operand<CT> lds_operand(const uint32_t* base, F idx) {
    Operand<CT> o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = idx(j);
        if constexpr (CT == CT_F32) {
            float2 v = e >= 0 ? *(const float2*)(base + 2 * e) : make_float2(0.f, 0.f);
            o.s[2 * j] = v.x;
            o.s[2 * j + 1] = v.y;
        } else {
            o.w[j] = e >= 0 ? base[e] : 0u;
        }
    }
    return o;
}

}  // namespace


// D[h] as raw bits (converted where it is used, so the load's latency is not waited for early)
template <int IO>
__device__ __forceinline__ uint32_t load1_raw(const void* base, int64_t i) {
    if constexpr (IO == CT_F32) return ((const uint32_t*)base)[i];
    else return ((const uint16_t*)base)[i];
}
template <int IO>
__device__ __forceinline__ float raw1_to_f32(uint32_t w) {
    if constexpr (IO == CT_F32) return __uint_as_float(w);
    else return unpack_lo<IO>(w);
}

}  // namespace lcv
