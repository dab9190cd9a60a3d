// plan.cpp -- factorisation plans and the constant tables (DFT-block images, twiddles).
//
// Every table entry is exp(-2 pi i e / P) for an integer exponent e that is reduced modulo P
// in integer arithmetic before the angle is formed, evaluated in double precision and then
// rounded once to the operand type (bf16 / fp16 / fp32).  The pages ask for the FFT to be
// factored into small dense DFT blocks that run on matrix units ("FlashFFTConv" abstract;
// "FlashConv" page, Mechanism), accepting that the block form does more arithmetic than a
// radix-2 FFT (FlashConv page, Limitations); the block sizes here are the gfx950 MFMA shapes.
#include "plan.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>


namespace lcv {

bool force_multipass() {
    static const bool f = [] {
        const char* e = std::getenv("LCONV_FORCE_PATH");
        return e && std::strcmp(e, "multipass") == 0;
    }();
    return f;
}

bool log_enabled() {
    static const bool f = [] {
        const char* e = std::getenv("LCONV_LOG");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return f;
}

bool make_plan_1d(int64_t N, Plan1D* p) {
    if (N < 1 || N > ((int64_t)1 << 22)) return false;
    int64_t M = 512;
    while (M < 2 * N) M *= 2;
    // testing switch: every length on the multi-pass path, with at least two columns (any
    // M >= 2N gives the same linear convolution)
    if (force_multipass() && M < 2 * kRowLen) M = 2 * kRowLen;
    p->N = N;
    p->M = M;
    if (M <= 256 * kMaxFusedR) {
        p->R = (int)(M / 256);
        p->M1 = 1;
        p->multipass = false;
    } else {
        p->R = kMaxFusedR;
        p->M1 = M / kRowLen;
        p->multipass = true;
    }
    return true;
}

namespace {

struct cplx {
    double re, im;
};

// exp(-2 pi i e / P) with e reduced exactly.
cplx omega(int64_t e, int64_t P) {
    int64_t r = e % P;
    if (r < 0) r += P;
    // use the symmetric range for a smaller argument
    long double ang = -2.0L * 3.14159265358979323846264338327950288L * (long double)r / (long double)P;
    return {(double)cosl(ang), (double)sinl(ang)};
}

uint16_t to_bf16(double x) {
    // round to 8 significant bits (ties to even) in double, then take the top half of the float
    if (x == 0.0) return std::signbit(x) ? 0x8000 : 0;
    int e;
    double m = std::frexp(x, &e);
    double r = std::ldexp(std::nearbyint(m * 256.0), e - 8);
    float f = (float)r;
    uint32_t bits;
    std::memcpy(&bits, &f, 4);
    uint32_t lsb = (bits >> 16) & 1u;
    bits += 0x7fffu + lsb;
    return (uint16_t)(bits >> 16);
}

uint16_t to_f16(double x) {
    // single rounding: round to 11 significant bits in double (|x| <= 1 here, so the result
    // is a normal or exactly representable half), then convert exactly
    _Float16 h = (_Float16)0.0f;
    if (x != 0.0) {
        int e;
        double m = std::frexp(x, &e);
        h = (_Float16)std::ldexp(std::nearbyint(m * 2048.0), e - 11);
    } else {
        h = (_Float16)x;
    }
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

// Append the lane image of complex matrix G (G(x, ci): x = output index = lane % 16,
// ci = contracted complex index) to `out`, in compute type ct.
template <typename F>
void append_image(std::vector<uint8_t>& out, int ct, F G) {
    const size_t esz = ct == CT_F32 ? 4 : 2;
    size_t base = out.size();
    out.resize(base + 64 * 16 * esz);
    for (int lane = 0; lane < 64; ++lane) {
        int g = lane / 16, x = lane % 16;
        double slots[16];
        for (int s = 0; s < 8; ++s) {
            int ci = 4 * g + s / 2, part = s % 2;
            cplx v = G(x, ci);
            slots[s] = part == 0 ? v.re : -v.im;      // real-output rows: [Gr, -Gi]
            slots[8 + s] = part == 0 ? v.im : v.re;   // imag-output rows: [Gi,  Gr]
        }
        uint8_t* dst = out.data() + base + (size_t)lane * 16 * esz;
        for (int s = 0; s < 16; ++s) {
            if (ct == CT_F32) {
                float f = (float)slots[s];
                std::memcpy(dst + 4 * s, &f, 4);
            } else {
                uint16_t b = ct == CT_BF16 ? to_bf16(slots[s]) : to_f16(slots[s]);
                std::memcpy(dst + 2 * s, &b, 2);
            }
        }
    }
}

std::vector<uint8_t> build_fused_tables(int R, int ct) {
    FusedTableLayout L = fused_table_layout(R, ct);
    const int64_t M = 256 * (int64_t)R;
    std::vector<uint8_t> t;
    t.reserve(L.total);
    // F1: contract n1 -> k1 (radix R), image (rb, kc): rows k1 = 16 rb + x, inputs n1 = 16 kc + ci
    for (int rb = 0; rb < L.rb1; ++rb)
        for (int kc = 0; kc < L.kc1; ++kc)
            append_image(t, ct, [&](int x, int ci) {
                int k1 = 16 * rb + x, n1 = 16 * kc + ci;
                if (k1 >= R || n1 >= R) return cplx{0, 0};
                return omega((int64_t)k1 * n1, R);
            });
    // I3: contract k1 -> n1 (inverse radix R), rows n1 = 16 rb + x, inputs k1 = 16 kc + ci
    for (int rb = 0; rb < L.rb3; ++rb)
        for (int kc = 0; kc < L.kc3; ++kc)
            append_image(t, ct, [&](int x, int ci) {
                int n1 = 16 * rb + x, k1 = 16 * kc + ci;
                if (k1 >= R || n1 >= R) return cplx{0, 0};
                return omega(-(int64_t)k1 * n1, R);
            });
    // F2[k1]: G(k2, n2) = w16^(n2 k2) * w_{16R}^(n2 k1) = w_{16R}^(n2 (k1 + R k2))
    for (int k1 = 0; k1 < R; ++k1)
        append_image(t, ct, [&](int k2, int n2) { return omega((int64_t)n2 * (k1 + R * k2), 16 * R); });
    // F3[k1]: G(k3, n3) = w16^(n3 k3) * w_M^(n3 k1) = w_M^(n3 (k1 + 16 R k3))
    for (int k1 = 0; k1 < R; ++k1)
        append_image(t, ct, [&](int k3, int n3) { return omega((int64_t)n3 * (k1 + 16 * R * k3), M); });
    // I1[k1]: G(n3, k3) = conj(w_M^(n3 (k1 + 16 R k3)))
    for (int k1 = 0; k1 < R; ++k1)
        append_image(t, ct, [&](int n3, int k3) { return omega(-(int64_t)n3 * (k1 + 16 * R * k3), M); });
    // I2[k1]: G(n2, k2) = conj(w_{16R}^(n2 (k1 + R k2)))
    for (int k1 = 0; k1 < R; ++k1)
        append_image(t, ct, [&](int n2, int k2) { return omega(-(int64_t)n2 * (k1 + R * k2), 16 * R); });
    // TW: lane (g, c), j -> w_256^((4g + j) c), fp32 complex
    size_t base = t.size();
    t.resize(base + 64 * 4 * 8);
    for (int lane = 0; lane < 64; ++lane) {
        int g = lane / 16, c = lane % 16;
        for (int j = 0; j < 4; ++j) {
            cplx w = omega((int64_t)(4 * g + j) * c, 256);
            float f[2] = {(float)w.re, (float)w.im};
            std::memcpy(t.data() + base + ((size_t)lane * 4 + j) * 8, f, 8);
        }
    }
    t.resize(L.total, 0);
    return t;
}

std::vector<uint8_t> build_colmx_tables(int P, int ct) {
    const ColMxGrid G = colmx_grid(P);
    std::vector<uint8_t> t;
    // forward first stage: rows k1 = 16 rb + x, inputs n1 = 16 kc + ci (zero input past H)
    for (int rb = 0; rb < G.rbk; ++rb)
        for (int kc = 0; kc < G.hb; ++kc)
            append_image(t, ct, [&](int x, int ci) {
                const int k1 = 16 * rb + x, n1 = 16 * kc + ci;
                return n1 < G.H ? omega((int64_t)k1 * n1, G.R) : cplx{0, 0};
            });
    // inverse first stage: rows n1 = 16 rb + x (kept only below H), inputs k1 = 16 kc + ci
    for (int rb = 0; rb < G.hb; ++rb)
        for (int kc = 0; kc < G.rbk; ++kc)
            append_image(t, ct, [&](int x, int ci) {
                const int n1 = 16 * rb + x, k1 = 16 * kc + ci;
                return n1 < G.H ? omega(-(int64_t)k1 * n1, G.R) : cplx{0, 0};
            });
    append_image(t, ct, [&](int k2, int n2) { return omega((int64_t)n2 * k2, 16); });
    append_image(t, ct, [&](int n2, int k2) { return omega(-(int64_t)n2 * k2, 16); });
    append_image(t, ct, [&](int r, int n2) { return omega((int64_t)n2 * (15 - r), 16); });
    return t;
}

std::vector<uint8_t> build_dense_dft_tables(int P, int ct) {
    const int NB = P / 16;
    std::vector<uint8_t> t;
    for (int kb = 0; kb < NB; ++kb)
        for (int nb = 0; nb < NB; ++nb)
            append_image(t, ct, [&](int r, int c) { return omega((int64_t)(16 * kb + r) * (16 * nb + c), P); });
    for (int mb = 0; mb < NB; ++mb)
        for (int kb = 0; kb < NB; ++kb)
            append_image(t, ct, [&](int r, int c) { return omega(-(int64_t)(16 * mb + r) * (16 * kb + c), P); });
    // interleaved blocks (NB even): 32-row groups kp split by parity, k = 32 kp + 2 r + par
    for (int kq = 0; kq < NB; ++kq)  // kq = 2 kp + par: forward, output rows interleaved
        for (int nb = 0; nb < NB; ++nb)
            append_image(t, ct, [&](int r, int c) {
                return omega((int64_t)(32 * (kq / 2) + 2 * r + kq % 2) * (16 * nb + c), P);
            });
    for (int mb = 0; mb < NB; ++mb)  // inverse, input columns interleaved
        for (int kq = 0; kq < NB; ++kq)
            append_image(t, ct, [&](int r, int c) {
                return omega(-(int64_t)(16 * mb + r) * (32 * (kq / 2) + 2 * c + kq % 2), P);
            });
    return t;
}

struct DevBuf {
    void* ptr = nullptr;
    std::vector<uint8_t> host;  // kept alive for the lifetime of the cache
};

std::mutex g_mu;
std::map<std::tuple<int, int, int, int64_t, int64_t>, DevBuf> g_cache;  // (dev, kind, ct, a, b)
std::map<int, int> g_cu;

const void* get_or_build(int kind, int ct, int64_t a, int64_t b,
                         std::vector<uint8_t> (*build)(int, int, int64_t, int64_t), hipError_t* err,
                         bool may_build = true) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { *err = e; return nullptr; }
    std::lock_guard<std::mutex> lk(g_mu);
    auto key = std::make_tuple(dev, kind, ct, a, b);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second.ptr;
    if (!may_build) { *err = hipErrorNotReady; return nullptr; }
    DevBuf buf;
    buf.host = build(kind, ct, a, b);
    e = hipMalloc(&buf.ptr, buf.host.size());
    if (e != hipSuccess) { *err = e; return nullptr; }
    // blocking copy: the table is complete and visible to every stream before first use
    e = hipMemcpy(buf.ptr, buf.host.data(), buf.host.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) { hipFree(buf.ptr); *err = e; return nullptr; }
    const void* p = buf.ptr;
    g_cache.emplace(key, std::move(buf));
    return p;
}

std::vector<uint8_t> build_any(int kind, int ct, int64_t a, int64_t b) {
    if (kind == 0) return build_fused_tables((int)a, ct);
    if (kind == 3) return build_colmx_tables((int)a, ct);
    if (kind == 4) return build_dense_dft_tables((int)a, ct);
    if (kind == 2) {  // P-point DFT twiddles
        std::vector<uint8_t> t((size_t)a * 8);
        float* f = (float*)t.data();
        for (int64_t e = 0; e < a; ++e) {
            cplx w = omega(e, a);
            f[2 * e] = (float)w.re;
            f[2 * e + 1] = (float)w.im;
        }
        return t;
    }
    // kind 1: column twiddles for (M = a, M1 = b)
    const int64_t M = a, M1 = b;
    const int64_t nlo = 2048, nhi = M / 2048 > 0 ? M / 2048 : 1;
    std::vector<uint8_t> t((size_t)(nlo + nhi + M1) * 8);
    float* f = (float*)t.data();
    for (int64_t r = 0; r < nlo; ++r) { cplx w = omega(r, M); f[2 * r] = (float)w.re; f[2 * r + 1] = (float)w.im; }
    f += 2 * nlo;
    for (int64_t r = 0; r < nhi; ++r) { cplx w = omega(2048 * r, M); f[2 * r] = (float)w.re; f[2 * r + 1] = (float)w.im; }
    f += 2 * nhi;
    for (int64_t r = 0; r < M1; ++r) { cplx w = omega(r, M1); f[2 * r] = (float)w.re; f[2 * r + 1] = (float)w.im; }
    return t;
}

}  // namespace

FusedTableLayout fused_table_layout(int R, int ct) {
    FusedTableLayout L;
    L.img_bytes = (ct == CT_F32 ? 4 : 2) * 16 * 64;
    L.rb1 = (R + 15) / 16;
    L.kc1 = (R + 15) / 16;
    L.rb3 = (R + 15) / 16;
    L.kc3 = (R + 15) / 16;
    size_t o = 0;
    L.f1 = o; o += L.img_bytes * L.rb1 * L.kc1;
    L.i3 = o; o += L.img_bytes * L.rb3 * L.kc3;
    L.f2 = o; o += L.img_bytes * R;
    L.f3 = o; o += L.img_bytes * R;
    L.i1 = o; o += L.img_bytes * R;
    L.i2 = o; o += L.img_bytes * R;
    L.tw = o; o += 64 * 4 * 8;
    L.total = (o + 255) & ~(size_t)255;
    return L;
}

const void* fused_tables(int R, int ct, hipError_t* err, bool build) {
    return get_or_build(0, ct, R, 0, build_any, err, build);
}

bool col_tables(int64_t M, int64_t M1, ColTables* out, hipError_t* err, bool build) {
    const void* p = get_or_build(1, 0, M, M1, build_any, err, build);
    if (!p) return false;
    const int64_t nlo = 2048, nhi = M / 2048 > 0 ? M / 2048 : 1;
    out->lo = (const float*)p;
    out->hi = out->lo + 2 * nlo;
    out->col = out->hi + 2 * nhi;
    return true;
}

const void* colmx_tables(int64_t P, int ct, hipError_t* err, bool build) {
    return get_or_build(3, ct, P, 0, build_any, err, build);
}

const float* dft_table(int64_t P, hipError_t* err) {
    return (const float*)get_or_build(2, 0, P, 0, build_any, err);
}

const void* dense_dft_tables(int64_t P, int ct, hipError_t* err) {
    if ((P != 32 && P != 64) || ct == CT_F32) { *err = hipErrorInvalidValue; return nullptr; }
    return get_or_build(4, ct, P, 0, build_any, err);
}

int device_cu_count(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { *err = e; return 0; }
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_cu.find(dev);
    if (it != g_cu.end()) return it->second;
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0) { *err = e != hipSuccess ? e : hipErrorInvalidDevice; return 0; }
    g_cu[dev] = n;
    return n;
}

void release_tables() {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_cache) {
        int dev = std::get<0>(kv.first), cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(dev) == hipSuccess) {
            hipFree(kv.second.ptr);
            hipSetDevice(cur);
        }
    }
    g_cache.clear();
}

}  // namespace lcv
