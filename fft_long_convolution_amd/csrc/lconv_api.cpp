// lconv_api.cpp -- the C ABI: argument validation (host only, before any HIP call), plan
// selection and kernel dispatch.  See include/lconv.h for the contract.
#include "lconv.h"

#include <cstdint>
#include <cstring>

#include "kernels.h"
#include "plan.h"

using namespace lcv;

namespace {

constexpr size_t kChunkTarget = (size_t)64 << 20;  // multi-pass workspace per chunk (MALL-sized)

size_t dtype_size(lconv_dtype_t dt) { return dt == LCONV_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == LCONV_F32 || dt == LCONV_F16 || dt == LCONV_BF16; }
// complex element bytes of the compute type used on the multi-pass path
size_t work_complex_size(lconv_dtype_t dt, bool filter) { return (filter || dt == LCONV_F32) ? 8 : 4; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// lengths the forward call and the filter transform take (any N: ragged rows are staged)
bool n_in_range(int64_t N) { return N >= 1 && N <= LCONV_MAX_N; }
// lengths the kernels take directly: rows of whole 16-byte groups
bool n_supported(int64_t N) { return n_in_range(N) && (N % 8) == 0; }
int64_t round8(int64_t N) { return (N + 7) / 8 * 8; }
size_t round256(size_t b) { return (b + 255) / 256 * 256; }
// staging for N not a multiple of 8: `tensors` zero-padded copies of [rows][round8(N)]
size_t staging_bytes(int64_t rows, int64_t N, lconv_dtype_t dt, int tensors) {
    if (N % 8 == 0) return 0;
    return (size_t)tensors * round256((size_t)rows * (size_t)round8(N) * dtype_size(dt));
}

// sequences = complex transforms: pairs of batch rows per channel
int64_t pairs_per_channel(int64_t B) { return (B + 1) / 2; }

int64_t chunk_seqs(int64_t total, int64_t M, size_t csz) {
    int64_t per = (int64_t)(kChunkTarget / ((size_t)M * csz));
    if (per < 1) per = 1;
    return per < total ? per : total;
}

lconv_status_t hip_status(hipError_t e) { return e == hipSuccess ? LCONV_SUCCESS : LCONV_ERR_HIP; }

// the calls on rows of whole 16-byte groups (N a multiple of 8), after validation
lconv_status_t filter_fft_aligned(const void* k, void* k_f, int64_t H, int64_t N, lconv_dtype_t dtype,
                                  void* workspace, hipStream_t stream);
lconv_status_t fftconv_fwd_aligned(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                   const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                   void* workspace, hipStream_t stream);

}  // namespace

extern "C" {

int lconv_abi_version(void) { return LCONV_ABI_VERSION; }

const char* lconv_status_string(lconv_status_t s) {
    switch (s) {
    case LCONV_SUCCESS: return "success";
    case LCONV_ERR_NULL_POINTER: return "a required pointer is NULL";
    case LCONV_ERR_INVALID_SHAPE: return "invalid shape (negative size or size overflow)";
    case LCONV_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case LCONV_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case LCONV_ERR_ALIASING: return "the output overlaps an input";
    case LCONV_ERR_WORKSPACE: return "workspace missing or too small";
    case LCONV_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t lconv_filter_fft_bytes(int64_t H, int64_t N, lconv_dtype_t dtype) {
    Plan1D p;
    int64_t t;
    if (!dtype_ok(dtype) || H < 0 || !n_in_range(N) || !make_plan_1d(N, &p)) return 0;
    if (!mul_ok(H, p.M, &t) || !mul_ok(t, 2 * (int64_t)dtype_size(dtype), &t)) return 0;
    return (size_t)t;
}

size_t lconv_filter_fft_workspace_bytes(int64_t H, int64_t N, lconv_dtype_t dtype) {
    Plan1D p;
    if (!dtype_ok(dtype) || H < 0 || !n_in_range(N) || !make_plan_1d(N, &p)) return 0;
    if (H == 0) return 0;
    const size_t stage = staging_bytes(H, N, dtype, 1);
    if (!p.multipass) return stage;
    const size_t csz = work_complex_size(dtype, true);
    return stage + (size_t)chunk_seqs(H, p.M, csz) * (size_t)p.M * csz;
}

size_t lconv_fftconv_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype) {
    Plan1D p;
    int64_t seqs, rows;
    if (!dtype_ok(dtype) || B < 0 || H < 0 || !n_in_range(N) || !make_plan_1d(N, &p)) return 0;
    if (B == 0 || H == 0) return 0;
    if (!mul_ok(pairs_per_channel(B), H, &seqs) || !mul_ok(B, H, &rows)) return 0;
    const size_t stage = staging_bytes(rows, N, dtype, 4);  // u, q, v, y
    if (!p.multipass) return stage;
    const size_t csz = work_complex_size(dtype, false);
    return stage + (size_t)chunk_seqs(seqs, p.M, csz) * (size_t)p.M * csz;
}

size_t lconv_filter_fft2d_bytes(int64_t C, int64_t S, lconv_dtype_t dtype) {
    int64_t t;
    if (!dtype_ok(dtype) || dtype == LCONV_F32 || C < 0 || S != LCONV_2D_SIDE) return 0;
    // spectrum of the (2S x 2S) transform in the 2D kernel's order, complex in dtype
    if (!mul_ok(C, 4 * S * S, &t) || !mul_ok(t, 2 * (int64_t)dtype_size(dtype), &t)) return 0;
    return (size_t)t;
}

lconv_status_t lconv_filter_fft(const void* k, void* k_f, int64_t H, int64_t N, lconv_dtype_t dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t t;
    if (!mul_ok(H, N, &t) || !mul_ok(t, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (H == 0 || N == 0) return LCONV_SUCCESS;
    if (!n_in_range(N)) return LCONV_ERR_UNSUPPORTED;
    if (!k || !k_f) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(k) || !aligned16(k_f)) return LCONV_ERR_MISALIGNED;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(k_f, kf_bytes, k, (size_t)(H * N) * dtype_size(dtype))) return LCONV_ERR_ALIASING;
    const size_t need = lconv_filter_fft_workspace_bytes(H, N, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
        if (overlap(workspace, need, k_f, kf_bytes) || overlap(workspace, need, k, (size_t)(H * N) * dtype_size(dtype)))
            return LCONV_ERR_ALIASING;
    }
    if (N % 8 != 0) {  // ragged rows: stage zero-padded copies (the padding taps are zero)
        const size_t stage = staging_bytes(H, N, dtype, 1);
        if (launch_pad_rows(k, workspace, H, N, round8(N), (int)dtype_size(dtype), stream) != hipSuccess)
            return LCONV_ERR_HIP;
        return filter_fft_aligned(workspace, k_f, H, round8(N), dtype, (char*)workspace + stage, stream);
    }
    return filter_fft_aligned(k, k_f, H, N, dtype, workspace, stream);
}

}  // extern "C"

namespace {

lconv_status_t filter_fft_aligned(const void* k, void* k_f, int64_t H, int64_t N, lconv_dtype_t dtype,
                                  void* workspace, hipStream_t stream) {
    Plan1D p;
    make_plan_1d(N, &p);
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const void* tabs = fused_tables(p.R, CT_F32, &err);
    if (!tabs) return LCONV_ERR_HIP;
    if (!p.multipass) {
        Fused1DArgs a{};
        a.u = k; a.y = k_f; a.tables = tabs;
        a.B = 1; a.H = H; a.N = N; a.nitems = H;
        a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1;
        return hip_status(launch_fused1d(p.R, dtype, MODE_FILTER, false, false, a, cus, stream));
    }
    ColTables ct;
    if (!col_tables(p.M, p.M1, &ct, &err)) return LCONV_ERR_HIP;
    const int64_t per = chunk_seqs(H, p.M, work_complex_size(dtype, true));
    for (int64_t h0 = 0; h0 < H; h0 += per) {
        const int64_t ns = per < H - h0 ? per : H - h0;
        ColArgs c{};
        c.u = k; c.ws = workspace; c.tw_lo = ct.lo; c.tw_hi = ct.hi; c.tw_col = ct.col;
        c.B = 1; c.H = H; c.N = N; c.M = p.M; c.M1 = p.M1; c.seq0 = h0; c.nseq = ns;
        c.seq_per_h = 1; c.filter = 1;
        err = launch_col_fwd(dtype, c, stream);
        if (err != hipSuccess) return LCONV_ERR_HIP;
        Fused1DArgs a{};
        a.u = workspace; a.y = k_f; a.tables = tabs;
        a.nitems = ns * p.M1; a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = p.M1;
        a.seq0 = h0; a.seq_per_h = 1;
        err = launch_fused1d(32, dtype, MODE_ROWFWD, false, false, a, cus, stream);
        if (err != hipSuccess) return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

}  // namespace

extern "C" {

lconv_status_t lconv_fftconv_fwd(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                 const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    if (!n_in_range(N)) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y) || (q && !aligned16(q)) ||
        (v && !aligned16(v)))
        return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(y, act, u, act) || overlap(y, act, q, act) || overlap(y, act, v, act) ||
        overlap(y, act, k_f, kf_bytes) || overlap(y, act, D, (size_t)H * es))
        return LCONV_ERR_ALIASING;
    const size_t need = lconv_fftconv_workspace_bytes(B, H, N, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
        if (overlap(workspace, need, y, act) || overlap(workspace, need, u, act) ||
            overlap(workspace, need, q, act) || overlap(workspace, need, v, act) ||
            overlap(workspace, need, k_f, kf_bytes) || overlap(workspace, need, D, (size_t)H * es))
            return LCONV_ERR_ALIASING;
    }
    if (N % 8 != 0) {
        // ragged rows: zero-padded copies of u, q, v (zero inputs past N change no output before
        // N), the aligned path at round8(N), and the first N outputs of each row copied back
        const int64_t rows = B * H, N8 = round8(N);
        const size_t one = staging_bytes(rows, N, dtype, 1);
        char* st = (char*)workspace;
        void *su = st, *sq = q ? st + one : nullptr, *sv = v ? st + 2 * one : nullptr, *sy = st + 3 * one;
        const int esz = (int)es;
        if (launch_pad_rows(u, su, rows, N, N8, esz, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (q && launch_pad_rows(q, sq, rows, N, N8, esz, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (v && launch_pad_rows(v, sv, rows, N, N8, esz, stream) != hipSuccess) return LCONV_ERR_HIP;
        const lconv_status_t r = fftconv_fwd_aligned(su, k_f, D, sy, sq, sv, B, H, N8, dtype, st + 4 * one, stream);
        if (r != LCONV_SUCCESS) return r;
        return hip_status(launch_unpad_rows(sy, y, rows, N, N8, esz, stream));
    }
    return fftconv_fwd_aligned(u, k_f, D, y, q, v, B, H, N, dtype, workspace, stream);
}

}  // extern "C"

namespace {

lconv_status_t fftconv_fwd_aligned(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                   const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                   void* workspace, hipStream_t stream) {
    Plan1D p;
    make_plan_1d(N, &p);
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const void* tabs = fused_tables(p.R, ct, &err);
    if (!tabs) return LCONV_ERR_HIP;
    const int64_t Bp = pairs_per_channel(B), seqs = Bp * H;
    if (!p.multipass) {
        Fused1DArgs a{};
        a.u = u; a.q = q; a.v = v; a.y = y; a.kf = k_f; a.D = D; a.tables = tabs;
        a.B = B; a.H = H; a.N = N; a.nitems = seqs;
        a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1;
        return hip_status(launch_fused1d(p.R, dtype, MODE_CONV, q != nullptr, v != nullptr, a, cus, stream));
    }
    ColTables ctab;
    if (!col_tables(p.M, p.M1, &ctab, &err)) return LCONV_ERR_HIP;
    const int64_t per = chunk_seqs(seqs, p.M, work_complex_size(dtype, false));
    for (int64_t s0 = 0; s0 < seqs; s0 += per) {
        const int64_t ns = per < seqs - s0 ? per : seqs - s0;
        ColArgs c{};
        c.u = u; c.q = q; c.v = v; c.y = y; c.ws = workspace;
        c.tw_lo = ctab.lo; c.tw_hi = ctab.hi; c.tw_col = ctab.col;
        c.B = B; c.H = H; c.N = N; c.M = p.M; c.M1 = p.M1; c.seq0 = s0; c.nseq = ns;
        c.seq_per_h = Bp; c.filter = 0;
        if (launch_col_fwd(dtype, c, stream) != hipSuccess) return LCONV_ERR_HIP;
        Fused1DArgs a{};
        a.u = workspace; a.y = workspace; a.kf = k_f; a.D = D; a.tables = tabs;
        a.nitems = ns * p.M1; a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = p.M1;
        a.seq0 = s0; a.seq_per_h = Bp;
        if (launch_fused1d(32, dtype, MODE_ROW, false, false, a, cus, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (launch_col_inv(dtype, c, stream) != hipSuccess) return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

}  // namespace

extern "C" {

int lconv_freq_blocks(int64_t N) {
    Plan1D p;
    if (!n_supported(N) || N > LCONV_BWD_MAX_N || !make_plan_1d(N, &p) || p.multipass) return 0;
    return p.R;
}


lconv_status_t lconv_fftconv_sparse_fwd(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                        const void* v, int64_t B, int64_t H, int64_t N, uint32_t keep,
                                        lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    const int R = lconv_freq_blocks(N);
    if (R == 0) return LCONV_ERR_UNSUPPORTED;
    if (R < 32 && (keep >> R) != 0) return LCONV_ERR_UNSUPPORTED;
    for (int r = 0; r < R; ++r)
        if (((keep >> r) & 1u) != ((keep >> ((R - r) % R)) & 1u)) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y) || (q && !aligned16(q)) ||
        (v && !aligned16(v)))
        return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(y, act, u, act) || overlap(y, act, q, act) || overlap(y, act, v, act) ||
        overlap(y, act, k_f, kf_bytes) || overlap(y, act, D, (size_t)H * es))
        return LCONV_ERR_ALIASING;
    Plan1D p;
    make_plan_1d(N, &p);
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const void* tabs = fused_tables(p.R, ct, &err);
    if (!tabs) return LCONV_ERR_HIP;
    Fused1DArgs a{};
    a.u = u; a.q = q; a.v = v; a.y = y; a.kf = k_f; a.D = D; a.tables = tabs;
    a.B = B; a.H = H; a.N = N; a.nitems = pairs_per_channel(B) * H; a.keep = keep;
    a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1;
    return hip_status(launch_fused1d(p.R, dtype, MODE_SPARSE, q != nullptr, v != nullptr, a, cus, stream));
}

}  // extern "C"

namespace {

lconv_status_t partial_impl(const void* u, const void* k_f, const void* D, void* y, const void* q, const void* v,
                            int64_t B, int64_t H, int64_t N, int64_t L, lconv_dtype_t dtype, int local,
                            hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0 || L < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    if (L < 8 || L > 4096 || (L % 8) != 0 || (N % 8) != 0 || N > ((int64_t)1 << 40)) return LCONV_ERR_UNSUPPORTED;
    Plan1D p;
    if (!make_plan_1d(L, &p) || p.multipass) return LCONV_ERR_UNSUPPORTED;
    // sequences of a channel: (batch row, block) windows, transformed two at a time
    const int64_t C = p.M / 2, nch = (N + C - 1) / C;
    int64_t nseq, items;
    if (!mul_ok(B, nch, &nseq) || !mul_ok((nseq + 1) / 2, H, &items) || nseq >= ((int64_t)1 << 32) ||
        items >= ((int64_t)1 << 31))
        return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y) || (q && !aligned16(q)) ||
        (v && !aligned16(v)))
        return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, L, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(y, act, u, act) || overlap(y, act, q, act) || overlap(y, act, v, act) ||
        overlap(y, act, k_f, kf_bytes) || overlap(y, act, D, (size_t)H * es))
        return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const void* tabs = fused_tables(p.R, ct, &err);
    if (!tabs) return LCONV_ERR_HIP;
    if (local && p.M == 8192 && dtype != LCONV_F32 && N % C == 0) {
        // whole blocks convolved on their own: per batch row, the blocks of a channel are the
        // batch rows (stride C) of a plain convolution of length C on the pipelined kernel
        for (int64_t b = 0; b < B; ++b) {
            const int64_t off = b * H * N * (int64_t)es;
            Fused1DArgs a{};
            a.u = (const char*)u + off; a.y = (char*)y + off;
            a.q = q ? (const char*)q + off : nullptr; a.v = v ? (const char*)v + off : nullptr;
            a.kf = k_f; a.D = D; a.tables = tabs;
            a.B = nch; a.H = H; a.N = C; a.sb = C; a.sh = N; a.nitems = (nch + 1) / 2 * H;
            a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1;
            const hipError_t e = launch_fused1d(p.R, dtype, MODE_CONV, q != nullptr, v != nullptr, a, cus, stream);
            if (e != hipSuccess) return hip_status(e);
        }
        return LCONV_SUCCESS;
    }
    Fused1DArgs a{};
    a.u = u; a.q = q; a.v = v; a.y = y; a.kf = k_f; a.D = D; a.tables = tabs;
    a.B = B; a.H = H; a.N = N; a.nitems = items; a.nchunk = nch;
    a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1; a.local = local;
    return hip_status(launch_fused1d(p.R, dtype, MODE_PART, q != nullptr, v != nullptr, a, cus, stream));
}

}  // namespace

extern "C" {

lconv_status_t lconv_fftconv_partial_fwd(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                         const void* v, int64_t B, int64_t H, int64_t N, int64_t L,
                                         lconv_dtype_t dtype, hipStream_t stream) {
    return partial_impl(u, k_f, D, y, q, v, B, H, N, L, dtype, 0, stream);
}

}  // extern "C"

namespace {

// The gradient call; with c (the forward's saved pre-gate output) dv = dy (.) c replaces the
// forward-by-dy launch.
lconv_status_t bwd_impl(const void* dy, const void* u, const void* k_f, const void* D, const void* q,
                        const void* v, const void* c, void* du, void* dq, void* dv, float* dk, float* dD,
                        int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t, hn;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t) || !mul_ok(H, N, &hn) ||
        !mul_ok(hn, 8, &t))
        return LCONV_ERR_INVALID_SHAPE;
    if (H == 0 || N == 0) return LCONV_SUCCESS;
    if (!n_supported(N) || N > LCONV_BWD_MAX_N) return LCONV_ERR_UNSUPPORTED;
    if (!q) dq = nullptr;  // ignored without the gate it belongs to
    if (!v) dv = nullptr;
    if (B == 0) {          // empty batch: the filter gradients are zero sums
        if ((dk && !aligned16(dk)) || (dD && !aligned16(dD))) return LCONV_ERR_MISALIGNED;
        if (dk && hipMemsetAsync(dk, 0, (size_t)hn * 4, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (dD && hipMemsetAsync(dD, 0, (size_t)H * 4, stream) != hipSuccess) return LCONV_ERR_HIP;
        return LCONV_SUCCESS;
    }
    if (!dy || !u || !k_f || !D || !du || (q && !dq) || (v && !dv)) return LCONV_ERR_NULL_POINTER;
    const void* ptrs[] = {dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    // every output against every input and every other output
    const void* ins[] = {dy, u, k_f, D, q, v, c};
    const size_t in_sz[] = {act, act, kf_bytes, (size_t)H * es, act, act, act};
    const void* outs[] = {du, dq, dv, dk, dD};
    const size_t out_sz[] = {act, act, act, (size_t)hn * 4, (size_t)H * 4};
    for (int o = 0; o < 5; ++o) {
        for (int i = 0; i < 7; ++i)
            if (overlap(outs[o], out_sz[o], ins[i], in_sz[i])) return LCONV_ERR_ALIASING;
        for (int o2 = o + 1; o2 < 5; ++o2)
            if (overlap(outs[o], out_sz[o], outs[o2], out_sz[o2])) return LCONV_ERR_ALIASING;
    }
    Plan1D p;
    make_plan_1d(N, &p);
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const void* tabs = fused_tables(p.R, ct, &err);
    if (!tabs) return LCONV_ERR_HIP;
    const int64_t seqs = pairs_per_channel(B) * H;
    Fused1DArgs base{};
    base.kf = k_f; base.D = D; base.tables = tabs;
    base.B = B; base.H = H; base.N = N;
    base.inv_m = 1.0f / (float)p.M; base.M = p.M; base.M1 = 1;
    // dv = dy (.) (k * x + D x): from the saved pre-gate output, or the forward convolution with
    // dy as its post-gate
    if (v && c) {
        if (launch_mul_rows(dy, c, dv, elems, (int)ct, stream) != hipSuccess) return LCONV_ERR_HIP;
    } else if (v) {
        Fused1DArgs a = base;
        a.u = u; a.q = q; a.v = dy; a.y = dv; a.nitems = seqs;
        if (launch_fused1d(p.R, dtype, MODE_CONV, q != nullptr, true, a, cus, stream) != hipSuccess)
            return LCONV_ERR_HIP;
    }
    // du = q (.) dx, dq = u (.) dx: the adjoint chain on ds = dy (.) v
    {
        Fused1DArgs a = base;
        a.u = dy; a.q = v; a.v = q; a.e2 = u; a.y = du; a.y2 = dq; a.nitems = seqs;
        if (launch_fused1d(p.R, dtype, MODE_ADJ, v != nullptr, q != nullptr, a, cus, stream) != hipSuccess)
            return LCONV_ERR_HIP;
    }
    // dk, dD: per channel, the batch sum of the correlation of ds with x
    if (dk || dD) {
        Fused1DArgs a = base;
        a.u = u; a.q = q; a.e2 = dy; a.v = v; a.y = dk; a.y2 = dD; a.nitems = H;
        if (launch_dk1d(p.R, dtype, q != nullptr, v != nullptr, a, cus, stream) != hipSuccess)
            return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

}  // namespace

extern "C" {

lconv_status_t lconv_fftconv_bwd(const void* dy, const void* u, const void* k_f, const void* D, const void* q,
                                 const void* v, void* du, void* dq, void* dv, float* dk, float* dD, int64_t B,
                                 int64_t H, int64_t N, lconv_dtype_t dtype, hipStream_t stream) {
    return bwd_impl(dy, u, k_f, D, q, v, nullptr, du, dq, dv, dk, dD, B, H, N, dtype, stream);
}

lconv_status_t lconv_fftconv_bwd_saved(const void* dy, const void* u, const void* k_f, const void* D,
                                       const void* q, const void* v, const void* c, void* du, void* dq, void* dv,
                                       float* dk, float* dD, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                       hipStream_t stream) {
    if (!c && v && B > 0 && H > 0 && N > 0) return LCONV_ERR_NULL_POINTER;
    return bwd_impl(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype, stream);
}

lconv_status_t lconv_fftconv_fwd_save(const void* u, const void* k_f, const void* D, void* y, void* c,
                                      const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                      lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    if (!n_supported(N) || N > LCONV_BWD_MAX_N) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y || !c) return LCONV_ERR_NULL_POINTER;
    const void* ptrs[] = {u, k_f, D, y, c, q, v};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    const void* ins[] = {u, k_f, D, q, v};
    const size_t in_sz[] = {act, kf_bytes, (size_t)H * es, act, act};
    for (int i = 0; i < 5; ++i)
        if (overlap(y, act, ins[i], in_sz[i]) || overlap(c, act, ins[i], in_sz[i])) return LCONV_ERR_ALIASING;
    if (overlap(y, act, c, act)) return LCONV_ERR_ALIASING;
    Plan1D p;
    make_plan_1d(N, &p);
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const void* tabs = fused_tables(p.R, ct, &err);
    if (!tabs) return LCONV_ERR_HIP;
    Fused1DArgs a{};
    a.u = u; a.q = q; a.v = v; a.y = y; a.y2 = c; a.kf = k_f; a.D = D; a.tables = tabs;
    a.B = B; a.H = H; a.N = N; a.nitems = pairs_per_channel(B) * H;
    a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1;
    return hip_status(launch_fused1d(p.R, dtype, MODE_SAVE, q != nullptr, v != nullptr, a, cus, stream));
}

lconv_status_t lconv_filter_fft2d(const void* k, void* k_f, int64_t C, int64_t S, lconv_dtype_t dtype,
                                  hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (C < 0 || S < 0) return LCONV_ERR_INVALID_SHAPE;
    if (C == 0) return LCONV_SUCCESS;
    if (S != LCONV_2D_SIDE || dtype == LCONV_F32) return LCONV_ERR_UNSUPPORTED;
    if (!k || !k_f) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(k) || !aligned16(k_f)) return LCONV_ERR_MISALIGNED;
    const size_t kf_bytes = lconv_filter_fft2d_bytes(C, S, dtype);
    if (overlap(k_f, kf_bytes, k, (size_t)(C * S * S) * dtype_size(dtype))) return LCONV_ERR_ALIASING;
    Conv2DArgs a{};
    a.u = k; a.kf = k_f; a.C = C; a.B = 1; a.filter = 1;
    a.inv_p2 = 1.0f / (float)(4 * S * S);
    return hip_status(launch_conv2d(dtype, a, stream));
}

lconv_status_t lconv_fftconv2d_fwd(const void* u, const void* k_f, const void* D, void* y, int64_t B, int64_t C,
                                   int64_t S, lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || C < 0 || S < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, C, &t) || !mul_ok(t, S * S, &elems)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || C == 0) return LCONV_SUCCESS;
    if (S != LCONV_2D_SIDE || dtype == LCONV_F32) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y)) return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    if (overlap(y, act, u, act) || overlap(y, act, k_f, lconv_filter_fft2d_bytes(C, S, dtype)) ||
        overlap(y, act, D, (size_t)C * es))
        return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const void* tabs = fused_tables(1, (int)dtype, &err);  // 256-point transform blocks
    if (!tabs) return LCONV_ERR_HIP;
    Conv2DArgs a{};
    a.u = u; a.kf = k_f; a.D = D; a.y = y; a.tables = tabs;
    a.B = B; a.C = C; a.filter = 0; a.cus = cus;
    a.inv_p2 = 1.0f / (float)(4 * S * S);
    return hip_status(launch_conv2d(dtype, a, stream));
}

// ---- 3D ---------------------------------------------------------------------------------------

namespace {
bool s3_ok(int64_t S) { return S == 16 || S == 32; }
// workspace bytes per unit: S slices of (2S)^2 complex in the pass's compute type
size_t ws3_unit(int64_t S, size_t csz) { return (size_t)S * 4 * S * S * csz; }
int64_t chunk3(int64_t units, int64_t S, size_t csz) {
    int64_t per = (int64_t)(kChunkTarget / ws3_unit(S, csz));
    if (per < 1) per = 1;
    return per < units ? per : units;
}
}  // namespace

size_t lconv_filter_fft3d_bytes(int64_t C, int64_t S, lconv_dtype_t dtype) {
    int64_t t;
    if (!dtype_ok(dtype) || C < 0 || !s3_ok(S)) return 0;
    if (!mul_ok(C, 8 * S * S * S, &t) || !mul_ok(t, 2 * (int64_t)dtype_size(dtype), &t)) return 0;
    return (size_t)t;
}

size_t lconv_filter_fft3d_workspace_bytes(int64_t C, int64_t S, lconv_dtype_t dtype) {
    if (!dtype_ok(dtype) || C <= 0 || !s3_ok(S)) return 0;
    return (size_t)chunk3(C, S, 8) * ws3_unit(S, 8);
}

size_t lconv_fftconv3d_workspace_bytes(int64_t B, int64_t C, int64_t S, lconv_dtype_t dtype) {
    int64_t units;
    if (!dtype_ok(dtype) || B <= 0 || C <= 0 || !s3_ok(S)) return 0;
    if (!mul_ok(pairs_per_channel(B), C, &units)) return 0;
    const size_t csz = work_complex_size(dtype, false);
    return (size_t)chunk3(units, S, csz) * ws3_unit(S, csz);
}

lconv_status_t lconv_filter_fft3d(const void* k, void* k_f, int64_t C, int64_t S, lconv_dtype_t dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (C < 0 || S < 0) return LCONV_ERR_INVALID_SHAPE;
    if (C == 0) return LCONV_SUCCESS;
    if (!s3_ok(S)) return LCONV_ERR_UNSUPPORTED;
    if (!k || !k_f) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(k) || !aligned16(k_f)) return LCONV_ERR_MISALIGNED;
    const size_t kf_bytes = lconv_filter_fft3d_bytes(C, S, dtype);
    const size_t k_bytes = (size_t)(C * S * S * S) * dtype_size(dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(k_f, kf_bytes, k, k_bytes)) return LCONV_ERR_ALIASING;
    const size_t need = lconv_filter_fft3d_workspace_bytes(C, S, dtype);
    if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
    if (overlap(workspace, need, k_f, kf_bytes) || overlap(workspace, need, k, k_bytes)) return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const float* tw = dft_table(2 * S, &err);
    if (!tw) return LCONV_ERR_HIP;
    const int64_t per = chunk3(C, S, 8);
    for (int64_t u0 = 0; u0 < C; u0 += per) {
        Conv3DArgs a{};
        a.u = k; a.y = k_f; a.ws = workspace; a.tw = tw;
        a.B = 1; a.C = C; a.S = S; a.unit0 = u0; a.nunit = per < C - u0 ? per : C - u0;
        a.inv_p3 = 1.0f / (float)(8 * S * S * S); a.filter = 1;
        if (launch_conv3d(dtype, a, stream) != hipSuccess) return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

lconv_status_t lconv_fftconv3d_fwd(const void* u, const void* k_f, const void* D, void* y, int64_t B, int64_t C,
                                   int64_t S, lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || C < 0 || S < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, C, &t) || !mul_ok(S, S, &elems) || !mul_ok(elems, S, &elems) || !mul_ok(t, elems, &elems) ||
        !mul_ok(elems, 8, &t))
        return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || C == 0) return LCONV_SUCCESS;
    if (!s3_ok(S)) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y)) return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft3d_bytes(C, S, dtype);
    if (overlap(y, act, u, act) || overlap(y, act, k_f, kf_bytes) || overlap(y, act, D, (size_t)C * es))
        return LCONV_ERR_ALIASING;
    const size_t need = lconv_fftconv3d_workspace_bytes(B, C, S, dtype);
    if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
    if (overlap(workspace, need, y, act) || overlap(workspace, need, u, act) ||
        overlap(workspace, need, k_f, kf_bytes) || overlap(workspace, need, D, (size_t)C * es))
        return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const float* tw = dft_table(2 * S, &err);
    if (!tw) return LCONV_ERR_HIP;
    const int64_t units = pairs_per_channel(B) * C;
    const int64_t per = chunk3(units, S, work_complex_size(dtype, false));
    for (int64_t u0 = 0; u0 < units; u0 += per) {
        Conv3DArgs a{};
        a.u = u; a.kf = k_f; a.D = D; a.y = y; a.ws = workspace; a.tw = tw;
        a.B = B; a.C = C; a.S = S; a.unit0 = u0; a.nunit = per < units - u0 ? per : units - u0;
        a.inv_p3 = 1.0f / (float)(8 * S * S * S); a.filter = 0;
        if (launch_conv3d(dtype, a, stream) != hipSuccess) return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

// ---- state-space filters, chunked with state passing --------------------------------------------

namespace {
bool ssm_t_ok(int64_t T) { return T >= 256 && T <= 4096 && (T & (T - 1)) == 0; }
// prep layout: [k_f of the chunk filter][md][pw][ts][tc][k chunk], each 256-byte aligned
struct SsmPrep {
    size_t kf, md, pw, ts, tc, kc, total;
};
bool ssm_layout(int64_t H, int64_t NS, int64_t T, lconv_dtype_t dt, SsmPrep* L) {
    if (!dtype_ok(dt) || H < 1 || NS < 1 || NS > 256 || !ssm_t_ok(T)) return false;
    const size_t kf = lconv_filter_fft_bytes(H, T, dt);
    if (kf == 0) return false;
    size_t o = 0;
    L->kf = o; o += round256(kf);
    const size_t nsp = (size_t)ssm_blocks(NS) * ssm_block_modes(NS);
    L->md = o; o += round256((size_t)H * NS * 32);
    L->pw = o; o += round256((size_t)H * 17 * nsp * 8);
    L->ts = o; o += round256((size_t)H * ssm_image_bytes(NS));
    L->tc = o; o += round256((size_t)H * ssm_image_bytes(NS));
    L->kc = o; o += round256((size_t)H * T * dtype_size(dt));
    L->total = o;
    return true;
}
}  // namespace

size_t lconv_ssm_prep_bytes(int64_t H, int64_t NS, int64_t T, lconv_dtype_t dtype) {
    SsmPrep L;
    return ssm_layout(H, NS, T, dtype, &L) ? L.total : 0;
}

lconv_status_t lconv_ssm_prepare(const float* lam, const float* W, void* prep, int64_t H, int64_t NS,
                                 int64_t T, lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (H < 0 || NS < 0 || T < 0) return LCONV_ERR_INVALID_SHAPE;
    if (H == 0) return LCONV_SUCCESS;
    SsmPrep L;
    if (!ssm_layout(H, NS, T, dtype, &L)) return LCONV_ERR_UNSUPPORTED;
    if (!lam || !W || !prep) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(lam) || !aligned16(W) || !aligned16(prep)) return LCONV_ERR_MISALIGNED;
    const size_t pbytes = (size_t)H * NS * 8;
    if (overlap(prep, L.total, lam, pbytes) || overlap(prep, L.total, W, pbytes)) return LCONV_ERR_ALIASING;
    char* P = (char*)prep;
    SsmArgs a{};
    a.md = P + L.md; a.pw = P + L.pw; a.ts = P + L.ts; a.tc = P + L.tc; a.kchunk = P + L.kc;
    a.H = H; a.NS = NS; a.T = T; a.nsb = ssm_block_modes(NS); a.nmb = ssm_blocks(NS);
    if (launch_ssm_prepare(dtype, lam, W, a, stream) != hipSuccess) return LCONV_ERR_HIP;
    // the chunk filter's spectrum (single pass: T <= 4096 needs no workspace)
    return lconv_filter_fft(P + L.kc, P + L.kf, H, T, dtype, nullptr, 0, stream);
}

size_t lconv_fftconv_ssm_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t NS, int64_t T) {
    int64_t rows, t;
    if (B < 1 || H < 1 || N < 1 || NS < 1 || NS > 256 || !ssm_t_ok(T)) return 0;
    const int64_t nch = (N + T - 1) / T;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, nch, &t) || !mul_ok(t, NS, &t) || !mul_ok(t, 8, &t)) return 0;
    const int64_t parts = nch < kSsmMaxParts ? nch : kSsmMaxParts;
    // chunk sums, boundary states, the scan's part states
    return 2 * round256((size_t)t) + round256((size_t)(rows * parts * NS * 8));
}

lconv_status_t lconv_fftconv_ssm_fwd(const void* u, const void* prep, const void* D, void* y, const void* q,
                                     const void* v, int64_t B, int64_t H, int64_t N, int64_t NS, int64_t T,
                                     lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0 || NS < 0 || T < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    SsmPrep L;
    if (!ssm_layout(H, NS, T, dtype, &L) || (N % 8) != 0 || N > ((int64_t)1 << 40)) return LCONV_ERR_UNSUPPORTED;
    const size_t need = lconv_fftconv_ssm_workspace_bytes(B, H, N, NS, T);
    if (need == 0) return LCONV_ERR_UNSUPPORTED;
    if (!u || !prep || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(prep) || !aligned16(D) || !aligned16(y) || (q && !aligned16(q)) ||
        (v && !aligned16(v)))
        return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    if (overlap(y, act, u, act) || overlap(y, act, q, act) || overlap(y, act, v, act) ||
        overlap(y, act, prep, L.total) || overlap(y, act, D, (size_t)H * es))
        return LCONV_ERR_ALIASING;
    if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
    if (overlap(workspace, need, y, act) || overlap(workspace, need, u, act) || overlap(workspace, need, q, act) ||
        overlap(workspace, need, v, act) || overlap(workspace, need, prep, L.total))
        return LCONV_ERR_ALIASING;
    const char* P = (const char*)prep;
    // 1. each chunk's own convolution with k[0:T] (+ D x, gated): the partial mode, previous block zero
    const lconv_status_t r = partial_impl(u, P + L.kf, D, y, q, v, B, H, N, T, dtype, 1, stream);
    if (r != LCONV_SUCCESS) return r;
    // 2-4. chunk sums, scan of the boundary states, correction of every output
    SsmArgs a{};
    a.u = u; a.q = q; a.v = v; a.y = y;
    a.md = (void*)(P + L.md); a.pw = (void*)(P + L.pw); a.ts = (void*)(P + L.ts); a.tc = (void*)(P + L.tc);
    const int64_t nch = (N + T - 1) / T;
    const size_t gbytes = round256((size_t)(B * H * nch * NS * 8));
    a.g = workspace; a.cs = (char*)workspace + gbytes; a.sp = (char*)workspace + 2 * gbytes;
    a.B = B; a.H = H; a.N = N; a.NS = NS; a.T = T; a.nch = nch;
    // scan parts: enough (row, part, mode) threads to fill the device, at most kSsmMaxParts
    int64_t parts = (32768 + B * H * NS - 1) / (B * H * NS);
    parts = parts < kSsmMaxParts ? parts : kSsmMaxParts;
    parts = parts < nch ? parts : nch;
    a.plen = (nch + parts - 1) / parts;
    a.nparts = (nch + a.plen - 1) / a.plen;
    a.nsb = ssm_block_modes(NS); a.nmb = ssm_blocks(NS);
    return hip_status(launch_ssm_state(dtype, a, q != nullptr, v != nullptr, stream));
}

lconv_status_t lconv_release(void) {
    release_tables();
    return LCONV_SUCCESS;
}

}  // extern "C"
