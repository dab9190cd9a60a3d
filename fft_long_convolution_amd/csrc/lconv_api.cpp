// lconv_api.cpp -- the C ABI: argument validation (host only, before any HIP call), plan
// selection and kernel dispatch.  See include/lconv.h for the contract.
#include "lconv.h"

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "api_internal.h"
#include "kernels.h"
#include "plan.h"

using namespace lcv;

namespace {

// Multi-pass workspace per chunk.  1D: 128 MB, half the 256 MB last-level cache (MALL), which the
// chunk's workspace round trips (written by the column pass, read and rewritten by the row pass,
// read by the inverse column pass) stay in; measured 8% faster on the long workloads than 64 MB
// chunks (more items per workgroup in the row pass), 192 MB no faster.  3D: 64 MB.
constexpr size_t kChunkTarget1D = (size_t)128 << 20;
constexpr size_t kChunkTarget = (size_t)64 << 20;

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

// 2D sides the fused kernel takes: rows 1..128, columns 8..128 in whole 16-byte groups
constexpr int64_t kP2D = 256;
bool sides2d_ok(int64_t Hs, int64_t Ws) {
    return Hs >= 1 && Hs <= LCONV_2D_MAX_SIDE && Ws >= 8 && Ws <= LCONV_2D_MAX_SIDE && Ws % 8 == 0;
}

// sequences = complex transforms: pairs of batch rows per channel
int64_t pairs_per_channel(int64_t B) { return B / 2 + (B & 1); }  // ceil(B / 2) without overflow

int64_t chunk_seqs(int64_t total, int64_t M, size_t csz, size_t target = kChunkTarget1D) {
    int64_t per = (int64_t)(target / ((size_t)M * csz));
    if (per < 1) per = 1;
    return per < total ? per : total;
}

lconv_status_t hip_status(hipError_t e) { return e == hipSuccess ? LCONV_SUCCESS : LCONV_ERR_HIP; }

// LCONV_LOG: one stderr line per distinct (call, B, H, N, dtype) with the plan it runs
void log_plan(const char* call, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, const Plan1D& p,
              int64_t chunk_seqs_) {
    if (!log_enabled()) return;
    static std::mutex mu;
    static std::set<std::tuple<std::string, int64_t, int64_t, int64_t, int>> seen;
    std::lock_guard<std::mutex> lk(mu);
    if (!seen.insert(std::make_tuple(std::string(call), B, H, N, (int)dtype)).second) return;
    std::fprintf(stderr, "lconv: %s B=%lld H=%lld N=%lld dtype=%s: M=%lld, %s (R=%d, M1=%lld%s)",
                 call, (long long)B, (long long)H, (long long)N,
                 dtype == LCONV_F32 ? "f32" : dtype == LCONV_F16 ? "f16" : "bf16", (long long)p.M,
                 p.multipass ? "multi-pass" : "one workgroup per transform", p.R, (long long)p.M1,
                 force_multipass() ? ", forced" : "");
    if (p.multipass) std::fprintf(stderr, ", %lld sequences per chunk", (long long)chunk_seqs_);
    std::fprintf(stderr, "\n");
}

// the calls on rows of whole 16-byte groups (N a multiple of 8), after validation
lconv_status_t filter_fft_aligned(const void* k, void* k_f, int64_t H, int64_t N, lconv_dtype_t dtype,
                                  void* workspace, hipStream_t stream);
lconv_status_t fftconv_fwd_aligned(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                   const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                   void* workspace, size_t chunk_target, bool may_build, hipStream_t stream);

bool tables_ready(const Plan1D& p, lconv_dtype_t dtype);

// Workspace of the forward call when the multi-pass chunks hold at most `target` bytes:
// staging (N not a multiple of 8) followed by one chunk.  0 if nothing is needed; SIZE_MAX for
// invalid arguments or when not even one sequence fits the target.
size_t fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, size_t target) {
    Plan1D p;
    int64_t seqs, rows;
    if (!dtype_ok(dtype) || B < 0 || H < 0 || !n_in_range(N) || !make_plan_1d(N, &p)) return SIZE_MAX;
    if (B == 0 || H == 0) return 0;
    if (!mul_ok(pairs_per_channel(B), H, &seqs) || !mul_ok(B, H, &rows)) return SIZE_MAX;
    const size_t stage = staging_bytes(rows, N, dtype, 4);  // u, q, v, y
    if (!p.multipass) return stage;
    const size_t csz = work_complex_size(dtype, false);
    if (target < (size_t)p.M * csz) return SIZE_MAX;
    return stage + (size_t)chunk_seqs(seqs, p.M, csz, target) * (size_t)p.M * csz;
}

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
    case LCONV_ERR_NOT_PREPARED: return "lconv_prepare was not called for this device, length and dtype";
    case LCONV_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the static buffer holds";
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
    const size_t w = fwd_workspace_bytes(B, H, N, dtype, kChunkTarget1D);
    return w == SIZE_MAX ? 0 : w;
}

size_t lconv_filter_fft2d_bytes(int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype) {
    int64_t t;
    if (!dtype_ok(dtype) || C < 0 || !sides2d_ok(Hs, Ws) || dtype == LCONV_F32) return 0;
    // spectrum of the 256 x 256 transform in the 2D kernel's order, complex in dtype
    if (!mul_ok(C, (int64_t)kP2D * kP2D, &t) || !mul_ok(t, 2 * (int64_t)dtype_size(dtype), &t)) return 0;
    return (size_t)t;
}

size_t lconv_fftconv2d_workspace_bytes(int64_t B, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype) {
    (void)B; (void)C; (void)Hs; (void)Ws; (void)dtype;
    return 0;  // one fused kernel per image pair: the intermediate stays in LDS
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
    return fftconv_fwd_call(u, k_f, D, y, q, v, B, H, N, dtype, workspace, workspace_bytes, kChunkTarget1D,
                            true, stream);
}

}  // extern "C"

namespace lcv {

lconv_status_t fftconv_fwd_call(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                void* workspace, size_t workspace_bytes, size_t chunk_target, bool may_build,
                                hipStream_t stream) {
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
    const size_t need = fwd_workspace_bytes(B, H, N, dtype, chunk_target);
    if (need == SIZE_MAX) return LCONV_ERR_WORKSPACE;
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
        // the tables first: without them (may_build false) nothing is launched
        Plan1D p8;
        make_plan_1d(N8, &p8);
        if (!may_build && !tables_ready(p8, dtype)) return LCONV_ERR_NOT_PREPARED;
        if (launch_pad_rows(u, su, rows, N, N8, esz, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (q && launch_pad_rows(q, sq, rows, N, N8, esz, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (v && launch_pad_rows(v, sv, rows, N, N8, esz, stream) != hipSuccess) return LCONV_ERR_HIP;
        const lconv_status_t r = fftconv_fwd_aligned(su, k_f, D, sy, sq, sv, B, H, N8, dtype, st + 4 * one,
                                                     chunk_target, may_build, stream);
        if (r != LCONV_SUCCESS) return r;
        return hip_status(launch_unpad_rows(sy, y, rows, N, N8, esz, stream));
    }
    return fftconv_fwd_aligned(u, k_f, D, y, q, v, B, H, N, dtype, workspace, chunk_target, may_build, stream);
}

size_t fftconv_fwd_staging_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype) {
    int64_t rows;
    if (!dtype_ok(dtype) || B < 0 || H < 0 || !n_in_range(N) || !mul_ok(B, H, &rows)) return 0;
    return staging_bytes(rows, N, dtype, 4);
}

lconv_status_t prepare_tables(int64_t N, lconv_dtype_t dtype) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (!n_in_range(N)) return LCONV_ERR_UNSUPPORTED;
    Plan1D p;
    make_plan_1d(round8(N), &p);
    hipError_t err = hipSuccess;
    if (!device_cu_count(&err)) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    if (!fused_tables(p.R, ct, &err)) return LCONV_ERR_HIP;
    if (p.multipass) {
        ColTables ctab;
        if (!col_tables(p.M, p.M1, &ctab, &err)) return LCONV_ERR_HIP;
        if (ct != CT_F32 && colmx_supported(p.M1) && !colmx_tables(p.M1, ct, &err)) return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

}  // namespace lcv

namespace {

// every constant table the forward call needs for plan p is built on the current device
bool tables_ready(const Plan1D& p, lconv_dtype_t dtype) {
    hipError_t err = hipSuccess;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    if (!fused_tables(p.R, ct, &err, false)) return false;
    if (!p.multipass) return true;
    ColTables ctab;
    if (!col_tables(p.M, p.M1, &ctab, &err, false)) return false;
    return ct == CT_F32 || !colmx_supported(p.M1) || colmx_tables(p.M1, ct, &err, false);
}

lconv_status_t fftconv_fwd_aligned(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                   const void* v, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                   void* workspace, size_t chunk_target, bool may_build, hipStream_t stream) {
    Plan1D p;
    make_plan_1d(N, &p);
    if (!may_build && !tables_ready(p, dtype)) return LCONV_ERR_NOT_PREPARED;
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const void* tabs = fused_tables(p.R, ct, &err, may_build);
    if (!tabs) return LCONV_ERR_HIP;
    const int64_t Bp = pairs_per_channel(B), seqs = Bp * H;
    log_plan("fftconv_fwd", B, H, N, dtype, p,
             p.multipass ? chunk_seqs(seqs, p.M, work_complex_size(dtype, false), chunk_target) : 0);
    if (!p.multipass) {
        Fused1DArgs a{};
        a.u = u; a.q = q; a.v = v; a.y = y; a.kf = k_f; a.D = D; a.tables = tabs;
        a.B = B; a.H = H; a.N = N; a.nitems = seqs;
        a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = 1;
        return hip_status(launch_fused1d(p.R, dtype, MODE_CONV, q != nullptr, v != nullptr, a, cus, stream));
    }
    ColTables ctab;
    if (!col_tables(p.M, p.M1, &ctab, &err, may_build)) return LCONV_ERR_HIP;
    const void* cimg = nullptr;  // matrix-core column images (16-bit long columns)
    if (ct != CT_F32 && colmx_supported(p.M1)) {
        cimg = colmx_tables(p.M1, ct, &err, may_build);
        if (!cimg) return LCONV_ERR_HIP;
    }
    const size_t csz = work_complex_size(dtype, false);
    // One real row per sequence (B = 1) on the matrix-core passes: a real column's spectrum is
    // conjugate-symmetric in k_hi, so only rows 0 .. M1/2 are stored and row-transformed (the
    // filter and the output are real as well); the inverse column pass rebuilds the rest.
    const bool half = B == 1 && cimg && p.M1 >= 256;
    const int64_t rows = half ? p.M1 / 2 + 1 : p.M1;
    const int64_t full_per = chunk_seqs(seqs, p.M, csz, chunk_target);
    // as many sequences as the workspace sized for full rows holds
    const int64_t per = half ? chunk_seqs(seqs, rows * kRowLen, csz, (size_t)full_per * p.M * csz) : full_per;
    // equal chunks (sizes differ by at most one sequence), not full chunks and a short last one
    const int64_t nch = (seqs + per - 1) / per;
    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t s0 = seqs / nch * ci + (ci < seqs % nch ? ci : seqs % nch);
        const int64_t ns = seqs / nch + (ci < seqs % nch ? 1 : 0);
        ColArgs c{};
        c.u = u; c.q = q; c.v = v; c.y = y; c.ws = workspace;
        c.tw_lo = ctab.lo; c.tw_hi = ctab.hi; c.tw_col = ctab.col;
        c.B = B; c.H = H; c.N = N; c.M = p.M; c.M1 = p.M1; c.seq0 = s0; c.nseq = ns;
        c.seq_per_h = Bp; c.filter = 0; c.img = cimg; c.rows = rows;
        if (launch_col_fwd(dtype, c, stream) != hipSuccess) return LCONV_ERR_HIP;
        Fused1DArgs a{};
        a.u = workspace; a.y = workspace; a.kf = k_f; a.D = D; a.tables = tabs;
        a.nitems = ns * rows; a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = p.M1; a.wrows = rows;
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
    if (!n_supported(N) || !make_plan_1d(N, &p) || p.multipass) return 0;
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

// ---- learned Butterfly --------------------------------------------------------------------

namespace {

// fused plan for a learned-Butterfly call (R), or 0 when N is not served by one workgroup
int bfly_radix(int64_t N) {
    Plan1D p;
    if (!n_supported(N) || !make_plan_1d(N, &p) || p.multipass) return 0;
    return p.R;
}

size_t bfly_conv_offset(int R, lconv_dtype_t dtype) {
    return dtype == LCONV_F32 ? 0 : fused_table_layout(R, CT_F32).total;
}

}  // namespace

int64_t lconv_butterfly_blocks_count(int64_t N) {
    const int R = bfly_radix(N);
    return R ? 2 * (int64_t)R * R + 4 * 256 * (int64_t)R : 0;
}

size_t lconv_butterfly_tables_bytes(int64_t N, lconv_dtype_t dtype) {
    if (!dtype_ok(dtype)) return 0;
    const int R = bfly_radix(N);
    if (!R) return 0;
    return bfly_conv_offset(R, dtype) + fused_table_layout(R, (int)dtype).total;
}

lconv_status_t lconv_butterfly_tables(const void* blocks, void* tables, int64_t N, lconv_dtype_t dtype,
                                      hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (N < 1) return LCONV_ERR_INVALID_SHAPE;
    const int R = bfly_radix(N);
    if (!R) return LCONV_ERR_UNSUPPORTED;
    if (!blocks || !tables) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(blocks) || !aligned16(tables)) return LCONV_ERR_MISALIGNED;
    const size_t nb = (size_t)lconv_butterfly_blocks_count(N) * 8, nt = lconv_butterfly_tables_bytes(N, dtype);
    if (overlap(blocks, nb, tables, nt)) return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const void* plan = fused_tables(R, CT_F32, &err);  // for its fixed twiddle section
    if (!plan) return LCONV_ERR_HIP;
    const FusedTableLayout L32 = fused_table_layout(R, CT_F32);
    // fp32 images (the filter transform), then the compute-type images (the convolution)
    const size_t offs[2] = {0, bfly_conv_offset(R, dtype)};
    const int cts[2] = {CT_F32, (int)dtype};
    for (int i = 0; i < (dtype == LCONV_F32 ? 1 : 2); ++i) {
        const FusedTableLayout L = fused_table_layout(R, cts[i]);
        char* out = (char*)tables + offs[i];
        if (launch_bfly_images(blocks, out, R, cts[i], L, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (hipMemcpyAsync(out + L.tw, (const char*)plan + L32.tw, 64 * 4 * 8, hipMemcpyDeviceToDevice, stream) !=
            hipSuccess)
            return LCONV_ERR_HIP;
    }
    return LCONV_SUCCESS;
}

lconv_status_t lconv_butterfly_filter(const void* k, void* k_f, const void* tables, int64_t H, int64_t N,
                                      lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    if (H == 0 || N == 0) return LCONV_SUCCESS;
    const int R = bfly_radix(N);
    if (!R) return LCONV_ERR_UNSUPPORTED;
    if (!k || !k_f || !tables) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(k) || !aligned16(k_f) || !aligned16(tables)) return LCONV_ERR_MISALIGNED;
    int64_t elems;
    if (!mul_ok(H, N, &elems)) return LCONV_ERR_INVALID_SHAPE;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(k_f, kf_bytes, k, (size_t)elems * dtype_size(dtype)) ||
        overlap(k_f, kf_bytes, tables, lconv_butterfly_tables_bytes(N, dtype)))
        return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int64_t M = 256 * (int64_t)R;
    Fused1DArgs a{};
    a.u = k; a.y = k_f; a.tables = tables;  // the fp32 images come first
    a.B = 1; a.H = H; a.N = N; a.nitems = H;
    a.inv_m = 1.0f / (float)M; a.M = M; a.M1 = 1;
    return hip_status(launch_fused1d(R, dtype, MODE_FILTER, false, false, a, cus, stream));
}

lconv_status_t lconv_butterfly_fwd(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                   const void* v, const void* tables, int64_t B, int64_t H, int64_t N,
                                   lconv_dtype_t dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    const int R = bfly_radix(N);
    if (!R) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y || !tables) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y) || !aligned16(tables) ||
        (q && !aligned16(q)) || (v && !aligned16(v)))
        return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, N, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(y, act, u, act) || overlap(y, act, q, act) || overlap(y, act, v, act) ||
        overlap(y, act, k_f, kf_bytes) || overlap(y, act, D, (size_t)H * es) ||
        overlap(y, act, tables, lconv_butterfly_tables_bytes(N, dtype)))
        return LCONV_ERR_ALIASING;
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const int64_t M = 256 * (int64_t)R;
    Fused1DArgs a{};
    a.u = u; a.q = q; a.v = v; a.y = y; a.kf = k_f; a.D = D;
    a.tables = (const char*)tables + bfly_conv_offset(R, dtype);
    a.B = B; a.H = H; a.N = N; a.nitems = B * H;  // one real row per transform
    a.inv_m = 1.0f / (float)M; a.M = M; a.M1 = 1;
    return hip_status(launch_fused1d(R, dtype, MODE_LBF, q != nullptr, v != nullptr, a, cus, stream));
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
    if (!mul_ok(B, nch, &nseq) || !mul_ok(nseq / 2 + (nseq & 1), H, &items) || nseq >= ((int64_t)1 << 32) ||
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
// Workspace of the gradient for sequences past one workgroup (zero otherwise), in 256-byte
// aligned parts: the forward call's chunk workspace (for [B][H] and for [1][B*H] rows), rev(ds),
// the forward results, x = q (.) u, the rows' spectra with their transform workspace, and the
// zero skip of the row filters.
struct BwdLongLayout {
    size_t fws, ds, t, xs, kf, kfws, zd, part;
    size_t o_ds, o_t, o_xs, o_kf, o_kfws, o_zd, o_part, total;
};

bool bwd_long_layout(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, BwdLongLayout* L) {
    int64_t rows, elems;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, N, &elems) || rows == 0) return false;
    const size_t es = dtype_size(dtype), act = round256((size_t)elems * es);
    const size_t f1 = fwd_workspace_bytes(B, H, N, dtype, kChunkTarget1D);
    const size_t f2 = fwd_workspace_bytes(1, rows, N, dtype, kChunkTarget1D);
    const size_t kf = lconv_filter_fft_bytes(rows, N, dtype);
    if (f1 == SIZE_MAX || f2 == SIZE_MAX || kf == 0) return false;
    L->fws = round256(f1 > f2 ? f1 : f2);
    L->ds = L->t = L->xs = act;
    L->kf = round256(kf);
    L->kfws = round256(lconv_filter_fft_workspace_bytes(rows, N, dtype));
    L->zd = round256((size_t)rows * es);
    L->part = round256((size_t)H * dot_slices(N) * sizeof(float));
    L->o_ds = L->fws;
    L->o_t = L->o_ds + L->ds;
    L->o_xs = L->o_t + L->t;
    L->o_kf = L->o_xs + L->xs;
    L->o_kfws = L->o_kf + L->kf;
    L->o_zd = L->o_kfws + L->kfws;
    L->o_part = L->o_zd + L->zd;
    L->total = L->o_part + L->part;
    return true;
}

// Spectra of the rows x = q (.) u (u alone without q), each the filter of a channel of its own,
// for the filter gradient of long sequences: in the 16-bit compute type, through the forward
// column pass on the matrix cores (gated there) and the row transform.  With M1 >= 256 (two rows
// per workgroup) only the rows k_hi <= M1/2 are formed: the half-row row pass of the
// one-row-per-sequence call that follows reads no others.  false: not this path (fp32, or column
// lengths below 16); the caller then takes lconv_filter_fft.
bool row_spectra16(const void* u, const void* q, void* kf, int64_t rows, int64_t N, lconv_dtype_t dtype,
                   void* workspace, hipStream_t stream, lconv_status_t* st) {
    if (dtype == LCONV_F32) return false;
    Plan1D p;
    make_plan_1d(N, &p);
    if (!p.multipass || !colmx_supported(p.M1)) return false;
    *st = LCONV_ERR_HIP;
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return true;
    const int ct = (int)dtype;
    const void* tabs = fused_tables(32, ct, &err);
    const void* cimg = colmx_tables(p.M1, ct, &err);
    ColTables ctab;
    if (!tabs || !cimg || !col_tables(p.M, p.M1, &ctab, &err)) return true;
    // the chunks of a one-row-per-sequence forward call over these rows (its workspace size)
    const size_t csz = work_complex_size(dtype, false);
    const bool half = p.M1 >= 256;
    const int64_t wr = half ? p.M1 / 2 + 1 : p.M1;
    const int64_t full_per = chunk_seqs(rows, p.M, csz, kChunkTarget1D);
    const int64_t per = half ? chunk_seqs(rows, wr * kRowLen, csz, (size_t)full_per * p.M * csz) : full_per;
    const int64_t nch = (rows + per - 1) / per;
    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t s0 = rows / nch * ci + (ci < rows % nch ? ci : rows % nch);
        const int64_t ns = rows / nch + (ci < rows % nch ? 1 : 0);
        ColArgs c{};
        c.u = u; c.q = q; c.ws = workspace;
        c.tw_lo = ctab.lo; c.tw_hi = ctab.hi; c.tw_col = ctab.col;
        c.B = 1; c.H = rows; c.N = N; c.M = p.M; c.M1 = p.M1; c.seq0 = s0; c.nseq = ns;
        c.seq_per_h = 1; c.filter = 0; c.img = cimg; c.rows = wr;
        if (launch_col_fwd(dtype, c, stream) != hipSuccess) return true;
        Fused1DArgs a{};
        a.u = workspace; a.y = kf; a.tables = tabs;
        a.nitems = ns * wr; a.inv_m = 1.0f / (float)p.M; a.M = p.M; a.M1 = p.M1; a.wrows = wr;
        a.seq0 = s0; a.seq_per_h = 1;
        if (launch_fused1d(32, dtype, MODE_ROWFWD16, false, false, a, cus, stream) != hipSuccess) return true;
    }
    *st = LCONV_SUCCESS;
    return true;
}

// dk, dD of a long sequence, from rev(ds) already in the workspace part L.o_ds: each row's
// x = q (.) u as a filter of its own (B*H channels of one row each), applied to rev(ds) with a
// zero skip, then reversed and summed over the batch; the part L.o_t is overwritten.
lconv_status_t dk_long(const void* dy, const void* u, const void* q, const void* v, float* dk, float* dD,
                       int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, void* workspace,
                       const BwdLongLayout& L, hipStream_t stream) {
    char* w = (char*)workspace;
    void *fws = w, *ds = w + L.o_ds, *t = w + L.o_t, *xs = w + L.o_xs, *kf = w + L.o_kf, *kfws = w + L.o_kfws,
         *zd = w + L.o_zd;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const int64_t rows = B * H, elems = rows * N;
    lconv_status_t st;
    if (!row_spectra16(u, q, kf, rows, N, dtype, fws, stream, &st)) {
        const void* x = u;
        if (q) {
            if (launch_mul_rows(q, u, xs, elems, ct, stream) != hipSuccess) return LCONV_ERR_HIP;
            x = xs;
        }
        st = lconv_filter_fft(x, kf, rows, N, dtype, kfws, L.kfws, stream);
    }
    if (st != LCONV_SUCCESS) return st;
    if (launch_zero_words(zd, (int64_t)(L.zd / 4), stream) != hipSuccess) return LCONV_ERR_HIP;
    st = fftconv_fwd_call(ds, kf, zd, t, nullptr, nullptr, 1, rows, N, dtype, fws, L.fws, kChunkTarget1D, true,
                          stream);
    if (st != LCONV_SUCCESS) return st;
    if (launch_rev_batch_sum(t, dk, dD, B, H, N, ct, stream) != hipSuccess) return LCONV_ERR_HIP;
    // lag 0 again, as the direct fp32 sum: the correlation's rows pass through memory in the
    // dtype, and at lag 0 their batch sum can cancel
    if (launch_dot_lag0(u, q, dy, v, (float*)(w + L.o_part), dk, dD, B, H, N, ct, stream) != hipSuccess)
        return LCONV_ERR_HIP;
    return LCONV_SUCCESS;
}

// The gradient of a long sequence through the multi-pass forward call.  Reversing a row turns a
// correlation over later positions into a causal convolution:
//   dx = rev(k * rev(ds)) + D ds            (ds = dy (.) v);  du = q (.) dx, dq = u (.) dx
//   dk[h][t] = sum_b (x_b * rev(ds_b))[N-1-t]   with x_b = q (.) u the filter of row b
// so every transform is the forward path's; the reversals and gates are elementwise passes.
lconv_status_t bwd_long(const void* dy, const void* u, const void* k_f, const void* D, const void* q,
                        const void* v, const void* c, void* du, void* dq, void* dv, float* dk, float* dD,
                        int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, void* workspace,
                        hipStream_t stream) {
    BwdLongLayout L;
    bwd_long_layout(B, H, N, dtype, &L);
    char* w = (char*)workspace;
    void *fws = w, *ds = w + L.o_ds, *t = w + L.o_t;
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const int64_t rows = B * H, elems = rows * N;
    lconv_status_t st;
    // dv = dy (.) (k * x + D x)
    if (v && c) {
        if (launch_mul_rows(dy, c, dv, elems, ct, stream) != hipSuccess) return LCONV_ERR_HIP;
    } else if (v) {
        st = fftconv_fwd_call(u, k_f, D, dv, q, dy, B, H, N, dtype, fws, L.fws, kChunkTarget1D, true, stream);
        if (st != LCONV_SUCCESS) return st;
    }
    // rev(ds), then t = k * rev(ds) + D rev(ds), then du = q (.) rev(t), dq = u (.) rev(t)
    if (launch_rev_gate(dy, v, ds, rows, N, ct, stream) != hipSuccess) return LCONV_ERR_HIP;
    st = fftconv_fwd_call(ds, k_f, D, t, nullptr, nullptr, B, H, N, dtype, fws, L.fws, kChunkTarget1D, true, stream);
    if (st != LCONV_SUCCESS) return st;
    if (launch_rev_gated_out(t, q, q ? u : nullptr, du, q ? dq : nullptr, rows, N, ct, stream) != hipSuccess)
        return LCONV_ERR_HIP;
    if (dk || dD) return dk_long(dy, u, q, v, dk, dD, B, H, N, dtype, workspace, L, stream);
    return LCONV_SUCCESS;
}

lconv_status_t bwd_impl(const void* dy, const void* u, const void* k_f, const void* D, const void* q,
                        const void* v, const void* c, void* du, void* dq, void* dv, float* dk, float* dD,
                        int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t, hn;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t) || !mul_ok(H, N, &hn) ||
        !mul_ok(hn, 8, &t))
        return LCONV_ERR_INVALID_SHAPE;
    if (H == 0 || N == 0) return LCONV_SUCCESS;
    if (!n_supported(N)) return LCONV_ERR_UNSUPPORTED;
    if (!q) dq = nullptr;  // ignored without the gate it belongs to
    if (!v) dv = nullptr;
    if (B == 0) {          // empty batch: the filter gradients are zero sums
        if ((dk && !aligned16(dk)) || (dD && !aligned16(dD))) return LCONV_ERR_MISALIGNED;
        // a fill kernel, not a memset node: the call stays safe to capture in a graph
        if (dk && launch_zero_words(dk, hn, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (dD && launch_zero_words(dD, H, stream) != hipSuccess) return LCONV_ERR_HIP;
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
    if (p.multipass) {
        const size_t need = lconv_fftconv_bwd_workspace_bytes(B, H, N, dtype);
        if (need == 0) return LCONV_ERR_INVALID_SHAPE;
        if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
        for (int i = 0; i < 7; ++i)
            if (overlap(workspace, need, ins[i], in_sz[i])) return LCONV_ERR_ALIASING;
        for (int o = 0; o < 5; ++o)
            if (overlap(workspace, need, outs[o], out_sz[o])) return LCONV_ERR_ALIASING;
        return bwd_long(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype, workspace, stream);
    }
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

// Workspace of the partial convolution's gradient, in 256-byte aligned parts: rev(ds) and the
// convolution result t (inside the long-sequence layout when N needs the multi-pass path, whose
// filter-gradient parts follow), then the full-length filter gradient [H][N] fp32.
struct PartBwdLayout {
    size_t o_ds, o_t, o_dkf, total;
    bool lng;
    BwdLongLayout L;
};

bool part_bwd_layout(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype, PartBwdLayout* P) {
    int64_t rows, elems, hn;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, N, &elems) || !mul_ok(H, N, &hn) || rows == 0 || N == 0)
        return false;
    Plan1D p;
    if (!make_plan_1d(N, &p)) return false;
    P->lng = p.multipass;
    const size_t act = round256((size_t)elems * dtype_size(dtype));
    if (P->lng) {
        if (!bwd_long_layout(B, H, N, dtype, &P->L)) return false;
        P->o_ds = P->L.o_ds;
        P->o_t = P->L.o_t;
        P->o_dkf = P->L.total;
    } else {
        P->o_ds = 0;
        P->o_t = act;
        P->o_dkf = 2 * act;
    }
    P->total = P->o_dkf + round256((size_t)hn * sizeof(float));
    return true;
}

// Gradients of the partial convolution.  The filter has L taps, so the correlations keep the
// banded structure of the forward call:
//   dv = dy (.) (k * x + D x)                 the partial forward gated by dy
//   dx = rev(k * rev(ds)) + D ds              the partial forward on time-reversed rows
//   dk[h][tau] = the full-length correlation's lag tau < min(L, N) (zero for tau >= N)
// The last comes from the full-length filter gradient (one fused launch for N <= 4096, the
// multi-pass correlations past that), of which the first L lags are kept.
lconv_status_t partial_bwd_impl(const void* dy, const void* u, const void* k_f, const void* D, const void* q,
                                const void* v, void* du, void* dq, void* dv, float* dk, float* dD, int64_t B,
                                int64_t H, int64_t N, int64_t L, lconv_dtype_t dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0 || L < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t, hl;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t) || !mul_ok(H, L, &hl) ||
        !mul_ok(hl, 8, &t) || !mul_ok(H, N, &t) || !mul_ok(t, 8, &t))
        return LCONV_ERR_INVALID_SHAPE;
    if (H == 0) return LCONV_SUCCESS;
    if (L < 8 || L > 4096 || (L % 8) != 0 || (N % 8) != 0 || (N > 0 && !n_supported(N)))
        return LCONV_ERR_UNSUPPORTED;
    Plan1D pl;
    if (!make_plan_1d(L, &pl) || pl.multipass) return LCONV_ERR_UNSUPPORTED;
    if (!q) dq = nullptr;  // ignored without the gate it belongs to
    if (!v) dv = nullptr;
    if (B == 0 || N == 0) {  // no pair of positions: the filter gradients are zero sums
        if ((dk && !aligned16(dk)) || (dD && !aligned16(dD))) return LCONV_ERR_MISALIGNED;
        if (dk && launch_zero_words(dk, hl, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (dD && launch_zero_words(dD, H, stream) != hipSuccess) return LCONV_ERR_HIP;
        return LCONV_SUCCESS;
    }
    if (!dy || !u || !k_f || !D || !du || (q && !dq) || (v && !dv)) return LCONV_ERR_NULL_POINTER;
    const void* ptrs[] = {dy, u, k_f, D, q, v, du, dq, dv, dk, dD, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const size_t kf_bytes = lconv_filter_fft_bytes(H, L, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    PartBwdLayout P;
    if (!part_bwd_layout(B, H, N, dtype, &P)) return LCONV_ERR_INVALID_SHAPE;
    if (!workspace || workspace_bytes < P.total) return LCONV_ERR_WORKSPACE;
    const void* ins[] = {dy, u, k_f, D, q, v};
    const size_t in_sz[] = {act, act, kf_bytes, (size_t)H * es, act, act};
    const void* outs[] = {du, dq, dv, dk, dD, workspace};
    const size_t out_sz[] = {act, act, act, (size_t)hl * 4, (size_t)H * 4, P.total};
    for (int o = 0; o < 6; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[o], out_sz[o], ins[i], in_sz[i])) return LCONV_ERR_ALIASING;
        for (int o2 = o + 1; o2 < 6; ++o2)
            if (overlap(outs[o], out_sz[o], outs[o2], out_sz[o2])) return LCONV_ERR_ALIASING;
    }
    char* w = (char*)workspace;
    void *ds = w + P.o_ds, *tt = w + P.o_t;
    float* dkf = (float*)(w + P.o_dkf);
    const int ct = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
    const int64_t rows = B * H;
    lconv_status_t st;
    if (v) {
        st = partial_impl(u, k_f, D, dv, q, dy, B, H, N, L, dtype, 0, stream);
        if (st != LCONV_SUCCESS) return st;
    }
    if (launch_rev_gate(dy, v, ds, rows, N, ct, stream) != hipSuccess) return LCONV_ERR_HIP;
    st = partial_impl(ds, k_f, D, tt, nullptr, nullptr, B, H, N, L, dtype, 0, stream);
    if (st != LCONV_SUCCESS) return st;
    if (launch_rev_gated_out(tt, q, q ? u : nullptr, du, q ? dq : nullptr, rows, N, ct, stream) != hipSuccess)
        return LCONV_ERR_HIP;
    if (!dk && !dD) return LCONV_SUCCESS;
    if (P.lng) {
        st = dk_long(dy, u, q, v, dkf, dD, B, H, N, dtype, workspace, P.L, stream);
        if (st != LCONV_SUCCESS) return st;
    } else {
        hipError_t err = hipSuccess;
        const int cus = device_cu_count(&err);
        if (!cus) return LCONV_ERR_HIP;
        Plan1D pn;
        make_plan_1d(N, &pn);
        const void* tabs = fused_tables(pn.R, ct, &err);
        if (!tabs) return LCONV_ERR_HIP;
        Fused1DArgs a{};
        a.u = u; a.q = q; a.e2 = dy; a.v = v; a.y = dkf; a.y2 = dD; a.tables = tabs;
        a.B = B; a.H = H; a.N = N; a.nitems = H;
        a.inv_m = 1.0f / (float)pn.M; a.M = pn.M; a.M1 = 1;
        if (launch_dk1d(pn.R, dtype, q != nullptr, v != nullptr, a, cus, stream) != hipSuccess)
            return LCONV_ERR_HIP;
    }
    if (dk && launch_copy_cols(dkf, dk, H, N, L, stream) != hipSuccess) return LCONV_ERR_HIP;
    return LCONV_SUCCESS;
}

}  // namespace

extern "C" {

size_t lconv_fftconv_partial_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype) {
    if (!dtype_ok(dtype) || B <= 0 || H <= 0 || N <= 0 || (N % 8) != 0 || !n_supported(N)) return 0;
    PartBwdLayout P;
    return part_bwd_layout(B, H, N, dtype, &P) ? P.total : 0;
}

lconv_status_t lconv_fftconv_partial_bwd(const void* dy, const void* u, const void* k_f, const void* D,
                                         const void* q, const void* v, void* du, void* dq, void* dv, float* dk,
                                         float* dD, int64_t B, int64_t H, int64_t N, int64_t L,
                                         lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    return partial_bwd_impl(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, L, dtype, workspace,
                            workspace_bytes, stream);
}

size_t lconv_fftconv_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype) {
    Plan1D p;
    if (!dtype_ok(dtype) || B < 0 || H < 0 || !n_supported(N) || !make_plan_1d(N, &p)) return 0;
    if (!p.multipass || B == 0 || H == 0) return 0;
    BwdLongLayout L;
    return bwd_long_layout(B, H, N, dtype, &L) ? L.total : 0;
}

lconv_status_t lconv_fftconv_bwd(const void* dy, const void* u, const void* k_f, const void* D, const void* q,
                                 const void* v, void* du, void* dq, void* dv, float* dk, float* dD, int64_t B,
                                 int64_t H, int64_t N, lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    return bwd_impl(dy, u, k_f, D, q, v, nullptr, du, dq, dv, dk, dD, B, H, N, dtype, workspace, workspace_bytes,
                    stream);
}

lconv_status_t lconv_fftconv_bwd_saved(const void* dy, const void* u, const void* k_f, const void* D,
                                       const void* q, const void* v, const void* c, void* du, void* dq, void* dv,
                                       float* dk, float* dD, int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!c && v && B > 0 && H > 0 && N > 0) return LCONV_ERR_NULL_POINTER;
    return bwd_impl(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype, workspace, workspace_bytes,
                    stream);
}

lconv_status_t lconv_fftconv_fwd_save(const void* u, const void* k_f, const void* D, void* y, void* c,
                                      const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                      lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &elems) || !mul_ok(elems, 8, &t)) return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || H == 0 || N == 0) return LCONV_SUCCESS;
    if (!n_supported(N)) return LCONV_ERR_UNSUPPORTED;
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
    if (p.multipass) {
        // the multi-pass forward without the post-gate gives c; y = v (.) c (or a copy of c)
        const size_t need = lconv_fftconv_workspace_bytes(B, H, N, dtype);
        if (!workspace || workspace_bytes < need) return LCONV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LCONV_ERR_MISALIGNED;
        for (int i = 0; i < 5; ++i)
            if (overlap(workspace, need, ins[i], in_sz[i])) return LCONV_ERR_ALIASING;
        if (overlap(workspace, need, y, act) || overlap(workspace, need, c, act)) return LCONV_ERR_ALIASING;
        const lconv_status_t st = fftconv_fwd_call(u, k_f, D, c, q, nullptr, B, H, N, dtype, workspace,
                                                   workspace_bytes, kChunkTarget1D, true, stream);
        if (st != LCONV_SUCCESS) return st;
        const int ctv = dtype == LCONV_F32 ? CT_F32 : (int)dtype;
        if (v) return hip_status(launch_mul_rows(c, v, y, elems, ctv, stream));
        return hip_status(hipMemcpyAsync(y, c, act, hipMemcpyDeviceToDevice, stream));
    }
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

lconv_status_t lconv_filter_fft2d(const void* k, void* k_f, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype,
                                  hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (C < 0 || Hs < 0 || Ws < 0) return LCONV_ERR_INVALID_SHAPE;
    if (C == 0) return LCONV_SUCCESS;
    if (!sides2d_ok(Hs, Ws) || dtype == LCONV_F32) return LCONV_ERR_UNSUPPORTED;
    if (!k || !k_f) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(k) || !aligned16(k_f)) return LCONV_ERR_MISALIGNED;
    const size_t kf_bytes = lconv_filter_fft2d_bytes(C, Hs, Ws, dtype);
    if (kf_bytes == 0) return LCONV_ERR_INVALID_SHAPE;
    if (overlap(k_f, kf_bytes, k, (size_t)(C * Hs * Ws) * dtype_size(dtype))) return LCONV_ERR_ALIASING;
    Conv2DArgs a{};
    a.u = k; a.kf = k_f; a.C = C; a.B = 1; a.filter = 1;
    a.Hs = (int)Hs; a.Ws = (int)Ws;
    a.inv_p2 = 1.0f / (float)(kP2D * kP2D);
    return hip_status(launch_conv2d(dtype, a, stream));
}

lconv_status_t lconv_fftconv2d_fwd(const void* u, const void* k_f, const void* D, void* y, int64_t B, int64_t C,
                                   int64_t Hs, int64_t Ws, lconv_dtype_t dtype, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    (void)workspace; (void)workspace_bytes;  // lconv_fftconv2d_workspace_bytes is 0: nothing to check
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || C < 0 || Hs < 0 || Ws < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t elems, t;
    if (!mul_ok(B, C, &t) || !mul_ok(Hs, Ws, &elems) || !mul_ok(t, elems, &elems) || !mul_ok(elems, 8, &t))
        return LCONV_ERR_INVALID_SHAPE;
    if (B == 0 || C == 0) return LCONV_SUCCESS;
    if (!sides2d_ok(Hs, Ws) || dtype == LCONV_F32) return LCONV_ERR_UNSUPPORTED;
    if (!u || !k_f || !D || !y) return LCONV_ERR_NULL_POINTER;
    if (!aligned16(u) || !aligned16(k_f) || !aligned16(D) || !aligned16(y)) return LCONV_ERR_MISALIGNED;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    if (overlap(y, act, u, act) || overlap(y, act, k_f, lconv_filter_fft2d_bytes(C, Hs, Ws, dtype)) ||
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
    a.Hs = (int)Hs; a.Ws = (int)Ws;
    a.inv_p2 = 1.0f / (float)(kP2D * kP2D);
    return hip_status(launch_conv2d(dtype, a, stream));
}

}  // extern "C"

namespace {

// Workspace of the 2D gradient, in 256-byte aligned parts: the adjoint spectrum [C], the
// spectra of the rotated output gradients [B*C], their convolutions with u [B*C][Hs][Ws] and a
// zero skip [B*C] (dtype).
struct Bwd2DLayout {
    size_t o_ka, o_kd, o_r, o_zd, total;
};

bool bwd2d_layout(int64_t B, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype, Bwd2DLayout* L) {
    int64_t bc, elems;
    if (!mul_ok(B, C, &bc) || !mul_ok(bc, Hs * Ws, &elems) || bc == 0) return false;
    const size_t ka = lconv_filter_fft2d_bytes(C, Hs, Ws, dtype), kd = lconv_filter_fft2d_bytes(bc, Hs, Ws, dtype);
    if (ka == 0 || kd == 0) return false;
    const size_t es = dtype_size(dtype);
    L->o_ka = 0;
    L->o_kd = round256(ka);
    L->o_r = L->o_kd + round256(kd);
    L->o_zd = L->o_r + round256((size_t)elems * es);
    L->total = L->o_zd + round256((size_t)bc * es);
    return true;
}

}  // namespace

extern "C" {

size_t lconv_fftconv2d_bwd_workspace_bytes(int64_t B, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype) {
    if (!dtype_ok(dtype) || dtype == LCONV_F32 || B <= 0 || C <= 0 || !sides2d_ok(Hs, Ws)) return 0;
    Bwd2DLayout L;
    return bwd2d_layout(B, C, Hs, Ws, dtype, &L) ? L.total : 0;
}

lconv_status_t lconv_fftconv2d_bwd(const void* dy, const void* u, const void* k_f, const void* D, void* du,
                                   float* dk, float* dD, int64_t B, int64_t C, int64_t Hs, int64_t Ws,
                                   lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    if (!dtype_ok(dtype)) return LCONV_ERR_UNSUPPORTED;
    if (B < 0 || C < 0 || Hs < 0 || Ws < 0) return LCONV_ERR_INVALID_SHAPE;
    int64_t img, elems, t;
    if (!mul_ok(Hs, Ws, &img) || !mul_ok(B, C, &t) || !mul_ok(t, img, &elems) || !mul_ok(elems, 8, &t) ||
        !mul_ok(C, img, &t) || !mul_ok(t, 8, &t))
        return LCONV_ERR_INVALID_SHAPE;
    if (C == 0) return LCONV_SUCCESS;
    if (!sides2d_ok(Hs, Ws) || dtype == LCONV_F32) return LCONV_ERR_UNSUPPORTED;
    if (B == 0) {  // empty batch: the filter gradients are zero sums
        if ((dk && !aligned16(dk)) || (dD && !aligned16(dD))) return LCONV_ERR_MISALIGNED;
        if (dk && launch_zero_words(dk, C * img, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (dD && launch_zero_words(dD, C, stream) != hipSuccess) return LCONV_ERR_HIP;
        return LCONV_SUCCESS;
    }
    if (!dy || !u || !k_f || !D || !du) return LCONV_ERR_NULL_POINTER;
    const void* ptrs[] = {dy, u, k_f, D, du, dk, dD, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return LCONV_ERR_MISALIGNED;
    Bwd2DLayout L;
    if (!bwd2d_layout(B, C, Hs, Ws, dtype, &L)) return LCONV_ERR_INVALID_SHAPE;
    if (!workspace || workspace_bytes < L.total) return LCONV_ERR_WORKSPACE;
    const size_t es = dtype_size(dtype), act = (size_t)elems * es;
    const void* ins[] = {dy, u, k_f, D};
    const size_t in_sz[] = {act, act, lconv_filter_fft2d_bytes(C, Hs, Ws, dtype), (size_t)C * es};
    const void* outs[] = {du, dk, dD, workspace};
    const size_t out_sz[] = {act, (size_t)(C * img) * 4, (size_t)C * 4, L.total};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[o], out_sz[o], ins[i], in_sz[i])) return LCONV_ERR_ALIASING;
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlap(outs[o], out_sz[o], outs[o2], out_sz[o2])) return LCONV_ERR_ALIASING;
    }
    hipError_t err = hipSuccess;
    const int cus = device_cu_count(&err);
    if (!cus) return LCONV_ERR_HIP;
    const void* tabs = fused_tables(1, (int)dtype, &err);  // 256-point transform blocks
    if (!tabs) return LCONV_ERR_HIP;
    char* w = (char*)workspace;
    // du = the forward convolution of dy with the adjoint spectrum (same D)
    if (launch_adj2d(k_f, w + L.o_ka, C, stream) != hipSuccess) return LCONV_ERR_HIP;
    Conv2DArgs a{};
    a.u = dy; a.kf = w + L.o_ka; a.D = D; a.y = du; a.tables = tabs;
    a.B = B; a.C = C; a.filter = 0; a.cus = cus;
    a.Hs = (int)Hs; a.Ws = (int)Ws;
    a.inv_p2 = 1.0f / (float)(kP2D * kP2D);
    if (launch_conv2d(dtype, a, stream) != hipSuccess) return LCONV_ERR_HIP;
    if (dk) {
        // per image, dk_b[a][e] = (u_b conv rot(dy_b))[Hs-1-a][Ws-1-e]: the B*C images as channels
        // of one image each, with the rotated dy as their filters and a zero skip
        const int64_t bc = B * C;
        Conv2DArgs f = a;   // the 2D kernel's row and column transforms in spectrum mode
        f.u = dy; f.kf = nullptr; f.D = nullptr; f.y = w + L.o_kd; f.B = 1; f.C = bc; f.spec = 1;
        if (launch_conv2d(dtype, f, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (launch_zero_words(w + L.o_zd, (int64_t)((bc * es + 3) / 4), stream) != hipSuccess) return LCONV_ERR_HIP;
        Conv2DArgs c = a;
        c.u = u; c.kf = w + L.o_kd; c.D = w + L.o_zd; c.y = w + L.o_r; c.B = 1; c.C = bc;
        if (launch_conv2d(dtype, c, stream) != hipSuccess) return LCONV_ERR_HIP;
        if (launch_dk2d_sum((int)dtype, w + L.o_r, dk, B, C, (int)Hs, (int)Ws, stream) != hipSuccess)
            return LCONV_ERR_HIP;
    }
    if (dD && launch_dd2d((int)dtype, dy, u, dD, B, C, img, stream) != hipSuccess) return LCONV_ERR_HIP;
    return LCONV_SUCCESS;
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
    // 16-bit S = 32: the matrix-core passes (dense 64-point DFT blocks)
    const void* img = nullptr;
    if (S == 32 && dtype != LCONV_F32) {
        img = dense_dft_tables(2 * S, (int)dtype, &err);
        if (!img) return LCONV_ERR_HIP;
    }
    const int64_t units = pairs_per_channel(B) * C;
    const int64_t per = chunk3(units, S, work_complex_size(dtype, false));
    for (int64_t u0 = 0; u0 < units; u0 += per) {
        Conv3DArgs a{};
        a.u = u; a.kf = k_f; a.D = D; a.y = y; a.ws = workspace; a.tw = tw; a.img = img;
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
