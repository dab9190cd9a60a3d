// The C ABI's host code under the address and undefined-behaviour sanitizers: every size query
// and the argument checks of every entry point, with addresses that are never dereferenced
// (checks run before any HIP call), and valid calls that reach the HIP runtime (no device here:
// LCONV_ERR_HIP).  Exit status 0 when every status is the documented one.
#include <cstdint>
#include <cstdio>

#include "lconv.h"

static int failures = 0;
#define EXPECT(call, want)                                                                     \
    do {                                                                                       \
        const int got_ = (int)(call);                                                          \
        if (got_ != (int)(want)) {                                                             \
            std::fprintf(stderr, "line %d: %s = %d, expected %d\n", __LINE__, #call, got_,      \
                         (int)(want));                                                         \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)

static void* at(uint64_t a) { return (void*)(uintptr_t)a; }

int main() {
    const lconv_dtype_t BF = LCONV_BF16, F32 = LCONV_F32;
    void *A = at(1ull << 32), *Bq = at(2ull << 32), *C = at(3ull << 32), *Y = at(4ull << 32), *W = at(5ull << 32);
    // size queries, including sizes that overflow
    const int64_t lengths[] = {1, 7, 8, 1000, 4096, 4097, 65536, (int64_t)1 << 21, (int64_t)1 << 22,
                               ((int64_t)1 << 22) + 1};
    for (int64_t n : lengths) {
        for (lconv_dtype_t dt : {LCONV_F32, LCONV_F16, LCONV_BF16}) {
            (void)lconv_filter_fft_bytes(768, n, dt);
            (void)lconv_filter_fft_workspace_bytes(768, n, dt);
            (void)lconv_fftconv_workspace_bytes(16, 768, n, dt);
            (void)lconv_fftconv_bwd_workspace_bytes(16, 768, n, dt);
        }
    }
    EXPECT(lconv_filter_fft_bytes(INT64_MAX, 4096, BF), 0);
    EXPECT(lconv_fftconv_workspace_bytes(INT64_MAX, INT64_MAX, 65536, BF), 0);
    EXPECT(lconv_fftconv_bwd_workspace_bytes(INT64_MAX, 2, 65536, BF), 0);
    EXPECT(lconv_filter_fft2d_bytes(INT64_MAX, 128, 128, BF), 0);
    EXPECT(lconv_filter_fft3d_bytes(INT64_MAX, 32, BF), 0);
    // forward
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 64, (lconv_dtype_t)9, nullptr, 0, nullptr),
           LCONV_ERR_UNSUPPORTED);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, -1, 3, 64, BF, nullptr, 0, nullptr), LCONV_ERR_INVALID_SHAPE);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, INT64_MAX, 2, 2, BF, nullptr, 0, nullptr),
           LCONV_ERR_INVALID_SHAPE);
    EXPECT(lconv_fftconv_fwd(nullptr, Bq, C, Y, nullptr, nullptr, 2, 3, 64, BF, nullptr, 0, nullptr),
           LCONV_ERR_NULL_POINTER);
    EXPECT(lconv_fftconv_fwd(at((1ull << 32) + 2), Bq, C, Y, nullptr, nullptr, 2, 3, 64, BF, nullptr, 0, nullptr),
           LCONV_ERR_MISALIGNED);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, A, nullptr, nullptr, 2, 3, 64, BF, nullptr, 0, nullptr), LCONV_ERR_ALIASING);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, 4, 4, 65536, BF, nullptr, 0, nullptr), LCONV_ERR_WORKSPACE);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 12, BF, nullptr, 0, nullptr), LCONV_ERR_WORKSPACE);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, 0, 3, 64, BF, nullptr, 0, nullptr), LCONV_SUCCESS);
    EXPECT(lconv_fftconv_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 64, BF, nullptr, 0, nullptr), LCONV_ERR_HIP);
    // filter spectra
    EXPECT(lconv_filter_fft(A, Y, 3, 64, BF, nullptr, 0, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_filter_fft(A, A, 3, 64, BF, nullptr, 0, nullptr), LCONV_ERR_ALIASING);
    EXPECT(lconv_filter_fft(A, Y, 3, (int64_t)1 << 21, BF, nullptr, 0, nullptr), LCONV_ERR_WORKSPACE);
    // gradients and the training pair
    EXPECT(lconv_fftconv_bwd(A, Bq, C, W, nullptr, nullptr, Y, nullptr, nullptr, nullptr, nullptr, 2, 3, 64, BF,
                             nullptr, 0, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_fftconv_bwd(A, Bq, C, W, A, nullptr, Y, nullptr, nullptr, nullptr, nullptr, 2, 3, 64, BF,
                             nullptr, 0, nullptr), LCONV_ERR_NULL_POINTER);
    EXPECT(lconv_fftconv_bwd(A, Bq, C, W, nullptr, nullptr, Y, nullptr, nullptr, nullptr, nullptr, 2, 3, 8192, BF,
                             nullptr, 0, nullptr), LCONV_ERR_WORKSPACE);
    EXPECT(lconv_fftconv_bwd(A, Bq, C, W, nullptr, nullptr, Y, nullptr, nullptr, nullptr, nullptr, 2, 3, 8192, BF,
                             A, lconv_fftconv_bwd_workspace_bytes(2, 3, 8192, BF), nullptr), LCONV_ERR_ALIASING);
    EXPECT(lconv_fftconv_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             (float*)Y, (float*)W, 0, 4, 64, BF, nullptr, 0, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_fftconv_fwd_save(A, Bq, C, Y, W, nullptr, nullptr, 2, 3, 8192, BF, nullptr, 0, nullptr),
           LCONV_ERR_WORKSPACE);
    EXPECT(lconv_fftconv_bwd_saved(A, Bq, C, W, nullptr, A, nullptr, Y, nullptr, at(6ull << 32), nullptr, nullptr,
                                   2, 3, 64, BF, nullptr, 0, nullptr), LCONV_ERR_NULL_POINTER);
    // partial, frequency-sparse
    EXPECT(lconv_fftconv_partial_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 1 << 20, 4096, BF, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_fftconv_partial_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 64, 8192, BF, nullptr), LCONV_ERR_UNSUPPORTED);
    EXPECT(lconv_fftconv_sparse_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 4096, 0x3u, BF, nullptr), LCONV_ERR_UNSUPPORTED);
    EXPECT(lconv_fftconv_sparse_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 4096, 0x1u, BF, nullptr), LCONV_ERR_HIP);
    // learned Butterfly
    EXPECT(lconv_butterfly_blocks_count(4096) == 2 * 32 * 32 + 1024 * 32 ? LCONV_SUCCESS : LCONV_ERR_INVALID_SHAPE,
           LCONV_SUCCESS);
    EXPECT(lconv_butterfly_tables(A, Y, 8192, BF, nullptr), LCONV_ERR_UNSUPPORTED);
    EXPECT(lconv_butterfly_tables(A, Y, 4096, BF, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_butterfly_filter(A, Y, W, 3, 4096, BF, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_butterfly_fwd(A, Bq, C, Y, nullptr, nullptr, W, 2, 3, 4096, BF, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_butterfly_fwd(A, Bq, C, Y, nullptr, nullptr, Y, 2, 3, 4096, BF, nullptr), LCONV_ERR_ALIASING);
    // 2D, 3D, state-space
    EXPECT(lconv_fftconv2d_fwd(A, Bq, C, Y, 2, 3, 100, 64, BF, nullptr, 0, nullptr), LCONV_ERR_HIP);
    EXPECT(lconv_fftconv2d_fwd(A, Bq, C, Y, 2, 3, 128, 12, BF, nullptr, 0, nullptr), LCONV_ERR_UNSUPPORTED);
    EXPECT(lconv_filter_fft2d(A, Y, 3, 128, 128, F32, nullptr), LCONV_ERR_UNSUPPORTED);
    EXPECT(lconv_fftconv3d_fwd(A, Bq, C, Y, 2, 3, 32, BF, nullptr, 0, nullptr), LCONV_ERR_WORKSPACE);
    EXPECT(lconv_fftconv_ssm_fwd(A, Bq, C, Y, nullptr, nullptr, 2, 3, 8192, 16, 1024, BF, nullptr, 0, nullptr),
           LCONV_ERR_WORKSPACE);
    for (int s = 0; s < 12; ++s) (void)lconv_status_string((lconv_status_t)s);
    EXPECT(lconv_release(), LCONV_SUCCESS);
    if (failures) std::fprintf(stderr, "%d failures\n", failures);
    else std::printf("ABI_SANITIZED_OK\n");
    return failures ? 1 : 0;
}
