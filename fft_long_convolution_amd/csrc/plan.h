// plan.h -- factorisation plans and per-device constant tables.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcv {

// Arithmetic / storage element types (numerically equal to lconv_dtype_t).
enum ComputeType { CT_F32 = 0, CT_F16 = 1, CT_BF16 = 2 };

// Transform length M = 256 * R of the fused one-workgroup path (R = 2..32 -> M = 512..8192).
//   n = 256 n1 + 16 n2 + n3          (n1 < R, n2, n3 < 16)
//   f = k1 + R k2 + 16 R k3          (k1 < R, k2, k3 < 16)
// Longer transforms split M = M1 * M2 with M2 = 8192 rows (four-step: a length-M1 column
// DFT, a twiddle, the row transform, and the reverse on the way back).
constexpr int kMaxFusedR = 32;
constexpr int64_t kRowLen = 8192;

struct Plan1D {
    int64_t N;      // sequence length
    int64_t M;      // transform length (>= 2N, power of two, >= 512)
    int R;          // M / 256 on the fused path; 32 on the row pass of the multi-pass path
    int64_t M1;     // 1 on the fused path; M / 8192 otherwise
    bool multipass;
};

// Returns false when N is outside the supported set.  With LCONV_FORCE_PATH=multipass in the
// environment (read once; for testing) every length takes the multi-pass plan with M >= 16384:
// the calls that need one workgroup per transform (partial, frequency-sparse, state-space) then
// return LCONV_ERR_UNSUPPORTED.
bool make_plan_1d(int64_t N, Plan1D* p);
bool force_multipass();
// LCONV_LOG set (and not "0"): the forward and filter calls print their plan to stderr, once per
// distinct call shape.
bool log_enabled();

// Layout of the fused-path table for (R, compute type), offsets in bytes.
struct FusedTableLayout {
    size_t img_bytes;             // one matrix image
    size_t f1, i3, f2, f3, i1, i2, tw, total;
    int rb1, kc1, rb3, kc3;       // F1 / I3 image grid (row blocks x K-chunks, full variant)
};
FusedTableLayout fused_table_layout(int R, int ct);

// Device pointer to the fused-path tables for (R, ct) on the current device (built on first
// use).  Returns nullptr and sets *err on failure.  With build = false a table that is not
// built yet is not built (nullptr, *err = hipErrorNotReady): no allocation, no copy.
const void* fused_tables(int R, int ct, hipError_t* err, bool build = true);

// Column-pass twiddles for the multi-pass path, on the current device:
//   w_lo[r] = exp(-2 pi i r / M) for r < 2048, w_hi[r] = exp(-2 pi i 2048 r / M) for r < M/2048,
//   w_col[e] = exp(-2 pi i e / M1) for e < M1.  fp32 complex (float2).
struct ColTables {
    const float* lo;
    const float* hi;
    const float* col;
};
bool col_tables(int64_t M, int64_t M1, ColTables* out, hipError_t* err, bool build = true);

// Matrix-core column passes of the multi-pass path, column length P = 16 R (R = 1 .. 64),
// 16-bit compute types (for R < 16 only the two 16-point images are used).  Digits n_hi = 16 n1 + n2, k_hi = k1 + R k2: the first stage is a
// radix-R DFT over n1 (forward: only n1 < H = R/2 is nonzero; inverse: only n1 < H is kept),
// the second a 16-point DFT over n2.  Image indices in the table: the forward first stage
// (k1 block rb, n1 block kc) at f1 + rb * hb + kc, the inverse first stage (n1 block rb, k1
// block kc) at i2 + rb * rbk + kc, the 16-point DFT and its inverse at f16 and i16, and the
// 16-point DFT with its output rows reversed (row r holds k2 = 15 - r) at f16r.
struct ColMxGrid {
    int R, H, rbk, hb;       // radix, half radix, 16-blocks of k1, 16-blocks of n1 < H
    int f1, i2, f16, i16, f16r, nimg;
};
constexpr ColMxGrid colmx_grid(int P) {
    const int R = P / 16, H = R / 2, rbk = R / 16, hb = (H + 15) / 16, b = 2 * rbk * hb;
    return ColMxGrid{R, H, rbk, hb, 0, rbk * hb, b, b + 1, b + 2, b + 3};
}
constexpr bool colmx_supported(int64_t P) { return P >= 16 && P <= 1024 && (P & (P - 1)) == 0; }
// Device pointer to those images for (P, ct) on the current device (ct 16-bit).
const void* colmx_tables(int64_t P, int ct, hipError_t* err, bool build = true);

// exp(-2 pi i e / P) for e < P, fp32 complex, on the current device (3D path).
const float* dft_table(int64_t P, hipError_t* err);

// The dense P-point DFT (P = 16 NB, NB <= 4) as 16 x 16 matrix-core images, 16-bit compute types:
// forward block (kb, nb) = w_P^{k n} for k = 16 kb + row, n = 16 nb + column, at kb NB + nb;
// inverse block (mb, kb) = w_P^{-m k}, at NB^2 + mb NB + kb.  Interleaved blocks, kq = 2 kp + par
// naming the frequencies k = 32 kp + 2 i + par (i < 16): forward rows k, inputs n = 16 nb + c, at
// 2 NB^2 + kq NB + nb; inverse rows m = 16 mb + r, inputs k, at 3 NB^2 + mb NB + kq.
const void* dense_dft_tables(int64_t P, int ct, hipError_t* err);

// Cached device properties of the current device.
int device_cu_count(hipError_t* err);

void release_tables();

}  // namespace lcv
