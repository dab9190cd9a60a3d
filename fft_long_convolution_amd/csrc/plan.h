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

// Returns false when N is outside the supported set.
bool make_plan_1d(int64_t N, Plan1D* p);

// Layout of the fused-path table for (R, compute type), offsets in bytes.
struct FusedTableLayout {
    size_t img_bytes;             // one matrix image
    size_t f1, i3, f2, f3, i1, i2, tw, total;
    int rb1, kc1, rb3, kc3;       // F1 / I3 image grid (row blocks x K-chunks, full variant)
};
FusedTableLayout fused_table_layout(int R, int ct);

// Device pointer to the fused-path tables for (R, ct) on the current device (built on first
// use).  Returns nullptr and sets *err on failure.
const void* fused_tables(int R, int ct, hipError_t* err);

// Column-pass twiddles for the multi-pass path, on the current device:
//   w_lo[r] = exp(-2 pi i r / M) for r < 2048, w_hi[r] = exp(-2 pi i 2048 r / M) for r < M/2048,
//   w_col[e] = exp(-2 pi i e / M1) for e < M1.  fp32 complex (float2).
struct ColTables {
    const float* lo;
    const float* hi;
    const float* col;
};
bool col_tables(int64_t M, int64_t M1, ColTables* out, hipError_t* err);

// exp(-2 pi i e / P) for e < P, fp32 complex, on the current device (3D path).
const float* dft_table(int64_t P, hipError_t* err);

// Cached device properties of the current device.
int device_cu_count(hipError_t* err);

void release_tables();

}  // namespace lcv
