// kernels.h -- launchers of the gfx950 kernels (host-callable, defined in the .hip files).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace lcv {

// ADJ is the adjoint of CONV: the same chain with the conjugate filter spectrum (a correlation,
// whose causal truncation keeps the outputs that depend on later inputs).  PART is CONV for a
// filter of at most M/2 taps on a sequence of any length, one block of M/2 outputs per item.
// SPARSE is CONV with the filter spectrum kept only on the frequency blocks set in `keep`.
// SAVE is CONV that also stores the pre-gate output c (the value v multiplies) to y2.
// ROWFWD16 is ROWFWD computed in the 16-bit io type (the spectra of the rows' own inputs in the
// long-sequence filter gradient), not in fp32.
enum Mode1D { MODE_CONV = 0, MODE_FILTER = 1, MODE_ROW = 2, MODE_ROWFWD = 3, MODE_ADJ = 4, MODE_PART = 5,
              MODE_SPARSE = 6, MODE_SAVE = 7, MODE_LBF = 8, MODE_ROWFWD16 = 9 };

struct Fused1DArgs {
    const void* u;       // CONV: u [B][H][N]; FILTER: k [H][N]; ROW/ROWFWD: workspace rows;
                         // ADJ: dy;  DK: u
    const void* q;       // CONV: pre-gate (nullable); ADJ: v (nullable); DK: q (nullable)
    const void* v;       // CONV: post-gate (nullable); ADJ: q (du = q dx; nullable); DK: v (nullable)
    const void* e2;      // ADJ: u (dq = u dx, used when v above is set); DK: dy
    void* y;             // CONV: y; FILTER/ROWFWD: k_f; ROW: workspace rows (in place);
                         // ADJ: du;  DK: dk [H][N] fp32 (nullable)
    void* y2;            // ADJ: dq (when v above is set);  SAVE: c (pre-gate output);  DK: dD [H] fp32
                         // (nullable)
    const void* kf;      // CONV/ROW/ADJ: k_f
    const void* D;       // CONV/ROW/ADJ: D [H]
    const void* tables;  // fused-path tables for (R, compute type)
    int64_t B, H, N;     // CONV/FILTER/PART shape
    int64_t nitems;      // CONV: pairs; FILTER: channels; ROW/ROWFWD: rows; PART: pairs x blocks
    int64_t nchunk;      // PART: blocks of M/2 positions per row
    uint32_t keep;       // SPARSE: bit k1 set = frequency block k1 (f mod R = k1) kept
    int local;           // PART: 1 = each block convolved on its own (previous block taken as zero)
    int64_t sb, sh;      // CONV with N = 4096, 16-bit: element strides between batch rows and between
                         // channels (0: the contiguous [B][H][N] layout); other kernels require 0
    int64_t per_wg;      // items per workgroup (set by the launcher)
    float inv_m;         // 1 / M
    int64_t M;           // full transform length (ROW/ROWFWD: M1 * 8192)
    int64_t M1;          // ROW/ROWFWD: rows per sequence
    int64_t wrows;       // ROW (16-bit): workspace rows stored per sequence (0: M1), rows 0 .. wrows-1
    int64_t seq0;        // ROW/ROWFWD: global index of the chunk's first sequence
    int64_t seq_per_h;   // ROW: sequences per channel (h = seq / seq_per_h); ROWFWD: 1
};

// dtype: io element type (ComputeType values); the compute type is fp32 for fp32 io and for
// the filter transforms, else the io type.
// gq / gv: the pre-gate q / post-gate v pointers are set (conv and adj modes).
hipError_t launch_fused1d(int R, int dtype, int mode, bool gq, bool gv, const Fused1DArgs& a,
                          int cus, hipStream_t stream);

// Per-mode instantiations (fused1d_conv.hip, fused1d_adj.hip, fused1d_part.hip), called by
// launch_fused1d.
hipError_t launch_fused1d_conv(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                               hipStream_t stream);
hipError_t launch_fused1d_adj(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                              hipStream_t stream);
hipError_t launch_fused1d_part(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                               hipStream_t stream);
hipError_t launch_fused1d_sparse(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                                 hipStream_t stream);
hipError_t launch_fused1d_lbf(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                              hipStream_t st);
// Learned-Butterfly factor blocks (A1, A2, A3, B1, B2, B3; fp32 complex, butterfly.hip) -> matrix
// images in the fused table layout L for (R, ct); the twiddle section is not touched.
hipError_t launch_bfly_images(const void* blocks, void* out, int R, int ct, const FusedTableLayout& L,
                              hipStream_t st);
hipError_t launch_fused1d_save(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                               hipStream_t stream);
// y[i] = dy[i] * c[i] for n elements of type dtype (stage.hip): dv from a saved pre-gate output.
hipError_t launch_mul_rows(const void* dy, const void* c, void* y, int64_t n, int dtype, hipStream_t stream);

// Filter gradient: per channel h (items = channels), the sum over batch pairs of
// conj(DFT(q u)) DFT(dy v), inverse-transformed; dk[h][n] for n < N and dD[h] = dk[h][0]
// (fp32).  gq / gv: q / v pointers are set.
hipError_t launch_dk1d(int R, int dtype, bool gq, bool gv, const Fused1DArgs& a, int cus,
                       hipStream_t stream);

struct ColArgs {
    const void* u;       // pass A input: u [B][H][N] (CONV) or k [H][N] (FILTER)
    const void* q;       // pass A pre-gate (nullable)
    const void* v;       // pass C post-gate (nullable)
    void* y;             // pass C output y [B][H][N]
    void* ws;            // workspace [S_chunk][M1][8192] complex (compute type)
    const float* tw_lo;  // exp(-2 pi i r / M), r < 2048
    const float* tw_hi;  // exp(-2 pi i 2048 r / M)
    const float* tw_col; // exp(-2 pi i e / M1)
    int64_t B, H, N;
    int64_t M, M1;
    int64_t seq0;        // first sequence (pair or channel) of this chunk
    int64_t nseq;        // sequences in this chunk
    int64_t seq_per_h;   // pairs per channel (CONV) or 1 (FILTER)
    int filter;          // 1: input is k (one real channel per sequence)
    const void* img;     // matrix-core column images (16-bit, column lengths 256..1024), or null
    int64_t rows;        // workspace rows stored per sequence: M1, or M1/2 + 1 when every sequence
                         // is one real row (its column spectra are conjugate-symmetric in k_hi, so
                         // rows k_hi > M1/2 are not stored; matrix-core passes with M1 >= 256 only)
};

// Pass A: per sequence and column n_lo, DFT over n_hi < M1/2 (zero above), twiddle
// exp(-2 pi i n_lo k_hi / M), store row-major [k_hi][n_lo] into the workspace.
hipError_t launch_col_fwd(int dtype, const ColArgs& a, hipStream_t stream);
// Pass C: inverse twiddle, inverse DFT over k_hi for n_hi < M1/2, gate, store y.
hipError_t launch_col_inv(int dtype, const ColArgs& a, hipStream_t stream);
// The same two passes on the matrix cores, for 16-bit types and M1 = 16 .. 1024 (a.img set).
hipError_t launch_colmx(bool fwd, int dtype, const ColArgs& a, hipStream_t stream);

struct Conv2DArgs {
    const void* u;       // [B][C][Hs][Ws]
    const void* kf;      // 2D spectrum (transform order)
    const void* D;       // [C]
    void* y;             // [B][C][Hs][Ws]
    const void* tables;
    int64_t B, C;
    int Hs, Ws;          // image sides: 1 <= Hs <= 128, 8 <= Ws <= 128 with Ws a multiple of 8
    float inv_p2;        // 1 / (2S)^2
    int filter;          // 1: u = k [C][S][S]; the spectrum is written to kf
    int spec;            // 1 (with B = 1): store the spectrum of each image rotated by 180 degrees,
                         // as a filter spectrum, to y (the 2D filter gradient's filters)
    int cus;             // compute units (persistent grid size)
};
hipError_t launch_conv2d(int dtype, const Conv2DArgs& a, hipStream_t stream);
// 2D gradient passes: the adjoint spectrum (-1)^(u+v) conj(K) in stored order; the batch sum of
// rotated per-image correlations into dk [C][Hs][Ws] fp32; dD[c] = sum dy u (fp32)
hipError_t launch_adj2d(const void* kf, void* ka, int64_t C, hipStream_t stream);
hipError_t launch_dk2d_sum(int dtype, const void* r, float* dk, int64_t B, int64_t C, int Hs, int Ws,
                           hipStream_t stream);
hipError_t launch_dd2d(int dtype, const void* dy, const void* u, float* dD, int64_t B, int64_t C, int64_t img,
                       hipStream_t stream);

// State passing for diagonal state-space filters (ssm.hip).  Modes are handled in blocks of
// ssm_block_modes(NS) = 64 (the last block zero-padded); NSP = blocks * block modes.
inline int ssm_block_modes(int64_t) { return 64; }
inline int ssm_blocks(int64_t NS) { return (int)((NS + ssm_block_modes(NS) - 1) / ssm_block_modes(NS)); }
// Bytes of one channel's operand images (sums or correction): per block, 4 tile positions x
// 4 NQ ops x 2 parts x 1 KiB.
constexpr int64_t kSsmMaxParts = 64;   // parts of the scan over chunks
inline int64_t ssm_image_bytes(int64_t NS) { return (int64_t)ssm_blocks(NS) * (ssm_block_modes(NS) / 16) * 32768; }
struct SsmArgs {
    const void* u;       // [B][H][N] io
    const void* q;       // pre-gate (nullable)
    const void* v;       // post-gate (nullable)
    void* y;             // [B][H][N] io: the chunk-local result, corrected in place
    void* md;            // [H][NS][4] fp32 complex: lam, W lam, lam^T, 0
    void* pw;            // [H][17][NSP] fp32 complex: lam^(64 e), zero for padding modes
    void* ts;            // [H][blocks] operand images of the chunk sums (bf16 hi / lo)
    void* tc;            // [H][blocks] operand images of the correction (bf16 hi / lo)
    void* g;             // [B*H][nch][NS] fp32 complex: chunk sums
    void* cs;            // [B*H][nch][NS] fp32 complex: W lam h_j, h_j the state before chunk j
    void* sp;            // [B*H][nparts][NS] fp32 complex: each part's final state from a zero start
    void* kchunk;        // prepare: k[H][T] io (the chunk filter)
    int64_t B, H, N, NS, T, nch;
    int64_t nparts, plen;   // the scan over chunks: parts of plen chunks
    int nsb, nmb;        // modes per block, blocks
    int mb;              // correction launch: its mode block
};
hipError_t launch_ssm_prepare(int dtype, const float* lam, const float* W, const SsmArgs& a,
                              hipStream_t stream);
hipError_t launch_ssm_state(int dtype, const SsmArgs& a, bool gq, bool gv, hipStream_t stream);

// Row reversals for the gradients of long sequences (stage.hip), rows of N (a multiple of 8)
// elements of type dtype:
//   out = rev(a (.) b)                          (b nullable)
//   d1 = g1 (.) rev(t),  d2 = g2 (.) rev(t)      (g1 nullable: d1 = rev(t); d2 nullable: skipped)
//   dk[h][t] = sum_b r[b][h][N-1-t] (fp32), dD[h] = dk[h][0]   (either nullable)
hipError_t launch_rev_gate(const void* a, const void* b, void* out, int64_t rows, int64_t N, int dtype,
                           hipStream_t stream);
hipError_t launch_rev_gated_out(const void* t, const void* g1, const void* g2, void* d1, void* d2, int64_t rows,
                                int64_t N, int dtype, hipStream_t stream);
// dD[h] and dk[h][0] as the direct fp32 sum over batch and time of (q u)(dy v) (gates optional),
// through S = dot_slices(N) partial sums per channel in part [H][S] (fp32).
inline int dot_slices(int64_t N) {
    const int64_t s = N / 8 / 256;
    return (int)(s < 1 ? 1 : (s > 64 ? 64 : s));
}
hipError_t launch_dot_lag0(const void* u, const void* q, const void* dy, const void* v, float* part, float* dk,
                           float* dD, int64_t B, int64_t H, int64_t N, int dtype, hipStream_t stream);
hipError_t launch_rev_batch_sum(const void* r, float* dk, float* dD, int64_t B, int64_t H, int64_t N, int dtype,
                                hipStream_t stream);

// Zero n 32-bit words (stage.hip): a kernel, so that callers under graph capture record no
// memset node.
hipError_t launch_zero_words(void* p, int64_t n, hipStream_t stream);
// dst [rows][L] fp32 = the first min(N, L) entries of each src [rows][N] row, zeros after
hipError_t launch_copy_cols(const float* src, float* dst, int64_t rows, int64_t N, int64_t L, hipStream_t stream);

// Row staging for N not a multiple of 8 (stage.hip): [rows][N] <-> [rows][N8] with a zero tail.
hipError_t launch_pad_rows(const void* src, void* dst, int64_t rows, int64_t N, int64_t N8, int esize,
                           hipStream_t stream);
hipError_t launch_unpad_rows(const void* src, void* dst, int64_t rows, int64_t N, int64_t N8, int esize,
                             hipStream_t stream);

// 3D (volumes of S^3, S = 16 or 32): the three passes for one chunk of units.  A unit is one
// pair of batch images of one channel (unit = c * ceil(B/2) + pair), or one channel's kernel in
// filter mode (unit = c).
struct Conv3DArgs {
    const void* u;       // [B][C][S][S][S]; filter mode: k [C][S][S][S]
    const void* kf;      // filter spectrum [C][P][P][P] complex (io type), P = 2S
    const void* D;       // [C]
    void* y;             // [B][C][S][S][S]; filter mode: the filter spectrum
    void* ws;            // workspace [nunit][S][P][P] complex (compute type; fp32 in filter mode)
    const float* tw;     // exp(-2 pi i e / P), e < P (fp32 complex)
    const void* img;     // dense P-point DFT images (16-bit S = 32 convolution: matrix-core passes)
    int64_t B, C, S;
    int64_t unit0, nunit;
    float inv_p3;        // 1 / P^3
    int filter;
};
hipError_t launch_conv3d(int dtype, const Conv3DArgs& a, hipStream_t stream);

}  // namespace lcv
