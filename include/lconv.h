/*
 * lconv.h -- C ABI of the MI355X (gfx950) causal long-convolution library.
 *
 * The operation (restated from the pages):
 *   * "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor Cores", abstract:
 *     long convolutions computed exactly through the FFT, with the FFT factored into matrix
 *     multiplications for matrix units and the whole chain fused to avoid memory traffic.
 *   * "FlashConv" (AIMech curated page), Mechanism: FFT, pointwise spectral product and inverse
 *     FFT fused on chip; sequences past the on-chip capacity are handled in chunks.
 *   * Caracal abstract on the "RubiConv" page: causality from one-sided zero padding plus
 *     truncation in the frequency domain.
 *   * "Native Multi-Dimensional Subquadratic Operators via Input Dependent Long
 *     Convolutions", abstract: global convolutions applied on the native 2D grid.
 *
 *   1D:  x = q (.) u                       (q optional, elementwise)
 *        y = v (.) ( irfft(rfft(x, M) * rfft(k, M))[:N] + D * x )   (v optional), M >= 2N
 *        i.e. y[b,h,t] = v[b,h,t] * ( sum_{s<=t} k[h,t-s] x[b,h,s] + D[h] x[b,h,t] ).
 *   2D:  y[b,c,i,j] = sum_{a,e} k[c,a,e] u[b,c,i+Hs/2-a,j+Ws/2-e] + D[c] u[b,c,i,j]
 *        (linear, not circular; kernel tap (a,e) sits at offset (a-Hs/2, e-Ws/2)).
 *
 * Conventions shared by every entry point
 *   * All data pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) on the
 *     current HIP device.  The caller owns and frees every buffer, including k_f and any
 *     workspace; sizes come from the *_bytes queries below.
 *   * Layouts are dense row-major: u, q, v, y are [B][H][N] with N contiguous; k is [H][N];
 *     D is [H].  2D: u, y are [B][C][Hs][Ws]; k is [C][Hs][Ws]; D is [C].  All share `dtype`.
 *   * k_f (the filter spectrum) is OPAQUE: produced by lconv_filter_fft* for one
 *     (H, N, dtype) or (C, Hs, Ws, dtype) and valid only for that shape and dtype.  Its size is
 *     lconv_filter_fft*_bytes(); the library cannot check the size of a buffer it is given,
 *     so a spectrum made for another shape or dtype is the caller's error.
 *   * Every call is asynchronous on `stream` (0 = the null stream); nothing synchronises.
 *     Faults during execution surface at the caller's next synchronising call.
 *   * Arguments are validated on the host before any HIP call.  On any error nothing is
 *     launched and outputs are untouched.  B, H, N (or B, C) equal to 0 is a valid no-op.
 *   * Pointers must be 16-byte aligned; y must not overlap any input.
 *   * The library allocates only its per-device constant tables (built once, lazily, kept
 *     until lconv_release()).  Calls are thread-safe.
 */
#ifndef LCONV_H
#define LCONV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bumped when entry points are added or a size query's result changes (3: the training pair
 * lconv_fftconv_fwd_save / lconv_fftconv_bwd_saved; the state-space workspace holds the scan's
 * part states.  4: lconv_prepare and lconv_fftconv_fwd_noalloc, two status codes.  5: 2D calls
 * take Hs x Ws images and a workspace; lconv_fftconv2d_workspace_bytes.  6: gradients and the
 * training pair for every supported N, with workspace arguments). */
#define LCONV_ABI_VERSION 8

/* The last enumerator only widens the type's range to every int, so that any value a C caller
 * passes is a valid value of the type (unknown ones are rejected with LCONV_ERR_UNSUPPORTED). */
typedef enum { LCONV_F32 = 0, LCONV_F16 = 1, LCONV_BF16 = 2, LCONV_DTYPE_MAX_ENUM = 0x7fffffff } lconv_dtype_t;

typedef enum {
    LCONV_SUCCESS = 0,
    LCONV_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                              */
    LCONV_ERR_INVALID_SHAPE = 2, /* negative size, size product overflow                    */
    LCONV_ERR_UNSUPPORTED = 3,   /* unknown dtype or a size outside the supported set       */
    LCONV_ERR_MISALIGNED = 4,    /* a pointer is not 16-byte aligned                        */
    LCONV_ERR_ALIASING = 5,      /* y overlaps an input                                     */
    LCONV_ERR_WORKSPACE = 6,     /* workspace NULL or smaller than the *_workspace_bytes    */
    LCONV_ERR_HIP = 7,           /* a HIP runtime call failed (including: no device)        */
    LCONV_ERR_NOT_PREPARED = 8,  /* lconv_fftconv_fwd_noalloc: lconv_prepare was not called for
                                    this device, length and dtype                          */
    LCONV_ERR_SCRATCH_LIMIT = 9  /* lconv_fftconv_fwd_noalloc: the call needs more scratch than
                                    LCONV_NOALLOC_SCRATCH_BYTES                            */
} lconv_status_t;

/* Largest supported sequence length (1D) and the largest supported 2D side. */
#define LCONV_MAX_N       ((int64_t)1 << 22)
#define LCONV_2D_MAX_SIDE 128

/* ---- size queries (pure host functions; 0 for invalid or unsupported arguments) ---------- */

/* Bytes of the opaque filter spectrum for H channels of length N. */
size_t lconv_filter_fft_bytes(int64_t H, int64_t N, lconv_dtype_t dtype);
/* Scratch bytes lconv_filter_fft needs (0: none). */
size_t lconv_filter_fft_workspace_bytes(int64_t H, int64_t N, lconv_dtype_t dtype);
/* Scratch bytes lconv_fftconv_fwd needs (0 when the whole transform fits one workgroup). */
size_t lconv_fftconv_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype);
/* Bytes of the opaque 2D filter spectrum for C channels of Hs x Ws kernels. */
size_t lconv_filter_fft2d_bytes(int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype);
/* Scratch bytes lconv_fftconv2d_fwd needs (0 for every supported shape: one fused kernel). */
size_t lconv_fftconv2d_workspace_bytes(int64_t B, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype);

/* ---- 1D --------------------------------------------------------------------------------- */

/*
 * Filter spectrum k_f from k[H][N]: the length-M DFT of each zero-padded filter, scaled by
 * 1/M and stored in the library's transform order (FlashConv page, Mechanism: the pointwise
 * spectral product needs the filter's spectrum; computing it once per filter keeps it out of
 * the per-call path).  Computed in fp32 arithmetic, stored in `dtype`.
 *   k         [H][N] dtype, device
 *   k_f       lconv_filter_fft_bytes(H, N, dtype) bytes, device, written
 *   workspace lconv_filter_fft_workspace_bytes(H, N, dtype) bytes (may be NULL if that is 0)
 * Supported: 1 <= N <= LCONV_MAX_N.  When N is not a multiple of 8 the rows are staged into
 * the workspace, zero-padded to the next multiple of 8 (the zero taps change nothing).
 */
lconv_status_t lconv_filter_fft(const void* k, void* k_f, int64_t H, int64_t N,
                                lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Causal long convolution, optional Hyena-style gating:
 *   y = v (.) ( (k * x)[:N] + D (.) x ),  x = q (.) u
 * (FlashFFTConv abstract: exact FFT convolution; Caracal abstract: causality by padding and
 * truncation; FlashConv Mechanism: fused FFT -> spectral product -> inverse FFT, chunked when
 * the sequence exceeds one compute unit).
 *   u, y      [B][H][N] dtype, device (y written)
 *   k_f       from lconv_filter_fft(k, ..., H, N, dtype)
 *   D         [H] dtype, device
 *   q, v      [B][H][N] dtype, device, or NULL (then treated as all ones)
 *   workspace lconv_fftconv_workspace_bytes(B, H, N, dtype) bytes (may be NULL if that is 0)
 * Supported: 1 <= N <= LCONV_MAX_N.  When N is not a multiple of 8, u, q, v are staged into the
 * workspace zero-padded to the next multiple of 8 (inputs past N change no output before N),
 * and the first N outputs of each row are copied back: two more passes over the data.
 * Arithmetic: fp32 I/O uses fp32 matrix-core products; bf16 and fp16 use bf16/fp16
 * matrix-core operands with fp32 accumulation, fp32 twiddles and fp32 pointwise products.
 */
lconv_status_t lconv_fftconv_fwd(const void* u, const void* k_f, const void* D, void* y,
                                 const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                 lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Frequency-sparse convolution: the gated causal convolution with the filter spectrum kept only
 * on some blocks of the decomposition ("FlashFFTConv" abstract: frequency-sparse convolutions,
 * computed by skipping blocks of the matrix decomposition, speed up pretrained models).  With
 * the transform length M = 256 R of the forward call, frequency block r (0 <= r < R) is the set
 * of frequencies f with f mod R = r; bit r of `keep` keeps it.  The result is
 *   y = v (.) ( IDFT_M( DFT_M(x) . K_keep )[:N] + D x ),   x = q (.) u,
 * K_keep the filter spectrum on the kept blocks and 0 elsewhere (so the effective filter is the
 * real length-M sequence IDFT(K_keep), applied circularly and truncated to N).  Dropped blocks
 * cost no transform work.  `keep` must be closed under r -> (R - r) mod R (otherwise the filter
 * would not be real): LCONV_ERR_UNSUPPORTED otherwise, as for bits at or above R.
 *   u, y, q, v, k_f, D   as for lconv_fftconv_fwd (k_f from lconv_filter_fft(k, ..., H, N, dtype))
 * Supported: N <= 4096 (one workgroup per transform), N a multiple of 8.  R: lconv_freq_blocks(N).
 * No workspace.
 */
lconv_status_t lconv_fftconv_sparse_fwd(const void* u, const void* k_f, const void* D, void* y,
                                        const void* q, const void* v, int64_t B, int64_t H,
                                        int64_t N, uint32_t keep, lconv_dtype_t dtype,
                                        hipStream_t stream);

/* Number of frequency blocks R = M / 256 of the transform for N (0 if N is unsupported by
 * lconv_fftconv_sparse_fwd). */
int lconv_freq_blocks(int64_t N);

/*
 * Learned Butterfly: the convolution above with its transforms replaced by factored matrices
 * whose dense blocks are free (learned) parameters ("Simple Hardware-Efficient Long Convolutions
 * for Sequence Modeling", abstract: the coefficients of the Butterfly decomposition are learned,
 * at the runtime of the fixed decomposition).  The factorization is the one the fused kernels
 * run for M = 256 R (N <= 4096): n = 256 n1 + 16 n2 + n3, f = k1 + R k2 + 16 R k3, and
 *   T[f, n]  = A3[k1][k3][n3] w256^{n3 k2} A2[k1][k2][n2] A1[k1][n1]          (forward)
 *   S[n, f]  = B3[n1][k1] B2[k1][n2][k2] conj(w256^{n3 k2}) B1[k1][n3][k3]     (inverse)
 * with w256 = exp(-2 pi i / 256) fixed.  With x = q u zero-padded to M, K = T k / M (k zero-padded):
 *   y[b,h,t] = v * ( Re( S (K[h] (.) T x[b,h]) )[t] + D[h] x[b,h,t] ),  t < N
 * For the DFT's blocks (A1 = w_R^{n1 k1}, A2[k1] = w_{16R}^{n2 (k1 + R k2)},
 * A3[k1] = w_M^{n3 (k1 + 16 R k3)}, B = their conjugate transposes) this is lconv_fftconv_fwd.
 * Each transform carries one real row (the pair packing of lconv_fftconv_fwd needs the
 * conjugate symmetry of the DFT), and D x is added in the time domain.
 *   blocks   fp32 complex (re, im), device: A1 [R][R] (k1, n1), A2 [R][16][16] (k1, k2, n2),
 *            A3 [R][16][16] (k1, k3, n3), B1 [R][16][16] (k1, n3, k3), B2 [R][16][16]
 *            (k1, n2, k2), B3 [R][R] (n1, k1), back to back: lconv_butterfly_blocks_count(N)
 *            complex values.  Only the columns n1 < R/2 of A1 and the rows n1 < R/2 of B3 are
 *            used (zero padding, causal truncation).
 *   tables   lconv_butterfly_tables_bytes(N, dtype) bytes, device, written by
 *            lconv_butterfly_tables (the blocks as matrix-core images, fp32 and dtype)
 *   k_f      lconv_filter_fft_bytes(H, N, dtype) bytes, written by lconv_butterfly_filter(k [H][N])
 *   u, y, q, v, D as for lconv_fftconv_fwd.
 * Supported: 8 <= N <= 4096, N a multiple of 8 (R = lconv_freq_blocks(N)); 0 from the size
 * queries and LCONV_ERR_UNSUPPORTED otherwise.  No workspace.  Errors as for lconv_fftconv_fwd;
 * tables overlapping an output give LCONV_ERR_ALIASING.
 */
int64_t lconv_butterfly_blocks_count(int64_t N);
size_t lconv_butterfly_tables_bytes(int64_t N, lconv_dtype_t dtype);
lconv_status_t lconv_butterfly_tables(const void* blocks, void* tables, int64_t N, lconv_dtype_t dtype,
                                      hipStream_t stream);
lconv_status_t lconv_butterfly_filter(const void* k, void* k_f, const void* tables, int64_t H, int64_t N,
                                      lconv_dtype_t dtype, hipStream_t stream);
lconv_status_t lconv_butterfly_fwd(const void* u, const void* k_f, const void* D, void* y, const void* q,
                                   const void* v, const void* tables, int64_t B, int64_t H, int64_t N,
                                   lconv_dtype_t dtype, hipStream_t stream);

/*
 * Partial convolution: the same gated causal convolution with a filter of L taps (zero beyond
 * them) on sequences of any length N ("FlashFFTConv" abstract: partial convolutions, computed by
 * skipping blocks of the decomposition, save memory and compute and let a model run on
 * sequences far longer than its filters).  The causal convolution matrix is then banded: each
 * block of C = M/2 outputs (M the transform length of the filter, from lconv_filter_fft with
 * length L) depends only on its own input block and the previous one, so every block is one
 * fused M-point transform of that window and all other blocks of the matrix are skipped.  Cost
 * O(N log L); the filter spectrum is stored at length L.
 *   y[b,h,t] = v * ( sum_{s = max(0, t-L+1)}^{t} k[h,t-s] x[b,h,s] + D[h] x[b,h,t] ),  x = q u
 *   u, y, q, v   [B][H][N] dtype, device (q, v may be NULL), y written
 *   k_f          from lconv_filter_fft(k, ..., H, L, dtype) with k [H][L]
 *   D            [H] dtype
 * The windows of a channel (batch row, block) are transformed two at a time as the real and
 * imaginary parts of one complex sequence, so B = 1 wastes nothing.
 * Supported: 8 <= L <= 4096 with L a multiple of 8; N >= 1 a multiple of 8 (N may be smaller or
 * larger than L, up to 2^40); H * ceil(B * ceil(N / C) / 2) < 2^31.  No workspace.
 */
lconv_status_t lconv_fftconv_partial_fwd(const void* u, const void* k_f, const void* D, void* y,
                                         const void* q, const void* v, int64_t B, int64_t H,
                                         int64_t N, int64_t L, lconv_dtype_t dtype,
                                         hipStream_t stream);

/*
 * Gradients of the partial convolution above, given dy = dL/dy (the partial convolutions of the
 * FlashFFTConv abstract, trained like the full-length ones).  With x = q (.) u, ds = dy (.) v:
 *   dx[t] = sum_{s = t}^{min(N, t+L)-1} k[h,s-t] ds[s] + D[h] ds[t];   du = q (.) dx, dq = u (.) dx
 *   dv = dy (.) ( (k * x)[:N] + D x )        (the partial forward call gated by dy)
 *   dk[h,tau] = sum_b sum_t ds[b,h,t] x[b,h,t-tau]  for tau < L (zero for tau >= N);  dD[h] = sum x ds
 *   dy, u, q, v, du, dq, dv   [B][H][N] dtype, as for lconv_fftconv_bwd (dq / dv ignored without q / v)
 *   k_f        from lconv_filter_fft(k, ..., H, L, dtype), as for lconv_fftconv_partial_fwd
 *   dk         [H][L] fp32, written (overwritten); NULL: not computed
 *   dD         [H] fp32, written; NULL: not computed
 *   workspace  lconv_fftconv_partial_bwd_workspace_bytes(B, H, N, dtype) bytes, device, 16-byte
 *              aligned (never 0 when B, H, N > 0)
 * dx is the partial forward call on time-reversed rows (the correlation over the next L positions
 * becomes a causal L-tap convolution), so it keeps the banded O(N log L) cost; rev(ds) and the
 * result pass through the workspace in dtype.  dk comes from the full-length filter gradient of
 * lconv_fftconv_bwd (its first L lags; an [H][N] fp32 part of the workspace), O(N log N).
 * B = 0 or N = 0 writes zeros to dk and dD.  Outputs must not overlap each other, any input or
 * the workspace.
 * Supported: as lconv_fftconv_partial_fwd, with N <= LCONV_MAX_N.
 */
size_t lconv_fftconv_partial_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype);
lconv_status_t lconv_fftconv_partial_bwd(const void* dy, const void* u, const void* k_f, const void* D,
                                         const void* q, const void* v, void* du, void* dq, void* dv,
                                         float* dk, float* dD, int64_t B, int64_t H, int64_t N,
                                         int64_t L, lconv_dtype_t dtype, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * Gradients of the gated causal convolution above, given dy = dL/dy (the training path the
 * FlashFFTConv abstract reports speed-ups for, and the 64K-long training of the "Simple
 * Hardware-Efficient Long Convolutions" abstract; the FFT convolution is exact, so its gradient
 * is that of the plain causal sum).  With x = q (.) u and ds = dy (.) v:
 *   dx[t] = sum_{s >= t} k[h,s-t] ds[s] + D[h] ds[t]     (correlation: conjugate spectrum)
 *   du = q (.) dx   (du = dx without q)          dq = u (.) dx
 *   dv = dy (.) ( (k * x)[:N] + D x )            (the forward convolution, gated by dy)
 *   dk[h,t] = sum_b sum_{s >= t} ds[b,h,s] x[b,h,s-t],   dD[h] = dk[h,0]
 *   dy, u     [B][H][N] dtype, device
 *   k_f, D    as for lconv_fftconv_fwd (the same spectrum)
 *   q, v      [B][H][N] dtype or NULL, as in the forward call
 *   du        [B][H][N] dtype, written
 *   dq        [B][H][N] dtype, written; required when q is given, ignored (may be NULL) otherwise
 *   dv        [B][H][N] dtype, written; required when v is given, ignored (may be NULL) otherwise
 *   dk        [H][N] fp32, written (overwritten, not accumulated); NULL: not computed
 *   dD        [H] fp32, written; NULL: not computed
 *   workspace lconv_fftconv_bwd_workspace_bytes(B, H, N, dtype) bytes (0, may be NULL, for
 *             N <= 4096)
 * B = 0 writes zeros to dk and dD.  Outputs must not overlap each other, any input or the
 * workspace.
 * N <= 4096 (one workgroup per transform): three fused launches; dk and dD are summed over the
 * batch in fp32 in the frequency domain and transformed once per channel.
 * 4096 < N <= LCONV_MAX_N: the correlations become causal convolutions of time-reversed rows,
 *   dx = rev(k * rev(ds)) + D ds,   dk[h,t] = sum_b (x_b * rev(ds_b))[N-1-t],
 * each run through the chunked multi-pass forward path (x_b as the filter of its own row), with
 * the reversals, gates and the batch sum as elementwise passes.  rev(ds) and the convolution
 * results pass through the workspace in dtype (one rounding each for 16-bit types).
 * Supported: N a multiple of 8, N <= LCONV_MAX_N.
 */
size_t lconv_fftconv_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, lconv_dtype_t dtype);
lconv_status_t lconv_fftconv_bwd(const void* dy, const void* u, const void* k_f, const void* D,
                                 const void* q, const void* v, void* du, void* dq, void* dv,
                                 float* dk, float* dD, int64_t B, int64_t H, int64_t N,
                                 lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Forward call for training: lconv_fftconv_fwd that also writes the pre-gate output
 *   c = (k * x)[:N] + D x        (y = v (.) c; c = y when v is NULL)
 * which the gradient of v needs (dv = dy (.) c, the same quantity lconv_fftconv_bwd otherwise
 * recomputes with a forward transform).
 *   c          [B][H][N] dtype, device, written; must not overlap y or any input
 *   workspace  lconv_fftconv_workspace_bytes(B, H, N, dtype) bytes, as for lconv_fftconv_fwd
 * N <= 4096: c is stored by the fused kernel beside y.  Longer: the multi-pass forward writes c
 * and one elementwise pass gives y = v (.) c.  Other arguments as for lconv_fftconv_fwd.
 * Supported: N a multiple of 8, N <= LCONV_MAX_N.
 */
lconv_status_t lconv_fftconv_fwd_save(const void* u, const void* k_f, const void* D, void* y, void* c,
                                      const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                      lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * lconv_fftconv_bwd with the pre-gate output c saved by lconv_fftconv_fwd_save: dv = dy (.) c
 * (one elementwise pass) instead of the forward transform gated by dy; du, dq, dk, dD as there.
 *   c  [B][H][N] dtype, device, as written by lconv_fftconv_fwd_save on the same u, q, k_f, D;
 *      required when v is given (LCONV_ERR_NULL_POINTER otherwise), ignored without v.
 * Other arguments, outputs, workspace and limits as for lconv_fftconv_bwd.
 */
lconv_status_t lconv_fftconv_bwd_saved(const void* dy, const void* u, const void* k_f, const void* D,
                                       const void* q, const void* v, const void* c, void* du, void* dq,
                                       void* dv, float* dk, float* dD, int64_t B, int64_t H, int64_t N,
                                       lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* ---- 2D (HyenaND-style) ------------------------------------------------------------------ */

/*
 * 2D filter spectrum ("Native Multi-Dimensional Subquadratic Operators via Input Dependent Long
 * Convolutions", abstract: global convolutions applied on the native 2D grid of the data; the
 * FlashConv page, Mechanism: the pointwise spectral product needs the filter's spectrum, built
 * once per filter).  The 256 x 256 DFT of each kernel placed with its centre tap (Hs/2, Ws/2) at
 * grid point (64, 64), scaled by 1/256^2, in the library's transform order (opaque).  fp32
 * arithmetic, stored in dtype.
 *   k    [C][Hs][Ws] dtype, device
 *   k_f  lconv_filter_fft2d_bytes(C, Hs, Ws, dtype) bytes, device, written
 * Supported: 1 <= Hs <= 128; 8 <= Ws <= 128 with Ws a multiple of 8; dtype bf16 or fp16
 * (LCONV_ERR_UNSUPPORTED otherwise, fp32 included).  C = 0 is a no-op.
 */
lconv_status_t lconv_filter_fft2d(const void* k, void* k_f, int64_t C, int64_t Hs, int64_t Ws,
                                  lconv_dtype_t dtype, hipStream_t stream);

/*
 * 2D linear (not circular) convolution with centred full-size kernels, cropped to the input
 * window, plus the D skip (same abstract: global convolutions on the native multi-dimensional
 * grid, with a fused FFT-convolution path):
 *   y[b,c,i,j] = sum_{a,e} k[c,a,e] u[b,c, i + Hs/2 - a, j + Ws/2 - e] + D[c] u[b,c,i,j]
 * (halves rounded down; u = 0 outside the image).
 *   u, y      [B][C][Hs][Ws] dtype, device (y written, must not overlap any input)
 *   k_f       from lconv_filter_fft2d(k, ..., C, Hs, Ws, dtype)
 *   D         [C] dtype, device
 *   workspace lconv_fftconv2d_workspace_bytes(...) bytes (0 for every supported shape; may be
 *             NULL)
 * One fused kernel per pair of images of one channel: row DFTs, column DFTs, spectral product,
 * inverse column and row DFTs restricted to the output window, all through LDS.  Supported
 * shapes and dtypes as for lconv_filter_fft2d.  B = 0 or C = 0 is a no-op.
 */
lconv_status_t lconv_fftconv2d_fwd(const void* u, const void* k_f, const void* D, void* y,
                                   int64_t B, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gradients of the 2D convolution above, given dy = dL/dy (HyenaND abstract: the operator is
 * trained like its 1D counterpart; it is linear in u, k and D):
 *   du[b,c,m,n] = sum_{i,j} dy[b,c,i,j] k[c, i+Hs/2-m, j+Ws/2-n] + D[c] dy[b,c,m,n]
 *   dk[c,a,e]   = sum_{b,i,j} dy[b,c,i,j] u[b,c, i+Hs/2-a, j+Ws/2-e]
 *   dD[c]       = sum_{b,i,j} dy[b,c,i,j] u[b,c,i,j]
 *   dy, u      [B][C][Hs][Ws] dtype, device
 *   k_f, D     as for lconv_fftconv2d_fwd (the same spectrum)
 *   du         [B][C][Hs][Ws] dtype, written
 *   dk         [C][Hs][Ws] fp32, written (overwritten); NULL: not computed
 *   dD         [C] fp32, written; NULL: not computed
 *   workspace  lconv_fftconv2d_bwd_workspace_bytes(B, C, Hs, Ws, dtype) bytes, device, 16-byte
 *              aligned
 * du is the forward kernel on dy with the adjoint spectrum (-1)^(u+v) conj(K) (the output window
 * at grid offset 64 moved back to the image at offset 0: a shift by half the 256-point grid),
 * formed from k_f by sign flips alone.  dk runs the forward kernel over the B*C images as
 * channels of one image, each with its own dy rotated by 180 degrees as the filter (spectra in
 * the workspace, from the same kernel's transforms of dy), and sums the rotated results over
 * the batch in fp32; the per-image
 * correlations pass through the workspace in dtype.  dD is a direct fp32 sum.
 * B = 0 writes zeros to dk and dD.  Outputs must not overlap each other, any input or the
 * workspace.  Supported: as lconv_fftconv2d_fwd.
 */
size_t lconv_fftconv2d_bwd_workspace_bytes(int64_t B, int64_t C, int64_t Hs, int64_t Ws, lconv_dtype_t dtype);
lconv_status_t lconv_fftconv2d_bwd(const void* dy, const void* u, const void* k_f, const void* D, void* du,
                                   float* dk, float* dD, int64_t B, int64_t C, int64_t Hs, int64_t Ws,
                                   lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ---- state-space filters: chunks with state passing --------------------------------------- */

/*
 * Long convolutions whose filter comes from a diagonal state-space model, run in chunks with the
 * boundary state passed between them ("FlashConv" page, Mechanism: when the sequence exceeds the
 * on-chip capacity, convolve chunk by chunk and propagate the state-space boundary state).
 * Filter: k[h,t] = Re sum_n W[h,n] lam[h,n]^t with NS complex modes per channel.  With chunk
 * length T and x = q (.) u, for t = jT + tau:
 *   y[t] = v * ( sum_{s in chunk j, s <= t} k[t-s] x[s] + Re sum_n W_n lam_n^(tau+1) h_j[n] + D x[t] )
 *   h_0 = 0,  h_{j+1}[n] = lam_n^T h_j[n] + sum_{tau<T} lam_n^(T-1-tau) x[jT + tau]
 * which equals the causal convolution with the whole filter.  The chunk convolution is the fused
 * transform of length 2T; the state terms cost O(NS) per element and run as matrix-core products
 * over 64-long segments (bf16 operands; for fp32 data split into high and remainder parts).
 *   lam, W   [H][NS] fp32 complex (interleaved re, im), device; |lam| < 1 for a decaying filter
 *   prep     lconv_ssm_prep_bytes(H, NS, T, dtype) bytes, written by lconv_ssm_prepare: the chunk
 *            filter's spectrum and tables of powers of lam (opaque)
 *   u, y, q, v [B][H][N] dtype (q, v may be NULL);  D [H] dtype
 *   workspace  lconv_fftconv_ssm_workspace_bytes(B, H, N, NS, T) bytes (chunk sums, boundary
 *              states, the per-part states of the scan over chunks)
 * Supported: T a power of two in [256, 4096]; 1 <= NS <= 256; N a multiple of 8.
 */
size_t lconv_ssm_prep_bytes(int64_t H, int64_t NS, int64_t T, lconv_dtype_t dtype);
lconv_status_t lconv_ssm_prepare(const float* lam, const float* W, void* prep, int64_t H, int64_t NS,
                                 int64_t T, lconv_dtype_t dtype, hipStream_t stream);
size_t lconv_fftconv_ssm_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t NS, int64_t T);
lconv_status_t lconv_fftconv_ssm_fwd(const void* u, const void* prep, const void* D, void* y,
                                     const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                     int64_t NS, int64_t T, lconv_dtype_t dtype, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* ---- 3D (HyenaND-style volumes) ------------------------------------------------------------ */

/*
 * The 2D operation one dimension up ("Native Multi-Dimensional Subquadratic Operators via Input
 * Dependent Long Convolutions", abstract: global convolutions on the native multi-dimensional
 * grid): a linear convolution with a centred full-size kernel (tap (a,e,f) at offset
 * (a-S/2, e-S/2, f-S/2)), cropped to the input window, plus the skip:
 *   y[b,c,i,j,l] = sum_{a,e,f} k[c,a,e,f] u[b,c,i+S/2-a,j+S/2-e,l+S/2-f] + D[c] u[b,c,i,j,l]
 * u, y [B][C][S][S][S] dtype; k [C][S][S][S]; D [C].  Supported: S = 16 or 32, any dtype.
 * The (2S)^3 transform does not fit one workgroup: both calls run passes over a caller-owned
 * workspace (sizes from the queries below; processed in chunks of at most 64 MB).
 */
size_t lconv_filter_fft3d_bytes(int64_t C, int64_t S, lconv_dtype_t dtype);
size_t lconv_filter_fft3d_workspace_bytes(int64_t C, int64_t S, lconv_dtype_t dtype);
size_t lconv_fftconv3d_workspace_bytes(int64_t B, int64_t C, int64_t S, lconv_dtype_t dtype);

/* 3D filter spectrum: the (2S)^3 DFT of each zero-padded kernel, scaled by 1/(2S)^3, in the
 * library's order (opaque), computed in fp32 and stored in dtype. */
lconv_status_t lconv_filter_fft3d(const void* k, void* k_f, int64_t C, int64_t S,
                                  lconv_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* 3D convolution (definition above); k_f from lconv_filter_fft3d. */
lconv_status_t lconv_fftconv3d_fwd(const void* u, const void* k_f, const void* D, void* y,
                                   int64_t B, int64_t C, int64_t S, lconv_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- set-up, and the forward call for callers that cannot allocate ------------------------ */

/*
 * Builds, on the current device, every constant table lconv_fftconv_fwd uses for sequences of
 * length N in `dtype` (DFT-block images, twiddles), and sets up the device's scratch buffer for
 * lconv_fftconv_fwd_noalloc.  The other entry points build their tables on first use, which
 * allocates device memory and uploads it with one blocking copy; calling this first moves that
 * work here.  Synchronous; call it once per (device, N, dtype) before capturing or timing.
 */
lconv_status_t lconv_prepare(int64_t N, lconv_dtype_t dtype);

/* Size of the library's static scratch buffer (one per GPU, held until the process ends). */
#define LCONV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * For callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: lconv_fftconv_fwd with its workspace taken from a
 * library-owned static device buffer of LCONV_NOALLOC_SCRATCH_BYTES, so the call makes no
 * allocation, no free and no host-to-device copy.  The caller still passes u, k_f, D, y, q, v.
 *   * lconv_prepare(N, dtype) must have been called on the current device first
 *     (LCONV_ERR_NOT_PREPARED otherwise; nothing is launched).
 *   * The multi-pass path (N > 4096) runs in chunks that fit the buffer; a call that needs more
 *     than it holds (staging for N not a multiple of 8 plus one sequence's transform) returns
 *     LCONV_ERR_SCRATCH_LIMIT before any launch.  For N a multiple of 8 every supported length
 *     fits.
 *   * All calls on one GPU share its buffer, which keeps the last call's contents (no part of it
 *     needs to start at zero): calls that overlap in time on one GPU (on different streams, or
 *     from different threads without ordering) race and give wrong results.  Order them.
 * Arguments, results and the other errors are those of lconv_fftconv_fwd.
 */
lconv_status_t lconv_fftconv_fwd_noalloc(const void* u, const void* k_f, const void* D, void* y,
                                         const void* q, const void* v, int64_t B, int64_t H, int64_t N,
                                         lconv_dtype_t dtype, hipStream_t stream);

/* ---- misc ------------------------------------------------------------------------------- */

const char* lconv_status_string(lconv_status_t s);
int lconv_abi_version(void);
/* Frees the per-device constant tables (they are rebuilt on next use). Not thread-safe
 * against concurrent calls. */
lconv_status_t lconv_release(void);

#ifdef __cplusplus
}
#endif
#endif /* LCONV_H */
