/*
 * oracle.c -- float64 CPU oracle for the causal long convolution and its 2D variant.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call this file;
 * only the tests, the smoke check and the bench's CPU-baseline leg use it. It shares no code,
 * headers, tables or helpers with the HIP library.
 *
 * What it computes (the plain definitions, not the fast algorithm):
 *
 *  1D, causal.  "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor Cores"
 *  (abstract) says the method speeds up *exact* FFT convolutions; "Simple Hardware-Efficient
 *  Long Convolutions for Sequence Modeling" (abstract) frames the operator as a long
 *  convolution over the sequence; the Caracal abstract (on the "RubiConv" page) makes an FFT
 *  mixer causal by zero padding on one side and truncating.  With the FFT length at least
 *  2N-1 the padded FFT product, truncated to N samples, equals the causal linear
 *  convolution, so the oracle is that convolution summed directly:
 *
 *      x[b,h,s]  = q[b,h,s] * u[b,h,s]                    (q = 1 when absent)
 *      y[b,h,t]  = v[b,h,t] * ( sum_{s=0..t} k[h,t-s] * x[b,h,s]  +  D[h] * x[b,h,t] )
 *                                                          (v = 1 when absent)
 *
 *  2D, non-causal.  "Native Multi-Dimensional Subquadratic Operators via Input Dependent Long
 *  Convolutions" (abstract) convolves images on their native grid with global kernels.  For
 *  Hs x Ws images the kernel k[c] has Hs x Ws taps, tap (a,e) sitting at offset
 *  (a - Hs/2, e - Ws/2) (halves rounded down); the full linear convolution is cropped to the
 *  Hs x Ws window starting at (Hs/2, Ws/2):
 *
 *      y[b,c,i,j] = sum_{a,e} k[c,a,e] * u[b,c, i + Hs/2 - a, j + Ws/2 - e] + D[c] * u[b,c,i,j]
 *
 *  with u = 0 outside [0,Hs) x [0,Ws).
 *
 * Inputs arrive in their storage dtype (fp32, fp16 or bf16 bit patterns) and are widened
 * exactly to double.  All sums run in ascending index order in double precision.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* IEEE binary16 -> double, exact (written out from the binary16 format definition). */
static double or_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);                 /* subnormal: mant * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant | 0x400), expo - 25); /* (1.mant) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double, exact: the 16 bits are the top half of a binary32. */
static double or_bf16_to_double(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

static double or_load(const void* p, int dt, int64_t i) {
    switch (dt) {
    case OR_F32: return (double)((const float*)p)[i];
    case OR_F16: return or_half_to_double(((const uint16_t*)p)[i]);
    default:     return or_bf16_to_double(((const uint16_t*)p)[i]);
    }
}

static void or_widen(const void* p, int dt, int64_t off, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_load(p, dt, off + i);
}

/* Exported for the tests: widen n elements of a dtype array into doubles. */
void oracle_widen(const void* p, int dt, int64_t n, double* out) { or_widen(p, dt, 0, n, out); }

/* A job is one slice [lo, hi) of a selection list, run on one thread. */
typedef struct {
    const void *u, *q, *v, *k, *D;
    int dt;
    int64_t B, H, N;   /* 1D: batch, channels, length.  2D: batch, channels, side S. */
    const int64_t* sel;
    double* out;
    int64_t lo, hi;
    int64_t L;         /* short-filter sums: filter length (k is [H][L]) */
} or_job;

static void or_parallel(void* (*fn)(void*), or_job proto, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    or_job* jobs = (or_job*)calloc((size_t)nthreads, sizeof(or_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int64_t per = (n + nthreads - 1) / nthreads;
    int used = 0;
    for (int i = 0; i < nthreads; ++i) {
        int64_t lo = (int64_t)i * per, hi = lo + per < n ? lo + per : n;
        if (lo >= hi) break;
        jobs[used] = proto;
        jobs[used].lo = lo;
        jobs[used].hi = hi;
        pthread_create(&th[used], NULL, fn, &jobs[used]);
        ++used;
    }
    for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

/* ------------------------------------------------------------------------------------------ */
/* 1D                                                                                          */
/* ------------------------------------------------------------------------------------------ */

/* x[s] = q*u for s in [0, len) of row (b,h), widened. */
static void or_row_x(const or_job* J, int64_t b, int64_t h, int64_t len, double* x) {
    int64_t off = (b * J->H + h) * J->N;
    or_widen(J->u, J->dt, off, len, x);
    if (J->q)
        for (int64_t s = 0; s < len; ++s) x[s] *= or_load(J->q, J->dt, off + s);
}

/* Full output rows: for each t, the causal sum over s = 0..t in ascending s, then the skip
 * term and the post-gate. */
static void* or_rows_worker(void* arg) {
    or_job* J = (or_job*)arg;
    const int64_t N = J->N;
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    double* k = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[2 * r], h = J->sel[2 * r + 1];
        or_row_x(J, b, h, N, x);
        or_widen(J->k, J->dt, h * N, N, k);
        double d = or_load(J->D, J->dt, h);
        double* y = J->out + r * N;
        int64_t off = (b * J->H + h) * N;
        for (int64_t t = 0; t < N; ++t) {
            double a = 0;
            for (int64_t s = 0; s <= t; ++s) a += k[t - s] * x[s];
            double val = a + d * x[t];
            if (J->v) val *= or_load(J->v, J->dt, off + t);
            y[t] = val;
        }
    }
    free(x);
    free(k);
    return NULL;
}

/* Single output positions (b,h,t); each costs t+1 multiply-adds. */
static void* or_points_worker(void* arg) {
    or_job* J = (or_job*)arg;
    const int64_t N = J->N;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[3 * r], h = J->sel[3 * r + 1], t = J->sel[3 * r + 2];
        int64_t off = (b * J->H + h) * N;
        double a = 0;
        for (int64_t s = 0; s <= t; ++s) {
            double xs = or_load(J->u, J->dt, off + s);
            if (J->q) xs *= or_load(J->q, J->dt, off + s);
            a += or_load(J->k, J->dt, h * N + (t - s)) * xs;
        }
        double xt = or_load(J->u, J->dt, off + t);
        if (J->q) xt *= or_load(J->q, J->dt, off + t);
        double val = a + or_load(J->D, J->dt, h) * xt;
        if (J->v) val *= or_load(J->v, J->dt, off + t);
        J->out[r] = val;
    }
    return NULL;
}

static int or_check1d(const void* u, const void* k, const void* D, const int64_t* sel,
                      int64_t nsel, double* out, int64_t B, int64_t H, int64_t N, int dt) {
    if (!u || !k || !D || !out || (nsel > 0 && !sel)) return -1;
    if (B < 1 || H < 1 || N < 1 || nsel < 0 || dt < 0 || dt > 2) return -1;
    return 0;
}

/* Full rows y[b,h,0:N] for each (b,h) in rows[2*nrows]; out is [nrows][N]. */
int oracle_conv1d_rows(const void* u, const void* q, const void* v, const void* k, const void* D,
                       int dt, int64_t B, int64_t H, int64_t N, const int64_t* rows,
                       int64_t nrows, double* out, int nthreads) {
    if (or_check1d(u, k, D, rows, nrows, out, B, H, N, dt)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= B || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= H)
            return -1;
    or_job J = {u, q, v, k, D, dt, B, H, N, rows, out, 0, 0, 0};
    or_parallel(or_rows_worker, J, nrows, nthreads);
    return 0;
}

/* Output values y[b,h,t] for each (b,h,t) in pts[3*npts]; out is [npts]. */
int oracle_conv1d_points(const void* u, const void* q, const void* v, const void* k,
                         const void* D, int dt, int64_t B, int64_t H, int64_t N,
                         const int64_t* pts, int64_t npts, double* out, int nthreads) {
    if (or_check1d(u, k, D, pts, npts, out, B, H, N, dt)) return -1;
    for (int64_t r = 0; r < npts; ++r)
        if (pts[3 * r] < 0 || pts[3 * r] >= B || pts[3 * r + 1] < 0 || pts[3 * r + 1] >= H ||
            pts[3 * r + 2] < 0 || pts[3 * r + 2] >= N)
            return -1;
    or_job J = {u, q, v, k, D, dt, B, H, N, pts, out, 0, 0, 0};
    or_parallel(or_points_worker, J, npts, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 1D with a short filter (partial convolution: FlashFFTConv abstract)                         */
/* ------------------------------------------------------------------------------------------ */
/* The filter has L taps, k[h][0..L), and is zero beyond them; the sequence has N >= 1 positions
 * (N may be larger or smaller than L).  The plain causal sum then runs over the last L inputs:
 *     y[b,h,t] = v * ( sum_{s = max(0, t-L+1)}^{t} k[h,t-s] x[b,h,s] + D[h] x[b,h,t] ),
 * x = q u, in ascending s.  Equal to the full-length sum with k zero-extended to N taps. */
static void* or_short_points_worker(void* arg) {
    or_job* J = (or_job*)arg;
    const int64_t N = J->N, L = J->L;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[3 * r], h = J->sel[3 * r + 1], t = J->sel[3 * r + 2];
        int64_t off = (b * J->H + h) * N;
        int64_t s0 = t - L + 1 > 0 ? t - L + 1 : 0;
        double a = 0;
        for (int64_t s = s0; s <= t; ++s) {
            double xs = or_load(J->u, J->dt, off + s);
            if (J->q) xs *= or_load(J->q, J->dt, off + s);
            a += or_load(J->k, J->dt, h * L + (t - s)) * xs;
        }
        double xt = or_load(J->u, J->dt, off + t);
        if (J->q) xt *= or_load(J->q, J->dt, off + t);
        double val = a + or_load(J->D, J->dt, h) * xt;
        if (J->v) val *= or_load(J->v, J->dt, off + t);
        J->out[r] = val;
    }
    return NULL;
}

/* y[b,h,t] with a length-L filter for each (b,h,t) in pts[3*npts]; out is [npts]. */
int oracle_conv1d_short_points(const void* u, const void* q, const void* v, const void* k,
                               const void* D, int dt, int64_t B, int64_t H, int64_t N, int64_t L,
                               const int64_t* pts, int64_t npts, double* out, int nthreads) {
    if (or_check1d(u, k, D, pts, npts, out, B, H, N, dt) || L < 1) return -1;
    for (int64_t r = 0; r < npts; ++r)
        if (pts[3 * r] < 0 || pts[3 * r] >= B || pts[3 * r + 1] < 0 || pts[3 * r + 1] >= H ||
            pts[3 * r + 2] < 0 || pts[3 * r + 2] >= N)
            return -1;
    or_job J = {u, q, v, k, D, dt, B, H, N, pts, out, 0, 0, L};
    or_parallel(or_short_points_worker, J, npts, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 1D with a length-M float64 filter, circular (frequency-sparse convolutions)                  */
/* ------------------------------------------------------------------------------------------ */
/* kS[h][0..M) is any real float64 filter of the transform length M >= 2N (for a
 * frequency-sparse convolution: the inverse DFT of the masked filter spectrum).  The output is
 * the length-M circular convolution of the zero-padded x with kS, truncated to N:
 *     y[b,h,t] = v * ( sum_{s=0}^{N-1} kS[h,(t-s) mod M] x[b,h,s] + D[h] x[b,h,t] ),  x = q u,
 * in ascending s.  With kS = k zero-padded this is the causal sum (nothing wraps: M >= 2N). */
typedef struct {
    or_job j;
    const double* kS;
    int64_t M;
} or_circ_job;

static void* or_circ_rows_worker(void* arg) {
    or_circ_job* W = (or_circ_job*)arg;
    const or_job* J = &W->j;
    const int64_t N = J->N, M = W->M;
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[2 * r], h = J->sel[2 * r + 1];
        or_row_x(J, b, h, N, x);
        const double* k = W->kS + h * M;
        double d = or_load(J->D, J->dt, h);
        int64_t off = (b * J->H + h) * N;
        for (int64_t t = 0; t < N; ++t) {
            double a = 0;
            for (int64_t s = 0; s < N; ++s) {
                int64_t m = t - s;
                if (m < 0) m += M;
                a += k[m] * x[s];
            }
            double val = a + d * x[t];
            if (J->v) val *= or_load(J->v, J->dt, off + t);
            J->out[r * N + t] = val;
        }
    }
    free(x);
    return NULL;
}

static void* or_circ_trampoline(void* arg) { return or_circ_rows_worker(arg); }

/* Full rows with a float64 length-M filter kS [H][M] (circular, truncated to N). */
int oracle_conv1d_circ_rows(const void* u, const void* q, const void* v, const double* kS,
                            const void* D, int dt, int64_t B, int64_t H, int64_t N, int64_t M,
                            const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    if (!u || !kS || !D || !out || (nrows > 0 && !rows)) return -1;
    if (B < 1 || H < 1 || N < 1 || M < 2 * N || nrows < 0 || dt < 0 || dt > 2) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= B || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= H)
            return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
    or_circ_job* jobs = (or_circ_job*)calloc((size_t)nthreads, sizeof(or_circ_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int64_t per = (nrows + nthreads - 1) / nthreads;
    int used = 0;
    for (int i = 0; i < nthreads; ++i) {
        int64_t lo = (int64_t)i * per, hi = lo + per < nrows ? lo + per : nrows;
        if (lo >= hi) break;
        or_job J = {u, q, v, NULL, D, dt, B, H, N, rows, out, lo, hi, 0};
        jobs[used].j = J;
        jobs[used].kS = kS;
        jobs[used].M = M;
        pthread_create(&th[used], NULL, or_circ_trampoline, &jobs[used]);
        ++used;
    }
    for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 1D backward (gradients of the causal convolution)                                           */
/* ------------------------------------------------------------------------------------------ */
/*
 * With s = k * x + D x (causal, truncated to N), y = v s and an output gradient gy, the chain
 * rule on the plain definition above gives (ds = gy v):
 *
 *     dx[b,h,t] = sum_{tau=t..N-1} k[h,tau-t] ds[b,h,tau] + D[h] ds[b,h,t]   (correlation)
 *     du = q dx,   dq = u dx,   dv = gy s,
 *     dk[h,tau] = sum_b sum_{t=tau..N-1} ds[b,h,t] x[b,h,t-tau],
 *     dD[h]     = sum_b sum_t ds[b,h,t] x[b,h,t]        (= dk[h,0]: D acts as an extra lag-0 tap)
 *
 * Sums run in ascending index order in double precision, from the exactly widened inputs.
 */
typedef struct {
    or_job j;
    const void* gy;
    double *du, *dq, *dv;
} or_bwd_job;

static void or_row_ds(const or_bwd_job* W, int64_t b, int64_t h, double* ds) {
    const or_job* J = &W->j;
    int64_t off = (b * J->H + h) * J->N;
    or_widen(W->gy, J->dt, off, J->N, ds);
    if (J->v)
        for (int64_t t = 0; t < J->N; ++t) ds[t] *= or_load(J->v, J->dt, off + t);
}

static void* or_bwd_rows_worker(void* arg) {
    or_bwd_job* W = (or_bwd_job*)arg;
    const or_job* J = &W->j;
    const int64_t N = J->N;
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    double* ds = (double*)malloc(sizeof(double) * (size_t)N);
    double* k = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[2 * r], h = J->sel[2 * r + 1];
        int64_t off = (b * J->H + h) * N;
        or_row_x(J, b, h, N, x);
        or_row_ds(W, b, h, ds);
        or_widen(J->k, J->dt, h * N, N, k);
        double d = or_load(J->D, J->dt, h);
        for (int64_t t = 0; t < N; ++t) {
            double a = 0;
            for (int64_t tau = t; tau < N; ++tau) a += k[tau - t] * ds[tau];
            double dx = a + d * ds[t];
            if (W->du) W->du[r * N + t] = J->q ? dx * or_load(J->q, J->dt, off + t) : dx;
            if (W->dq) W->dq[r * N + t] = dx * or_load(J->u, J->dt, off + t);
            if (W->dv) {
                double c = 0;
                for (int64_t s2 = 0; s2 <= t; ++s2) c += k[t - s2] * x[s2];
                W->dv[r * N + t] = or_load(W->gy, J->dt, off + t) * (c + d * x[t]);
            }
        }
    }
    free(x);
    free(ds);
    free(k);
    return NULL;
}

/* Gradient rows for each (b,h) in rows[2*nrows]: du, dq, dv are [nrows][N] (any may be NULL;
 * dq needs q, dv needs v). */
int oracle_conv1d_bwd_rows(const void* u, const void* q, const void* v, const void* k, const void* D,
                           const void* gy, int dt, int64_t B, int64_t H, int64_t N,
                           const int64_t* rows, int64_t nrows, double* du, double* dq, double* dv,
                           int nthreads) {
    if (!u || !k || !D || !gy || (nrows > 0 && !rows)) return -1;
    if (B < 1 || H < 1 || N < 1 || nrows < 0 || dt < 0 || dt > 2) return -1;
    if ((dq && !q) || (dv && !v)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= B || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= H)
            return -1;
    or_bwd_job W;
    or_job J = {u, q, v, k, D, dt, B, H, N, rows, NULL, 0, 0, 0};
    W.j = J;
    W.gy = gy;
    W.du = du;
    W.dq = dq;
    W.dv = dv;
    /* thread the row list by hand (the job carries extra fields) */
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
    or_bwd_job* jobs = (or_bwd_job*)calloc((size_t)nthreads, sizeof(or_bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int64_t per = (nrows + nthreads - 1) / nthreads;
    int used = 0;
    for (int i = 0; i < nthreads; ++i) {
        int64_t lo = (int64_t)i * per, hi = lo + per < nrows ? lo + per : nrows;
        if (lo >= hi) break;
        jobs[used] = W;
        jobs[used].j.lo = lo;
        jobs[used].j.hi = hi;
        pthread_create(&th[used], NULL, or_bwd_rows_worker, &jobs[used]);
        ++used;
    }
    for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* dk[h, 0:N] and dD[h] for each channel h in chans[nch]; dk is [nch][N], dD is [nch]. */
static void* or_dk_worker(void* arg) {
    or_bwd_job* W = (or_bwd_job*)arg;
    const or_job* J = &W->j;
    const int64_t N = J->N, B = J->B;
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    double* ds = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t h = J->sel[r];
        double* dk = W->du + r * N;   /* du carries dk, dq carries dD for this job kind */
        for (int64_t tau = 0; tau < N; ++tau) dk[tau] = 0;
        for (int64_t b = 0; b < B; ++b) {
            or_row_x(J, b, h, N, x);
            or_row_ds(W, b, h, ds);
            for (int64_t tau = 0; tau < N; ++tau) {
                double a = 0;
                for (int64_t t = tau; t < N; ++t) a += ds[t] * x[t - tau];
                dk[tau] += a;
            }
        }
        W->dq[r] = dk[0];
    }
    free(x);
    free(ds);
    return NULL;
}

int oracle_conv1d_bwd_dk(const void* u, const void* q, const void* v, const void* gy, int dt,
                         int64_t B, int64_t H, int64_t N, const int64_t* chans, int64_t nch,
                         double* dk, double* dD, int nthreads) {
    if (!u || !gy || !dk || !dD || (nch > 0 && !chans)) return -1;
    if (B < 1 || H < 1 || N < 1 || nch < 0 || dt < 0 || dt > 2) return -1;
    for (int64_t r = 0; r < nch; ++r)
        if (chans[r] < 0 || chans[r] >= H) return -1;
    or_bwd_job W;
    or_job J = {u, q, v, NULL, NULL, dt, B, H, N, chans, NULL, 0, 0, 0};
    W.j = J;
    W.gy = gy;
    W.du = dk;
    W.dq = dD;
    W.dv = NULL;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nch) nthreads = (int)(nch > 0 ? nch : 1);
    or_bwd_job* jobs = (or_bwd_job*)calloc((size_t)nthreads, sizeof(or_bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int64_t per = (nch + nthreads - 1) / nthreads;
    int used = 0;
    for (int i = 0; i < nthreads; ++i) {
        int64_t lo = (int64_t)i * per, hi = lo + per < nch ? lo + per : nch;
        if (lo >= hi) break;
        jobs[used] = W;
        jobs[used].j.lo = lo;
        jobs[used].j.hi = hi;
        pthread_create(&th[used], NULL, or_dk_worker, &jobs[used]);
        ++used;
    }
    for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* The same gradients at single positions, for sequences too long for full rows.  pts holds
 * (b, h, t) triples for du, dq, dv (each NULL when not wanted); dk_pts holds (h, tau) pairs for
 * dk.  Each value is summed exactly as the row versions above sum it. */
static double or_ds_at(const or_job* J, const void* gy, int64_t off, int64_t t) {
    double d = or_load(gy, J->dt, off + t);
    return J->v ? d * or_load(J->v, J->dt, off + t) : d;
}
static double or_x_at(const or_job* J, int64_t off, int64_t t) {
    double x = or_load(J->u, J->dt, off + t);
    return J->q ? x * or_load(J->q, J->dt, off + t) : x;
}

static void* or_bwd_points_worker(void* arg) {
    or_bwd_job* W = (or_bwd_job*)arg;
    const or_job* J = &W->j;
    const int64_t N = J->N;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[3 * r], h = J->sel[3 * r + 1], t = J->sel[3 * r + 2];
        int64_t off = (b * J->H + h) * N;
        double d = or_load(J->D, J->dt, h);
        double a = 0;
        for (int64_t tau = t; tau < N; ++tau) a += or_load(J->k, J->dt, h * N + (tau - t)) * or_ds_at(J, W->gy, off, tau);
        double dx = a + d * or_ds_at(J, W->gy, off, t);
        if (W->du) W->du[r] = J->q ? dx * or_load(J->q, J->dt, off + t) : dx;
        if (W->dq) W->dq[r] = dx * or_load(J->u, J->dt, off + t);
        if (W->dv) {
            double c = 0;
            for (int64_t s2 = 0; s2 <= t; ++s2) c += or_load(J->k, J->dt, h * N + (t - s2)) * or_x_at(J, off, s2);
            W->dv[r] = or_load(W->gy, J->dt, off + t) * (c + d * or_x_at(J, off, t));
        }
    }
    return NULL;
}

static void* or_dk_points_worker(void* arg) {
    or_bwd_job* W = (or_bwd_job*)arg;
    const or_job* J = &W->j;
    const int64_t N = J->N, B = J->B;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t h = J->sel[2 * r], tau = J->sel[2 * r + 1];
        double acc = 0;
        for (int64_t b = 0; b < B; ++b) {
            int64_t off = (b * J->H + h) * N;
            double a = 0;
            for (int64_t t = tau; t < N; ++t) a += or_ds_at(J, W->gy, off, t) * or_x_at(J, off, t - tau);
            acc += a;
        }
        W->du[r] = acc;
    }
    return NULL;
}

static void or_bwd_parallel(void* (*fn)(void*), or_bwd_job W, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    or_bwd_job* jobs = (or_bwd_job*)calloc((size_t)nthreads, sizeof(or_bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int64_t per = (n + nthreads - 1) / nthreads;
    int used = 0;
    for (int i = 0; i < nthreads; ++i) {
        int64_t lo = (int64_t)i * per, hi = lo + per < n ? lo + per : n;
        if (lo >= hi) break;
        jobs[used] = W;
        jobs[used].j.lo = lo;
        jobs[used].j.hi = hi;
        pthread_create(&th[used], NULL, fn, &jobs[used]);
        ++used;
    }
    for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

int oracle_conv1d_bwd_points(const void* u, const void* q, const void* v, const void* k, const void* D,
                             const void* gy, int dt, int64_t B, int64_t H, int64_t N, const int64_t* pts,
                             int64_t npts, double* du, double* dq, double* dv, int nthreads) {
    if (or_check1d(u, k, D, pts, npts, du ? du : (dq ? dq : dv), B, H, N, dt) || !gy) return -1;
    for (int64_t r = 0; r < npts; ++r)
        if (pts[3 * r] < 0 || pts[3 * r] >= B || pts[3 * r + 1] < 0 || pts[3 * r + 1] >= H ||
            pts[3 * r + 2] < 0 || pts[3 * r + 2] >= N)
            return -1;
    or_bwd_job W;
    or_job J = {u, q, v, k, D, dt, B, H, N, pts, NULL, 0, 0, 0};
    W.j = J;
    W.gy = gy;
    W.du = du;
    W.dq = q ? dq : NULL;
    W.dv = v ? dv : NULL;
    or_bwd_parallel(or_bwd_points_worker, W, npts, nthreads);
    return 0;
}

int oracle_conv1d_bwd_dk_points(const void* u, const void* q, const void* v, const void* gy, int dt,
                                int64_t B, int64_t H, int64_t N, const int64_t* pts, int64_t npts,
                                double* dk, int nthreads) {
    if (!u || !gy || !dk || (npts > 0 && !pts)) return -1;
    if (B < 1 || H < 1 || N < 1 || npts < 0 || dt < 0 || dt > 2) return -1;
    for (int64_t r = 0; r < npts; ++r)
        if (pts[2 * r] < 0 || pts[2 * r] >= H || pts[2 * r + 1] < 0 || pts[2 * r + 1] >= N) return -1;
    or_bwd_job W;
    or_job J = {u, q, v, NULL, NULL, dt, B, H, N, pts, NULL, 0, 0, 0};
    W.j = J;
    W.gy = gy;
    W.du = dk;
    W.dq = NULL;
    W.dv = NULL;
    or_bwd_parallel(or_dk_points_worker, W, npts, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 2D: direct summation at single positions                                                    */
/* ------------------------------------------------------------------------------------------ */

/* Images of Hs x Ws with a kernel of the same size whose centre tap is (Hs/2, Ws/2), halves
 * rounded down (the square S x S case has its centre at (S/2, S/2)):
 *   y[b,c,i,j] = sum_{a,e} k[c,a,e] u[b,c, i + Hs/2 - a, j + Ws/2 - e] + D[c] u[b,c,i,j],
 * summed with a outermost, then e, ascending; out-of-range input taps contribute 0. */
static void* or_points2d_worker(void* arg) {
    or_job* J = (or_job*)arg;
    const int64_t Hs = J->N, Ws = J->L, C = J->H, hh = Hs / 2, hw = Ws / 2;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[4 * r], c = J->sel[4 * r + 1];
        int64_t i = J->sel[4 * r + 2], j = J->sel[4 * r + 3];
        int64_t uoff = (b * C + c) * Hs * Ws, koff = c * Hs * Ws;
        double acc = 0;
        for (int64_t a = 0; a < Hs; ++a) {
            int64_t ii = i + hh - a;
            if (ii < 0 || ii >= Hs) continue;
            for (int64_t e = 0; e < Ws; ++e) {
                int64_t jj = j + hw - e;
                if (jj < 0 || jj >= Ws) continue;
                acc += or_load(J->k, J->dt, koff + a * Ws + e) *
                       or_load(J->u, J->dt, uoff + ii * Ws + jj);
            }
        }
        J->out[r] = acc + or_load(J->D, J->dt, c) * or_load(J->u, J->dt, uoff + i * Ws + j);
    }
    return NULL;
}

int oracle_conv2d_points(const void* u, const void* k, const void* D, int dt, int64_t B,
                         int64_t C, int64_t Hs, int64_t Ws, const int64_t* pts, int64_t npts,
                         double* out, int nthreads) {
    if (!u || !k || !D || !out || (npts > 0 && !pts)) return -1;
    if (B < 1 || C < 1 || Hs < 1 || Ws < 1 || npts < 0 || dt < 0 || dt > 2) return -1;
    for (int64_t r = 0; r < npts; ++r)
        if (pts[4 * r] < 0 || pts[4 * r] >= B || pts[4 * r + 1] < 0 || pts[4 * r + 1] >= C ||
            pts[4 * r + 2] < 0 || pts[4 * r + 2] >= Hs || pts[4 * r + 3] < 0 ||
            pts[4 * r + 3] >= Ws)
            return -1;
    or_job J = {u, NULL, NULL, k, D, dt, B, C, Hs, pts, out, 0, 0, Ws};
    or_parallel(or_points2d_worker, J, npts, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 3D (HyenaND-style, volumes)                                                                  */
/* ------------------------------------------------------------------------------------------ */
/* The 2D definition one dimension up ("Native Multi-Dimensional Subquadratic Operators via Input
 * Dependent Long Convolutions", abstract: global convolutions on the native multi-dimensional
 * grid): a linear convolution with a centred full-size kernel (tap (a,e,f) at offset
 * (a-S/2, e-S/2, f-S/2)), cropped to the input window, plus the skip D u:
 *   y[b,c,i,j,l] = sum_{a,e,f} k[c,a,e,f] u[b,c,i+S/2-a,j+S/2-e,l+S/2-f] + D[c] u[b,c,i,j,l],
 * summed with a outermost, then e, then f, ascending; out-of-range input taps contribute 0. */
static void* or_points3d_worker(void* arg) {
    or_job* J = (or_job*)arg;
    const int64_t S = J->N, C = J->H, half = S / 2;
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[5 * r], c = J->sel[5 * r + 1];
        int64_t i = J->sel[5 * r + 2], j = J->sel[5 * r + 3], l = J->sel[5 * r + 4];
        int64_t uoff = (b * C + c) * S * S * S, koff = c * S * S * S;
        double acc = 0;
        for (int64_t a = 0; a < S; ++a) {
            int64_t ii = i + half - a;
            if (ii < 0 || ii >= S) continue;
            for (int64_t e = 0; e < S; ++e) {
                int64_t jj = j + half - e;
                if (jj < 0 || jj >= S) continue;
                for (int64_t f = 0; f < S; ++f) {
                    int64_t ll = l + half - f;
                    if (ll < 0 || ll >= S) continue;
                    acc += or_load(J->k, J->dt, koff + (a * S + e) * S + f) *
                           or_load(J->u, J->dt, uoff + (ii * S + jj) * S + ll);
                }
            }
        }
        J->out[r] = acc + or_load(J->D, J->dt, c) * or_load(J->u, J->dt, uoff + (i * S + j) * S + l);
    }
    return NULL;
}

/* y[b,c,i,j,l] for each (b,c,i,j,l) in pts[5*npts]; u is [B][C][S][S][S], k is [C][S][S][S],
 * D is [C]. */
int oracle_conv3d_points(const void* u, const void* k, const void* D, int dt, int64_t B,
                         int64_t C, int64_t S, const int64_t* pts, int64_t npts, double* out,
                         int nthreads) {
    if (!u || !k || !D || !out || (npts > 0 && !pts)) return -1;
    if (B < 1 || C < 1 || S < 1 || npts < 0 || dt < 0 || dt > 2) return -1;
    for (int64_t r = 0; r < npts; ++r) {
        const int64_t* p = pts + 5 * r;
        if (p[0] < 0 || p[0] >= B || p[1] < 0 || p[1] >= C) return -1;
        for (int d = 2; d < 5; ++d)
            if (p[d] < 0 || p[d] >= S) return -1;
    }
    or_job J = {u, NULL, NULL, k, D, dt, B, C, S, pts, out, 0, 0, 0};
    or_parallel(or_points3d_worker, J, npts, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Diagonal state-space filters (FlashConv page, Mechanism: state passed between chunks)        */
/* ------------------------------------------------------------------------------------------ */
/* A channel's filter is generated by NS complex modes: k[h,t] = Re sum_n W[h,n] lam[h,n]^t.  The
 * convolution with it is the state recurrence run forward in time,
 *     s_n[t] = lam_n s_n[t-1] + x[t]   (s_n[-1] = 0),    y[t] = Re sum_n W_n s_n[t] + D x[t],
 * x = q u, then y *= v; this evaluates it that way (float64 complex, t ascending).  lam and W
 * are float64 complex [H][NS] (interleaved re, im). */
typedef struct {
    or_job j;
    const double *lam, *W;
    int64_t NS;
} or_ssm_job;

static void* or_ssm_rows_worker(void* arg) {
    or_ssm_job* S = (or_ssm_job*)arg;
    const or_job* J = &S->j;
    const int64_t N = J->N, NS = S->NS;
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    double* sr = (double*)malloc(sizeof(double) * (size_t)NS);
    double* si = (double*)malloc(sizeof(double) * (size_t)NS);
    for (int64_t r = J->lo; r < J->hi; ++r) {
        int64_t b = J->sel[2 * r], h = J->sel[2 * r + 1];
        or_row_x(J, b, h, N, x);
        const double* lam = S->lam + 2 * h * NS;
        const double* W = S->W + 2 * h * NS;
        double d = or_load(J->D, J->dt, h);
        int64_t off = (b * J->H + h) * N;
        for (int64_t n = 0; n < NS; ++n) sr[n] = si[n] = 0;
        for (int64_t t = 0; t < N; ++t) {
            double acc = 0;
            for (int64_t n = 0; n < NS; ++n) {
                const double lr = lam[2 * n], li = lam[2 * n + 1];
                const double nr = lr * sr[n] - li * si[n] + x[t];
                const double ni = lr * si[n] + li * sr[n];
                sr[n] = nr;
                si[n] = ni;
                acc += W[2 * n] * nr - W[2 * n + 1] * ni;
            }
            double val = acc + d * x[t];
            if (J->v) val *= or_load(J->v, J->dt, off + t);
            J->out[r * N + t] = val;
        }
    }
    free(x);
    free(sr);
    free(si);
    return NULL;
}

static void* or_ssm_trampoline(void* arg) { return or_ssm_rows_worker(arg); }

/* Full rows of the convolution with the state-space filter (lam, W), by the recurrence. */
int oracle_ssm_rows(const void* u, const void* q, const void* v, const double* lam, const double* W,
                    const void* D, int dt, int64_t B, int64_t H, int64_t N, int64_t NS,
                    const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    if (!u || !lam || !W || !D || !out || (nrows > 0 && !rows)) return -1;
    if (B < 1 || H < 1 || N < 1 || NS < 1 || nrows < 0 || dt < 0 || dt > 2) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= B || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= H)
            return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
    or_ssm_job* jobs = (or_ssm_job*)calloc((size_t)nthreads, sizeof(or_ssm_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int64_t per = (nrows + nthreads - 1) / nthreads;
    int used = 0;
    for (int i = 0; i < nthreads; ++i) {
        int64_t lo = (int64_t)i * per, hi = lo + per < nrows ? lo + per : nrows;
        if (lo >= hi) break;
        or_job J = {u, q, v, NULL, D, dt, B, H, N, rows, out, lo, hi, 0};
        jobs[used].j = J;
        jobs[used].lam = lam;
        jobs[used].W = W;
        jobs[used].NS = NS;
        pthread_create(&th[used], NULL, or_ssm_trampoline, &jobs[used]);
        ++used;
    }
    for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

