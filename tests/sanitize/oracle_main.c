/* The float64 oracle under the address and undefined-behaviour sanitizers: every exported sum on
 * small shapes with ragged edges (first and last positions, every gate combination, several
 * threads), plus a delta-input check on each family so a wrong result is reported too.  Exit
 * status 0 when every call accepts its arguments and every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_conv1d_rows(const void*, const void*, const void*, const void*, const void*, int, int64_t, int64_t,
                       int64_t, const int64_t*, int64_t, double*, int);
int oracle_conv1d_points(const void*, const void*, const void*, const void*, const void*, int, int64_t, int64_t,
                         int64_t, const int64_t*, int64_t, double*, int);
int oracle_conv1d_short_points(const void*, const void*, const void*, const void*, const void*, int, int64_t,
                               int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, int);
int oracle_conv1d_circ_rows(const void*, const void*, const void*, const double*, const void*, int, int64_t,
                            int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, int);
int oracle_conv1d_bwd_rows(const void*, const void*, const void*, const void*, const void*, const void*, int,
                           int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, double*, double*, int);
int oracle_conv1d_bwd_dk(const void*, const void*, const void*, const void*, int, int64_t, int64_t, int64_t,
                         const int64_t*, int64_t, double*, double*, int);
int oracle_conv1d_bwd_points(const void*, const void*, const void*, const void*, const void*, const void*, int,
                             int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, double*, double*, int);
int oracle_conv1d_bwd_dk_points(const void*, const void*, const void*, const void*, int, int64_t, int64_t,
                                int64_t, const int64_t*, int64_t, double*, int);
int oracle_conv2d_points(const void*, const void*, const void*, int, int64_t, int64_t, int64_t, int64_t,
                         const int64_t*, int64_t, double*, int);
int oracle_conv3d_points(const void*, const void*, const void*, int, int64_t, int64_t, int64_t, const int64_t*,
                         int64_t, double*, int);
int oracle_ssm_rows(const void*, const void*, const void*, const double*, const double*, const void*, int,
                    int64_t, int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, int);
void oracle_widen(const void*, int, int64_t, double*);

static int fails = 0;
#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            fprintf(stderr, "line %d: %s\n", __LINE__, #c);       \
            ++fails;                                              \
        }                                                         \
    } while (0)

static float* randf(int64_t n, unsigned* s) {
    float* a = malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        *s = *s * 1664525u + 1013904223u;
        a[i] = (float)((int)(*s >> 9) % 17 - 8) / 8.0f;
    }
    return a;
}

int main(void) {
    unsigned s = 7;
    enum { B = 3, H = 2, N = 37, F32 = 0 };
    float *u = randf(B * H * N, &s), *q = randf(B * H * N, &s), *v = randf(B * H * N, &s);
    float *k = randf(H * N, &s), *D = randf(H, &s), *gy = randf(B * H * N, &s);
    int64_t rows[B * H * 2];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) { rows[2 * (b * H + h)] = b; rows[2 * (b * H + h) + 1] = h; }
    double* y = malloc(sizeof(double) * B * H * N);
    int64_t pts[3 * 6] = {0, 0, 0, 2, 1, N - 1, 1, 0, N / 2, 2, 0, 1, 0, 1, N - 2, 1, 1, 5};
    double p[6], du[B * H * N], dq[B * H * N], dv[B * H * N], dk[H * N], dD[H];
    const void* gq[2] = {NULL, q};
    const void* gv[2] = {NULL, v};
    for (int g = 0; g < 4; ++g) {
        const void *qq = gq[g & 1], *vv = gv[g >> 1];
        CHECK(oracle_conv1d_rows(u, qq, vv, k, D, F32, B, H, N, rows, B * H, y, 3) == 0);
        CHECK(oracle_conv1d_points(u, qq, vv, k, D, F32, B, H, N, pts, 6, p, 2) == 0);
        for (int i = 0; i < 6; ++i) CHECK(p[i] == y[(pts[3 * i] * H + pts[3 * i + 1]) * N + pts[3 * i + 2]]);
        CHECK(oracle_conv1d_short_points(u, qq, vv, k, D, F32, B, H, N, 5, pts, 6, p, 2) == 0);
        CHECK(oracle_conv1d_bwd_rows(u, qq, vv, k, D, gy, F32, B, H, N, rows, B * H, du, qq ? dq : NULL,
                                     vv ? dv : NULL, 3) == 0);
        CHECK(oracle_conv1d_bwd_points(u, qq, vv, k, D, gy, F32, B, H, N, pts, 6, p, NULL, NULL, 2) == 0);
        CHECK(oracle_conv1d_bwd_dk(u, qq, vv, gy, F32, B, H, N, rows + 1, 1, dk, dD, 2) == 0);
        int64_t kp[4] = {0, 0, 1, N - 1};
        CHECK(oracle_conv1d_bwd_dk_points(u, qq, vv, gy, F32, B, H, N, kp, 2, p, 2) == 0);
    }
    /* a delta input reproduces the filter */
    float* e0 = calloc(N, sizeof(float));
    float zero = 0.f;
    e0[0] = 1.f;
    int64_t r0[2] = {0, 0};
    CHECK(oracle_conv1d_rows(e0, NULL, NULL, k, &zero, F32, 1, 1, N, r0, 1, y, 1) == 0);
    for (int t = 0; t < N; ++t) CHECK(y[t] == (double)k[t]);
    double* kS = calloc(2 * H * 2 * N, sizeof(double));
    CHECK(oracle_conv1d_circ_rows(u, q, v, kS, D, F32, B, H, N, 2 * N, rows, B * H, y, 2) == 0);
    /* 2D (rectangular, odd rows) and 3D */
    enum { S2h = 5, S2w = 8, S3 = 4 };
    float *u2 = randf(2 * 2 * S2h * S2w, &s), *k2 = randf(2 * S2h * S2w, &s);
    int64_t p2[4 * 3] = {0, 0, 0, 0, 1, 1, S2h - 1, S2w - 1, 1, 0, 2, 3};
    CHECK(oracle_conv2d_points(u2, k2, D, F32, 2, 2, S2h, S2w, p2, 3, p, 2) == 0);
    float *u3 = randf(2 * 2 * S3 * S3 * S3, &s), *k3 = randf(2 * S3 * S3 * S3, &s);
    int64_t p3[5 * 2] = {0, 0, 0, 0, 0, 1, 1, S3 - 1, S3 - 1, S3 - 1};
    CHECK(oracle_conv3d_points(u3, k3, D, F32, 2, 2, S3, p3, 2, p, 2) == 0);
    /* state-space rows */
    double lam[2 * H * 3], Wm[2 * H * 3];
    for (int i = 0; i < 2 * H * 3; ++i) { lam[i] = 0.5 / (1 + i); Wm[i] = 1.0 / (2 + i); }
    CHECK(oracle_ssm_rows(u, q, v, lam, Wm, D, F32, B, H, N, 3, rows, B * H, y, 3) == 0);
    /* argument checks reject out-of-range selections */
    int64_t bad[2] = {B, 0};
    CHECK(oracle_conv1d_rows(u, NULL, NULL, k, D, F32, B, H, N, bad, 1, y, 1) != 0);
    double w[4];
    uint16_t half[4] = {0x3c00, 0x8001, 0x7bff, 0x0400};
    oracle_widen(half, 1, 4, w);
    CHECK(w[0] == 1.0 && w[2] == 65504.0);
    free(u); free(q); free(v); free(k); free(D); free(gy); free(y); free(e0); free(kS);
    free(u2); free(k2); free(u3); free(k3);
    if (fails) fprintf(stderr, "%d failures\n", fails);
    else printf("ORACLE_SANITIZED_OK\n");
    return fails ? 1 : 0;
}
