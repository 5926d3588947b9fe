/* Drives every oracle entry point on exact-size heap buffers, for the three
 * dtypes and edge shapes (no rows, one column, ragged widths), so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build reports any access
 * outside a buffer or any undefined arithmetic. Test infrastructure: linked
 * with oracle/oracle.c by tests/test_host_sanitizers.py only. Exit status 0
 * when every call returned 0 and every result is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_encode(const double *src, int64_t n, int dtype, void *dst);
int orc_decode(const void *src, int64_t n, int dtype, double *dst);
int orc_elem_bytes(int dtype);
int orc_rmsnorm_fwd(const void *x, const void *gamma, int dtype, int64_t M, int64_t N, double eps,
                    float *rstd, double *y);
int orc_fused_add_rmsnorm_fwd(const void *x, const void *residual, const void *gamma, int dtype, int64_t M,
                              int64_t N, double eps, void *added, float *rstd, double *out);
int orc_rmsnorm_bwd(const void *x, const void *gamma, const void *dy, const float *rstd, int dtype, int64_t M,
                    int64_t N, double *dx, double *dgamma);
int orc_fused_add_rmsnorm_bwd(const void *added, const void *gamma, const void *dy, const void *dresidual_out,
                              const float *rstd, int dtype, int64_t M, int64_t N, double *dx, double *dgamma);
int orc_layernorm_fwd(const void *x, const void *gamma, const void *beta, int dtype, int64_t M, int64_t N,
                      double eps, float *mean, float *rstd, double *y);
int orc_layernorm_bwd(const void *x, const void *gamma, const void *dy, const float *mean, const float *rstd,
                      int dtype, int64_t M, int64_t N, double *dx, double *dgamma, double *dbeta);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double draw(void) { /* xorshift64*, uniform in (-2, 2) */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return ((double)((state * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0) * 4.0 - 2.0;
}

/* a buffer of exactly n elements of dtype (NULL when n == 0, as a caller may pass) */
static void *tensor(int dtype, int64_t n) {
    if (n == 0) return NULL;
    double *v = malloc((size_t)n * sizeof(double));
    void *t = malloc((size_t)n * (size_t)orc_elem_bytes(dtype));
    for (int64_t i = 0; i < n; ++i) v[i] = draw();
    if (orc_encode(v, n, dtype, t)) exit(10);
    free(v);
    return t;
}

static int finite_all(const double *v, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

int main(void) {
    static const int64_t shapes[][2] = {{0, 1}, {0, 9}, {1, 1}, {3, 7}, {2, 64}, {5, 257}, {1, 3001}};
    int failures = 0;
    for (int dtype = 0; dtype < 3; ++dtype) {
        for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
            const int64_t M = shapes[s][0], N = shapes[s][1], MN = M * N;
            void *x = tensor(dtype, MN), *res = tensor(dtype, MN), *dy = tensor(dtype, MN);
            void *dres = tensor(dtype, MN), *gamma = tensor(dtype, N), *beta = tensor(dtype, N);
            float *rstd = malloc((size_t)(M ? M : 1) * sizeof(float));
            float *mean = malloc((size_t)(M ? M : 1) * sizeof(float));
            double *y = malloc((size_t)(MN ? MN : 1) * sizeof(double));
            double *dx = malloc((size_t)(MN ? MN : 1) * sizeof(double));
            double *dg = malloc((size_t)N * sizeof(double)), *db = malloc((size_t)N * sizeof(double));
            void *added = MN ? malloc((size_t)MN * (size_t)orc_elem_bytes(dtype)) : NULL;
            int rc = 0;
            rc |= orc_rmsnorm_fwd(x, gamma, dtype, M, N, 1e-5, rstd, y);
            rc |= !finite_all(y, MN);
            rc |= orc_rmsnorm_bwd(x, gamma, dy, rstd, dtype, M, N, dx, dg);
            rc |= !finite_all(dx, MN) || !finite_all(dg, N);
            rc |= orc_fused_add_rmsnorm_fwd(x, res, gamma, dtype, M, N, 1e-6, added, rstd, y);
            rc |= orc_fused_add_rmsnorm_bwd(added, gamma, dy, dres, rstd, dtype, M, N, dx, dg);
            rc |= !finite_all(dx, MN) || !finite_all(dg, N);
            rc |= orc_fused_add_rmsnorm_bwd(added, gamma, dy, NULL, rstd, dtype, M, N, dx, dg);
            rc |= orc_layernorm_fwd(x, gamma, beta, dtype, M, N, 1e-5, mean, rstd, y);
            rc |= orc_layernorm_fwd(x, gamma, NULL, dtype, M, N, 1e-5, mean, rstd, y);
            rc |= !finite_all(y, MN);
            rc |= orc_layernorm_bwd(x, gamma, dy, mean, rstd, dtype, M, N, dx, dg, db);
            rc |= !finite_all(dx, MN) || !finite_all(dg, N) || !finite_all(db, N);
            if (rc) {
                fprintf(stderr, "failed: dtype %d, M %lld, N %lld\n", dtype, (long long)M, (long long)N);
                ++failures;
            }
            free(x); free(res); free(dy); free(dres); free(gamma); free(beta); free(rstd); free(mean);
            free(y); free(dx); free(dg); free(db); free(added);
        }
    }
    printf("oracle driver: %d failing cases\n", failures);
    return failures ? 1 : 0;
}
