/*
 * oracle.c - plain, slow, obviously-correct CPU reference for RMSNorm with a
 * saved per-row rstd, its backward, and the fused-add (prenorm residual)
 * variants of both; and for LayerNorm with saved mean and rstd and its
 * backward with the bias gradient.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file. The GPU library never links
 * it, and it shares nothing with the GPU library: the dtype decode/encode
 * routines, the loops and the arithmetic below are all written here from the
 * definitions, in fp64, single-threaded, rows in ascending order, columns in
 * ascending order.
 *
 * Pages cited, by title:
 *   [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
 *          rstd) to enable training / downstream (quack) integration"
 *   [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
 *          (PR 2/3, #769)" - its three commit messages and the PR body
 *   [P854] FlyDSL PR #854, "[Test] Expand RMSNorm backward configs, cache
 *          reuse, and Torch benchmarks"
 *
 * Readings taken where the pages leave a step open (each is also listed in the
 * design notes of the repository):
 *   - converting an fp32 result back to the I/O dtype rounds to nearest,
 *     ties to even (RNE); a NaN encodes as a quiet NaN.
 *   - the fused forward forms added = x + residual as one fp32 addition, then
 *     one RNE to the I/O dtype; rstd is taken over that stored, rounded added,
 *     which is also what the backward reads.
 *   - the backward uses the fp32 rstd exactly as stored by a forward (the same
 *     array the GPU path reads), widened exactly to fp64.
 *   - c1 divides by N (a mean over the row).
 *   - a NULL dresidual_out stands for a tensor of zeros.
 *   - LayerNorm is the textbook one: biased variance (divisor N), eps inside
 *     the square root, y = x_hat * gamma + beta; a NULL beta is zeros; the
 *     backward reads the fp32 mean and rstd a forward saved.
 *
 * Parity pins (tests marked "not gpu"): central finite differences of the
 * forward, an explicit O(N^2) Jacobian, float64 torch.autograd on the CPU,
 * closed forms (N = 1, constant rows, dy = 0, M = 1), the orthogonality
 * identity sum_j x_hat_j dx_j = N c1 eps r^3, scale and linearity
 * invariants, and the encode/decode routines against torch's conversions.
 * LayerNorm: hand-derived worked examples, float64 torch layer_norm
 * autograd, finite differences, the shift invariance sum_j dx_j = 0, and the
 * reduction to the RMSNorm backward on zero-mean rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's own dtype codes. They happen to carry the same numbers as the
 * GPU library's, but nothing is shared; the Python wrapper maps names. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2 };

/* ------------------------------------------------------------------------ */
/* Binary floating-point formats, from the IEEE 754 definition.              */
/* ------------------------------------------------------------------------ */

struct fmt {
    int mbits; /* stored mantissa (fraction) bits */
    int ebits; /* exponent bits */
};

static const struct fmt FMT_F32 = {23, 8};
static const struct fmt FMT_F16 = {10, 5};
static const struct fmt FMT_BF16 = {7, 8};

static int fmt_of(int dtype, struct fmt *f)
{
    switch (dtype) {
    case ORC_F32: *f = FMT_F32; return 0;
    case ORC_F16: *f = FMT_F16; return 0;
    case ORC_BF16: *f = FMT_BF16; return 0;
    default: return -1;
    }
}

static size_t elem_bytes(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* Exact value of an encoded pattern: (-1)^s * 2^(e - bias) * 1.m for normal
 * numbers, (-1)^s * 2^(1 - bias) * 0.m for subnormals. */
static double decode_bits(uint32_t bits, struct fmt f)
{
    uint32_t mmask = (1u << f.mbits) - 1u;
    uint32_t emax = (1u << f.ebits) - 1u;
    int bias = (1 << (f.ebits - 1)) - 1;
    uint32_t sign = (bits >> (f.mbits + f.ebits)) & 1u;
    uint32_t e = (bits >> f.mbits) & emax;
    uint32_t m = bits & mmask;
    double v;
    if (e == emax)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, 1 - bias - f.mbits);
    else
        v = ldexp((double)(m | (1u << f.mbits)), (int)e - bias - f.mbits);
    return sign ? -v : v;
}

/* Round v to the nearest value of format f, ties to even, and return its
 * encoding. The quantum of the binade [2^e, 2^(e+1)) is 2^(e - mbits);
 * subnormals share the quantum of the smallest normal binade. v / quantum is
 * rounded to an integer with nearbyint() under the default (to-nearest-even)
 * mode. A result at or past the all-ones exponent is infinity. */
static uint32_t encode_bits(double v, struct fmt f)
{
    uint32_t emax = (1u << f.ebits) - 1u;
    int bias = (1 << (f.ebits - 1)) - 1;
    uint32_t sign = signbit(v) ? 1u : 0u;
    uint32_t sbit = sign << (f.mbits + f.ebits);
    double a = fabs(v);
    int e;
    uint64_t q, bits;

    if (isnan(v))
        return sbit | (emax << f.mbits) | (1u << (f.mbits - 1));
    if (isinf(a))
        return sbit | (emax << f.mbits);
    if (a == 0.0)
        return sbit;
    (void)frexp(a, &e); /* a = fr * 2^e with fr in [0.5, 1) */
    e -= 1;             /* now a lies in [2^e, 2^(e+1)) */
    if (e < 1 - bias)
        e = 1 - bias;
    q = (uint64_t)nearbyint(ldexp(a, f.mbits - e));
    /* normal: biased exponent (e + bias), fraction q - 2^mbits; a carry of q to
     * 2^(mbits+1) bumps the exponent field by itself. Subnormal (e = 1 - bias,
     * q < 2^mbits): exponent field 0, fraction q. Both are this one sum. */
    bits = ((uint64_t)(e + bias - 1) << f.mbits) + q;
    if (bits >= ((uint64_t)emax << f.mbits))
        bits = (uint64_t)emax << f.mbits;
    return sbit | (uint32_t)bits;
}

/* A bf16 pattern is the upper half of the fp32 pattern of the same value, so
 * widening it is a shift; the same result as decode_bits, much faster. */
static double up_bf16(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Exact widening of element i of a typed array to fp64 ("up" in the notes). */
static double up(const void *p, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_F16: return decode_bits(((const uint16_t *)p)[i], FMT_F16);
    default: return up_bf16(((const uint16_t *)p)[i]);
    }
}

/* Store v, rounded once (RNE) to the dtype, as element i of a typed array. */
static void store_rne(void *p, int dtype, int64_t i, double v)
{
    switch (dtype) {
    case ORC_F32: ((float *)p)[i] = (float)v; break; /* C's conversion is RNE */
    case ORC_F16: ((uint16_t *)p)[i] = (uint16_t)encode_bits(v, FMT_F16); break;
    default: ((uint16_t *)p)[i] = (uint16_t)encode_bits(v, FMT_BF16); break;
    }
}

/* ------------------------------------------------------------------------ */
/* Conversions exported for tests.                                           */
/* ------------------------------------------------------------------------ */

int orc_decode(const void *src, int64_t n, int dtype, double *dst)
{
    struct fmt f;
    if (fmt_of(dtype, &f) || n < 0 || (n && (!src || !dst)))
        return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = up(src, dtype, i);
    return ORC_OK;
}

int orc_encode(const double *src, int64_t n, int dtype, void *dst)
{
    struct fmt f;
    if (fmt_of(dtype, &f) || n < 0 || (n && (!src || !dst)))
        return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        store_rne(dst, dtype, i, src[i]);
    return ORC_OK;
}

/* Same rounding as orc_encode but through the generic encoder for every
 * dtype, fp32 included, so a test can hold the encoder against C's own
 * double-to-float conversion. Returns raw bit patterns, one uint32 each. */
int orc_encode_bits(const double *src, int64_t n, int dtype, uint32_t *dst)
{
    struct fmt f;
    if (fmt_of(dtype, &f) || n < 0 || (n && (!src || !dst)))
        return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = encode_bits(src[i], f);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Forward passes that save rstd.                                            */
/* ------------------------------------------------------------------------ */

/* One row of the RMSNorm forward over an already-typed row a[0..N).
 * [I769] Implementation plan (current state): the forward's per-row
 * rrms = rsqrt(mean(x^2) + eps), output x * rrms * gamma.
 * [P800] PR-1 commit: the saved rstd is 1/RMS, fp32, one value per row. */
static void fwd_row(const void *a, int dtype, int64_t row, const void *gamma,
                    int64_t N, double eps, float *rstd, double *y)
{
    double sumsq = 0.0, r;
    for (int64_t j = 0; j < N; ++j) {
        double v = up(a, dtype, row * N + j);
        sumsq += v * v;
    }
    r = 1.0 / sqrt(sumsq / (double)N + eps);
    rstd[row] = (float)r;
    if (y)
        for (int64_t j = 0; j < N; ++j)
            y[row * N + j] = up(a, dtype, row * N + j) * r * up(gamma, dtype, j);
}

static int check_common(const void *gamma, int dtype, int64_t M, int64_t N, double eps)
{
    struct fmt f;
    if (fmt_of(dtype, &f) || M < 0 || N < 1 || !gamma || !(eps >= 0.0) || isinf(eps))
        return ORC_EINVAL;
    return ORC_OK;
}

/* Plain forward. Outputs: rstd (M fp32, required) and y (M*N fp64, unrounded,
 * nullable). */
int orc_rmsnorm_fwd(const void *x, const void *gamma, int dtype, int64_t M,
                    int64_t N, double eps, float *rstd, double *y)
{
    if (check_common(gamma, dtype, M, N, eps) || (M && (!x || !rstd)))
        return ORC_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        fwd_row(x, dtype, i, gamma, N, eps, rstd, y);
    return ORC_OK;
}

/* Fused-add forward. [P800] fused-add commit and PR body: added = x + residual
 * is returned as residual_out, and the rstd of added is saved. The sum is one
 * fp32 addition rounded once to the I/O dtype; the statistics and the output
 * are taken over that stored, rounded added. Outputs: added (M*N, I/O dtype,
 * required), rstd (M fp32, required), out (M*N fp64 unrounded, nullable). */
int orc_fused_add_rmsnorm_fwd(const void *x, const void *residual, const void *gamma,
                              int dtype, int64_t M, int64_t N, double eps,
                              void *added, float *rstd, double *out)
{
    if (check_common(gamma, dtype, M, N, eps) ||
        (M && (!x || !residual || !added || !rstd)))
        return ORC_EINVAL;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t k = i * N + j;
            float s = (float)up(x, dtype, k) + (float)up(residual, dtype, k);
            store_rne(added, dtype, k, (double)s);
        }
        fwd_row(added, dtype, i, gamma, N, eps, rstd, out);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward passes.                                                          */
/* ------------------------------------------------------------------------ */

/* One row of the RMSNorm backward. [I769] Implementation plan, Math: with
 * x_hat = x * rstd and wdy = dy * gamma, c1 = mean over the N columns of
 * x_hat * wdy, dx = (wdy - x_hat * c1) * rstd, and dweight gains dy * x_hat.
 * dx_row (N fp64) and dgamma (N fp64, accumulated) are nullable. */
static void bwd_row(const void *x, const void *gamma, const void *dy, float rstd_i,
                    int dtype, int64_t row, int64_t N, double *dx_row, double *dgamma)
{
    double r = (double)rstd_i;
    double c1 = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double x_hat = up(x, dtype, row * N + j) * r;
        double wdy = up(dy, dtype, row * N + j) * up(gamma, dtype, j);
        c1 += x_hat * wdy;
    }
    c1 /= (double)N;
    for (int64_t j = 0; j < N; ++j) {
        double x_hat = up(x, dtype, row * N + j) * r;
        double dyj = up(dy, dtype, row * N + j);
        double wdy = dyj * up(gamma, dtype, j);
        if (dx_row)
            dx_row[j] = (wdy - x_hat * c1) * r;
        if (dgamma)
            dgamma[j] += dyj * x_hat;
    }
}

/* Plain backward. Inputs x, gamma, dy (I/O dtype), rstd (M fp32 as saved by a
 * forward). Outputs (each nullable): dx (M*N fp64, unrounded) and dgamma (N
 * fp64, the sum over all M rows; overwritten, zero when M = 0). */
int orc_rmsnorm_bwd(const void *x, const void *gamma, const void *dy, const float *rstd,
                    int dtype, int64_t M, int64_t N, double *dx, double *dgamma)
{
    if (check_common(gamma, dtype, M, N, 0.0) || (M && (!x || !dy || !rstd)))
        return ORC_EINVAL;
    if (dgamma)
        for (int64_t j = 0; j < N; ++j)
            dgamma[j] = 0.0;
    for (int64_t i = 0; i < M; ++i)
        bwd_row(x, gamma, dy, rstd[i], dtype, i, N, dx ? dx + i * N : NULL, dgamma);
    return ORC_OK;
}

/* Fused-add backward. [P800] fused-add commit and PR body: d_added =
 * (wdy - a_hat * c1) * rstd is the plain backward taken over added, the total
 * is d_added + dresidual_out, and that one total is both dx and dresidual,
 * because added = x + residual. dresidual_out may be NULL (zeros). dweight
 * is the plain dweight over added. */
int orc_fused_add_rmsnorm_bwd(const void *added, const void *gamma, const void *dy,
                              const void *dresidual_out, const float *rstd, int dtype,
                              int64_t M, int64_t N, double *dx, double *dgamma)
{
    if (check_common(gamma, dtype, M, N, 0.0) || (M && (!added || !dy || !rstd)))
        return ORC_EINVAL;
    if (dgamma)
        for (int64_t j = 0; j < N; ++j)
            dgamma[j] = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        double *d_added = dx ? dx + i * N : NULL;
        bwd_row(added, gamma, dy, rstd[i], dtype, i, N, d_added, dgamma);
        if (d_added && dresidual_out)
            for (int64_t j = 0; j < N; ++j)
                d_added[j] += up(dresidual_out, dtype, i * N + j);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* LayerNorm: forward that saves mean and rstd, backward with dbias.         */
/* ------------------------------------------------------------------------ */

/* [I769] PR sequence and status updates: the LayerNorm follow-up mirrors the
 * RMSNorm backward with mean handling and a bias gradient, and its forward
 * saves mean and rstd (fp32). Taken here as the textbook layer norm over the
 * N columns of a row: mean = (1/N) sum x, var = (1/N) sum (x - mean)^2
 * (the biased variance), rstd = 1/sqrt(var + eps),
 * y = (x - mean) * rstd * gamma + beta. Outputs: mean, rstd (M fp32,
 * required), y (M*N fp64 unrounded, nullable). beta may be NULL (zeros). */
int orc_layernorm_fwd(const void *x, const void *gamma, const void *beta, int dtype,
                      int64_t M, int64_t N, double eps, float *mean, float *rstd, double *y)
{
    if (check_common(gamma, dtype, M, N, eps) || (M && (!x || !mean || !rstd)))
        return ORC_EINVAL;
    for (int64_t i = 0; i < M; ++i) {
        double mu = 0.0, var = 0.0, r;
        for (int64_t j = 0; j < N; ++j)
            mu += up(x, dtype, i * N + j);
        mu /= (double)N;
        for (int64_t j = 0; j < N; ++j) {
            double d = up(x, dtype, i * N + j) - mu;
            var += d * d;
        }
        var /= (double)N;
        r = 1.0 / sqrt(var + eps);
        mean[i] = (float)mu;
        rstd[i] = (float)r;
        if (y)
            for (int64_t j = 0; j < N; ++j) {
                double v = (up(x, dtype, i * N + j) - mu) * r * up(gamma, dtype, j);
                y[i * N + j] = beta ? v + up(beta, dtype, j) : v;
            }
    }
    return ORC_OK;
}

/* The LayerNorm backward, from the definition above, with the fp32 mean and
 * rstd a forward saved (widened exactly). Per row, with
 * x_hat = (x - mean) * rstd and wdy = dy * gamma:
 *   c1 = (1/N) sum x_hat * wdy, c2 = (1/N) sum wdy,
 *   dx = (wdy - x_hat * c1 - c2) * rstd,
 * and over all rows dgamma = sum dy * x_hat, dbeta = sum dy.
 * Outputs (each nullable): dx (M*N fp64 unrounded), dgamma, dbeta (N fp64,
 * overwritten; zero when M = 0). */
int orc_layernorm_bwd(const void *x, const void *gamma, const void *dy, const float *mean,
                      const float *rstd, int dtype, int64_t M, int64_t N, double *dx,
                      double *dgamma, double *dbeta)
{
    if (check_common(gamma, dtype, M, N, 0.0) || (M && (!x || !dy || !mean || !rstd)))
        return ORC_EINVAL;
    for (int64_t j = 0; j < N; ++j) {
        if (dgamma)
            dgamma[j] = 0.0;
        if (dbeta)
            dbeta[j] = 0.0;
    }
    for (int64_t i = 0; i < M; ++i) {
        double mu = (double)mean[i], r = (double)rstd[i];
        double c1 = 0.0, c2 = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double x_hat = (up(x, dtype, i * N + j) - mu) * r;
            double wdy = up(dy, dtype, i * N + j) * up(gamma, dtype, j);
            c1 += x_hat * wdy;
            c2 += wdy;
        }
        c1 /= (double)N;
        c2 /= (double)N;
        for (int64_t j = 0; j < N; ++j) {
            double x_hat = (up(x, dtype, i * N + j) - mu) * r;
            double dyj = up(dy, dtype, i * N + j);
            double wdy = dyj * up(gamma, dtype, j);
            if (dx)
                dx[i * N + j] = (wdy - x_hat * c1 - c2) * r;
            if (dgamma)
                dgamma[j] += dyj * x_hat;
            if (dbeta)
                dbeta[j] += dyj;
        }
    }
    return ORC_OK;
}

/* Element size, so the Python wrapper can check buffer lengths. */
int orc_elem_bytes(int dtype)
{
    struct fmt f;
    return fmt_of(dtype, &f) ? ORC_EINVAL : (int)elem_bytes(dtype);
}
