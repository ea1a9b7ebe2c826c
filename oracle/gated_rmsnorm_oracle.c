/*
 * FP64 CPU oracle for the SiLU-gated RMSNorm training forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP library; it is written straight from the definition, plainly and
 * slowly, in double precision, so that a reader can check it by eye.
 *
 * What it computes.  The operator is the "SiLU-gated RMSNorm" of flashinfer
 * PR #8701, "perf(cake_rmsnorm_silu_gate_train): L2-prefetching
 * extra-long forward on SM107" (PR description: the training kernel with a
 * forward and a backward; commit 10c6017 message: inputs x and the gate z,
 * rows packed; "How the tables were measured": BF16 inputs, a comparator
 * that evaluates the formula in FP32, a BF16 or an FP32 weight gradient).
 * The page prints no formula.
 * The plainest reading of the name, used here, normalises each row of D
 * values by its root mean square, scales by a weight w shared by all rows,
 * and gates elementwise with SiLU of z (called g below):
 *
 *     ms_i  = (1/D) sum_j x_ij^2
 *     r_i   = 1 / sqrt(ms_i + eps)
 *     n_ij  = x_ij r_i
 *     s_ij  = silu(g_ij) = g_ij sigma(g_ij)
 *     y_ij  = n_ij w_j s_ij
 *
 * The backward is the exact derivative of L = sum_ij dy_ij y_ij:
 *
 *     dg_ij = dy_ij w_j n_ij sigma_ij (1 + g_ij (1 - sigma_ij))
 *     dn_ij = dy_ij w_j s_ij
 *     dx_ij = r_i (dn_ij - n_ij c_i),  c_i = (1/D) sum_j dn_ij n_ij
 *     dw_j  = sum_i dy_ij n_ij s_ij
 *
 * dw is summed over rows in plain row order (row 0 first) in double
 * precision; the per-column sums are independent of each other, so the
 * columns are spread over threads without changing any column's order.
 * Rows are independent, so the per-row work is spread over threads too.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact value of a BF16 bit pattern: BF16 is the top half of an IEEE
 * binary32, so shifting the 16 bits up gives the same number as a float. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Logistic sigmoid, written so that exp() never overflows. */
static double sigmoid(double v)
{
    if (v >= 0.0)
        return 1.0 / (1.0 + exp(-v));
    double e = exp(v);
    return e / (1.0 + e);
}

/* r_i = 1 / sqrt(mean(x^2) + eps) for one row. */
static double row_rstd(const double *x, int64_t D, double eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < D; ++j)
        ss += x[j] * x[j];
    return 1.0 / sqrt(ss / (double)D + eps);
}

/* Forward of one row. */
static void fwd_row(const double *x, const double *g, const double *w,
                    int64_t D, double eps, double *y)
{
    double r = row_rstd(x, D, eps);
    for (int64_t j = 0; j < D; ++j) {
        double n = x[j] * r;
        double s = g[j] * sigmoid(g[j]);
        y[j] = n * w[j] * s;
    }
}

/* dx and dg of one row; returns r_i so the caller can form dw. */
static double bwd_row(const double *x, const double *g, const double *w,
                      const double *dy, int64_t D, double eps,
                      double *dx, double *dg)
{
    double r = row_rstd(x, D, eps);
    double c = 0.0;
    for (int64_t j = 0; j < D; ++j) {
        double sig = sigmoid(g[j]);
        double s = g[j] * sig;
        double dn = dy[j] * w[j] * s;
        c += dn * (x[j] * r);
    }
    c /= (double)D;
    for (int64_t j = 0; j < D; ++j) {
        double sig = sigmoid(g[j]);
        double s = g[j] * sig;
        double ds = sig * (1.0 + g[j] * (1.0 - sig)); /* d silu / d g */
        double n = x[j] * r;
        double dn = dy[j] * w[j] * s;
        dx[j] = r * (dn - n * c);
        dg[j] = dy[j] * w[j] * n * ds;
    }
    return r;
}

/* ---------------------------------------------------------------------- */
/* Double-precision inputs (used for finite differences and closed forms). */

void orc_fwd_f64(const double *x, const double *g, const double *w,
                 int64_t rows, int64_t D, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        fwd_row(x + i * D, g + i * D, w, D, eps, y + i * D);
}

void orc_bwd_f64(const double *x, const double *g, const double *w,
                 const double *dy, int64_t rows, int64_t D, double eps,
                 double *dx, double *dg, double *dw)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        r[i] = bwd_row(x + i * D, g + i * D, w, dy + i * D, D, eps,
                       dx + i * D, dg + i * D);
    /* dw_j = sum over rows, in row order, of dy * n * silu(g). */
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < rows; ++i) {
            double gij = g[i * D + j];
            double s = gij * sigmoid(gij);
            acc += dy[i * D + j] * (x[i * D + j] * r[i]) * s;
        }
        dw[j] = acc;
    }
    free(r);
}

/* ---------------------------------------------------------------------- */
/* BF16 inputs (bit patterns), exactly as the GPU receives them.  Each row is
 * decoded exactly into double and handed to the same row functions. */

static void decode_row(const uint16_t *src, int64_t D, double *dst)
{
    for (int64_t j = 0; j < D; ++j)
        dst[j] = bf16_bits_to_double(src[j]);
}

void orc_fwd_bf16(const uint16_t *x, const uint16_t *g, const uint16_t *w,
                  int64_t rows, int64_t D, double eps, double *y)
{
    double *wd = (double *)malloc(sizeof(double) * (size_t)D);
    decode_row(w, D, wd);
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)D);
        double *gr = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            decode_row(x + i * D, D, xr);
            decode_row(g + i * D, D, gr);
            fwd_row(xr, gr, wd, D, eps, y + i * D);
        }
        free(xr);
        free(gr);
    }
    free(wd);
}

/* dw may be NULL: then only dx and dg are produced (used when the oracle
 * checks a sample of rows of a large problem). */
void orc_bwd_bf16(const uint16_t *x, const uint16_t *g, const uint16_t *w,
                  const uint16_t *dy, int64_t rows, int64_t D, double eps,
                  double *dx, double *dg, double *dw)
{
    double *wd = (double *)malloc(sizeof(double) * (size_t)D);
    double *r = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    decode_row(w, D, wd);
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)D);
        double *gr = (double *)malloc(sizeof(double) * (size_t)D);
        double *dyr = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            decode_row(x + i * D, D, xr);
            decode_row(g + i * D, D, gr);
            decode_row(dy + i * D, D, dyr);
            r[i] = bwd_row(xr, gr, wd, dyr, D, eps, dx + i * D, dg + i * D);
        }
        free(xr);
        free(gr);
        free(dyr);
    }
    if (dw != NULL) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < D; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < rows; ++i) {
                double xij = bf16_bits_to_double(x[i * D + j]);
                double gij = bf16_bits_to_double(g[i * D + j]);
                double dyij = bf16_bits_to_double(dy[i * D + j]);
                double s = gij * sigmoid(gij);
                acc += dyij * (xij * r[i]) * s;
            }
            dw[j] = acc;
        }
    }
    free(r);
    free(wd);
}

/* ---------------------------------------------------------------------- */
/* Round a double to the nearest BF16 (ties to even), directly from double so
 * that there is no double rounding through binary32.  BF16 keeps 8
 * significant bits and binary32's exponent range: normal numbers have
 * exponents -126..127, below that the spacing is fixed at 2^-133. */
uint16_t orc_round_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    double q;
    if (a == 0.0) {
        q = 0.0;
    } else {
        int e;
        frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) */
        int ulp_exp = e - 8;        /* 8 significant bits */
        if (ulp_exp < -133)
            ulp_exp = -133;         /* subnormal spacing */
        q = ldexp(nearbyint(ldexp(a, -ulp_exp)), ulp_exp); /* ties-to-even */
    }
    uint16_t bits;
    if (q >= 0x1.0p128) {
        bits = 0x7F80;              /* overflow to infinity */
    } else {
        float f = (float)q;         /* exact: q has at most 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        bits = (uint16_t)(u >> 16);
    }
    return (uint16_t)(bits | (neg ? 0x8000u : 0u));
}

void orc_round_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t k = 0; k < n; ++k)
        out[k] = orc_round_bf16(v[k]);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
