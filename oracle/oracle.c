/*
 * CPU oracle for the row-wise reduce-then-rescale operations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the GPU library; it is deliberately plain and slow:
 *   - every quantity is computed in double precision (fp64),
 *   - each row is computed by the textbook definition, in the order the
 *     definition states it (no blocking, no fusion, no reordering),
 *   - libm's exp() and sqrt(); the file is built without -ffast-math,
 *   - rows are independent, so an OpenMP "parallel for" hands whole rows to
 *     host threads; a row's arithmetic is the same whatever thread runs it.
 *
 * Inputs arrive as doubles.  Every input element is an exact fp32 or bf16
 * value widened to double, which is exact, so the oracle sees exactly the
 * numbers the GPU sees.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "两个融合算子：RMSNorm 与 online softmax" (daleiyang.github.io,
 *        llm-inference-anatomy report 04)
 *   [P2] "GPU Kernel 工程（04）：共享内存与 reduction——softmax、LayerNorm 与
 *        online softmax" (arganzheng.life)
 *   [P3] "第23讲：为什么Attention必须先算Max？" (lilinji.mintlify.site)
 *   [P4] "Softmax 与归一化", CUDA 进阶手册 (anrans.github.io ai-infra-handbooks)
 *   [P5] "RMSNorm、Softmax 与在线归约" (notes.kuangjux.top)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Number of host threads the row loops use (1 when built without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Round a double to the nearest bfloat16 value, ties to even, returned as a
 * double.  bfloat16 is IEEE-style binary with 1 sign bit, 8 exponent bits
 * (bias 127, the same range as fp32) and 8 significant bits (7 stored).
 * [P2] section 十 prints bf16 output with the round-to-nearest conversion;
 * every fp->bf16 conversion in this oracle uses this one routine.
 *
 * Definition used: for |v| in [2^e, 2^(e+1)) with e >= -126 the spacing of
 * bf16 numbers is 2^(e-7); below 2^-126 (subnormals) it is 2^-133.  v is
 * divided by the spacing (exact: a power of two), rounded to an integer
 * with ties to even (rint in the default rounding mode), and scaled back.
 * A result of 2^128 or more is outside the format and becomes infinity.
 */
double oracle_round_bf16(double v) {
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    int k;
    frexp(v, &k);              /* |v| in [2^(k-1), 2^k) */
    int e = k - 1;
    if (e < -126) e = -126;    /* subnormal range shares the smallest spacing */
    double spacing = ldexp(1.0, e - 7);
    double q = rint(v / spacing);
    double r = q * spacing;
    if (fabs(r) >= ldexp(1.0, 128)) return copysign(INFINITY, v);
    return r;
}

/* Round a double to the nearest fp32 value, ties to even (C's conversion). */
double oracle_round_f32(double v) { return (double)(float)v; }

static double round_io(double v, int io_dtype) {
    return io_dtype == ORACLE_BF16 ? oracle_round_bf16(v) : oracle_round_f32(v);
}

/* Round n values to the I/O dtype (used by tests to build the expected
 * stored outputs from the fp64 results). */
void oracle_round_array(int io_dtype, int64_t n, const double* in, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_io(in[i], io_dtype);
}

/*
 * RMSNorm of one row, plain definition:
 *   ss = sum_j x_j^2,   r = 1 / sqrt(ss / H + eps),   y_j = x_j * r * gamma_j
 * eps is added to the mean square inside the square root, the mean divides
 * by H, and nothing is subtracted from x.
 * [P5] section "RMSNorm 归约什么" (the displayed formula for r and y_j);
 * [P2] section 二.1 and 八.1 (eps inside the root); [P4] section
 * "LayerNorm 与 RMSNorm" (the RMSNorm formula).
 */
static void rmsnorm_row(int64_t H, const double* x, const double* gamma, double eps,
                        double* y) {
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) ss += x[j] * x[j];
    double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t j = 0; j < H; ++j) y[j] = x[j] * r * gamma[j];
}

/* RMSNorm over M rows of width H (row-major, row stride H). Returns 0, or
 * -1 when H < 1 (an empty row has no mean square). */
int oracle_rmsnorm(int64_t M, int64_t H, const double* x, const double* gamma, double eps,
                   double* y) {
    if (H < 1 || M < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) rmsnorm_row(H, x + i * H, gamma, eps, y + i * H);
    return 0;
}

/*
 * Fused residual add + RMSNorm over M rows of width H.
 *   h_j = round_io(x_j + res_j)     -- the new residual, as stored
 *   y   = RMSNorm(h) with gamma     -- computed from the stored h
 * [P4] section "算子融合：fused_add_rms_norm" (residual = residual + hidden,
 * then hidden = rms_norm(residual) * w, both written back);
 * [P2] section 八.3 (read x and residual once, write the updated residual
 * and the normalised output).
 * The pages leave open whether y is computed from the unrounded sum or from
 * the residual as stored in the I/O dtype; this oracle takes the stored
 * residual, so the fused result equals running the add and then RMSNorm.
 * The sum x_j + res_j of two fp32 or bf16 numbers is exact in fp64, so h is
 * the correctly rounded sum.  res_out receives h (as a double holding an
 * I/O-dtype value); y receives the unrounded fp64 result.
 */
int oracle_fused_add_rmsnorm(int64_t M, int64_t H, const double* x, const double* res,
                             const double* gamma, double eps, int io_dtype,
                             double* res_out, double* y) {
    if (H < 1 || M < 0) return -1;
    if (io_dtype != ORACLE_F32 && io_dtype != ORACLE_BF16) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double* xr = x + i * H;
        const double* rr = res + i * H;
        double* hr = res_out + i * H;
        for (int64_t j = 0; j < H; ++j) hr[j] = round_io(xr[j] + rr[j], io_dtype);
        rmsnorm_row(H, hr, gamma, eps, y + i * H);
    }
    return 0;
}

/*
 * LayerNorm of one row, plain two-pass definition:
 *   mu = (1/H) sum_j x_j,   var = (1/H) sum_j (x_j - mu)^2,
 *   y_j = (x_j - mu) / sqrt(var + eps) * gamma_j + beta_j
 * [P2] section 八.2 (the LayerNorm formula, the variance over d, eps inside
 * the root); [P4] section "LayerNorm 与 RMSNorm" (the same formula) and its
 * exercise (mean first, then the variance from the centred values).  beta may
 * be NULL, meaning zero.
 */
static void layernorm_row(int64_t H, const double* x, const double* gamma, const double* beta,
                          double eps, double* y) {
    double sum = 0.0;
    for (int64_t j = 0; j < H; ++j) sum += x[j];
    double mu = sum / (double)H;
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) ss += (x[j] - mu) * (x[j] - mu);
    double var = ss / (double)H;
    double r = 1.0 / sqrt(var + eps);
    for (int64_t j = 0; j < H; ++j) y[j] = (x[j] - mu) * r * gamma[j] + (beta ? beta[j] : 0.0);
}

/* LayerNorm over M rows of width H. Returns 0, or -1 when H < 1. */
int oracle_layernorm(int64_t M, int64_t H, const double* x, const double* gamma,
                     const double* beta, double eps, double* y) {
    if (H < 1 || M < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) layernorm_row(H, x + i * H, gamma, beta, eps, y + i * H);
    return 0;
}

/*
 * Safe softmax of one row, three passes over the row:
 *   m = max_j x_j,   d = sum_j exp(x_j - m),   y_j = exp(x_j - m) / d
 * [P1] section "一、为什么要减 max" (subtract the row maximum; the shift
 * leaves the result unchanged); [P3] section 2.2 ④ (Formal Model) and
 * section 2.3 (the three scans); [P5] section "稳定 Softmax".
 * Masked entries hold -inf and contribute exp(-inf) = 0.  A row whose
 * entries are all -inf has m = -inf and x_j - m = -inf - (-inf) = NaN, so
 * every output is NaN, as IEEE arithmetic gives (the pages' reading of a
 * fully masked row).
 */
static void softmax_row(int64_t N, const double* x, double* y) {
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j)
        if (x[j] > m) m = x[j];
    double d = 0.0;
    for (int64_t j = 0; j < N; ++j) d += exp(x[j] - m);
    for (int64_t j = 0; j < N; ++j) y[j] = exp(x[j] - m) / d;
}

/* Softmax over M rows of width N. Returns 0, or -1 when N < 1. */
int oracle_softmax(int64_t M, int64_t N, const double* x, double* y) {
    if (N < 1 || M < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) softmax_row(N, x + i * N, y + i * N);
    return 0;
}

/*
 * Log-softmax of one row: y_j = log(exp(x_j - m) / d) = (x_j - m) - log(d),
 * with m and d of the safe softmax above (the log of the definition; PyTorch's
 * log-softmax switch is the form the pages cite: [P2] section 九, the
 * dispatch of SoftMax.cu).  Masked entries (-inf) give -inf; a fully masked
 * row gives NaN.
 */
static void log_softmax_row(int64_t N, const double* x, double* y) {
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j)
        if (x[j] > m) m = x[j];
    double d = 0.0;
    for (int64_t j = 0; j < N; ++j) d += exp(x[j] - m);
    double ld = log(d);
    for (int64_t j = 0; j < N; ++j) y[j] = (x[j] - m) - ld;
}

/* Log-softmax over M rows of width N. Returns 0, or -1 when N < 1. */
int oracle_log_softmax(int64_t M, int64_t N, const double* x, double* y) {
    if (N < 1 || M < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) log_softmax_row(N, x + i * N, y + i * N);
    return 0;
}

/*
 * Row statistics (m, d) of the safe softmax for each row, from the same
 * three-pass definition: m = max_j x_j, d = sum_j exp(x_j - m).
 * Tests use it to check the normaliser invariants (d >= 1 for a row with a
 * finite maximum, [P1] section "四、数值上到底安不安全").
 */
int oracle_softmax_stats(int64_t M, int64_t N, const double* x, double* m_out,
                         double* d_out) {
    if (N < 1 || M < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double* xr = x + i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j)
            if (xr[j] > m) m = xr[j];
        double d = 0.0;
        for (int64_t j = 0; j < N; ++j) d += exp(xr[j] - m);
        m_out[i] = m;
        d_out[i] = d;
    }
    return 0;
}
