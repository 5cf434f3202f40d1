/*
 * gemm_oracle.c -- the CPU oracle for the batched "mkl" GEMM with a fused
 * elementwise epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or helper with the GPU path.
 *
 * What it computes (written from the definition, deliberately slow and plain):
 *
 *   C[l][m][n] = epilogue( sum_{k=0}^{K-1} A[l][m][k] * B[l][n][k] )
 *
 *   - Operand modes (M,K,L) for A, (N,K,L) for B and (M,N,L) for C follow the
 *     tensor names mA_mkl / mB_nkl / mC_mnl of the persistent dense GEMM kernel
 *     signature on "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制", section 2.3.
 *     Storage is packed with the batch outermost and K contiguous:
 *     A is [L][M][K], B is [L][N][K], C is [L][M][N].
 *   - The sum is taken in IEEE binary64, in ascending k, starting from +0.0,
 *     with no fused multiply-add (build with -ffp-contract=off).  Every product
 *     of two fp32/fp16/bf16 values is exact in binary64.
 *   - The epilogue is applied once to the full-precision sum (the accumulator),
 *     never to a partial sum:
 *       identity: y = x
 *       ReLU:     y = (x > 0) ? x : 0   (the where(x > 0, x, 0) form of section
 *                 2.3 of the same page; also the compile-time do_relu epilogue
 *                 of section 7 of "CUTLASS CuTe DSL 控制流编程指南")
 *       SiLU:     y = x * sigmoid(x) = x / (1 + exp(-x))
 *   - The result is then rounded ONCE from binary64 to the output type
 *     (round to nearest, ties to even; overflow to +-inf; gradual underflow).
 *     Never binary64 -> binary32 -> bf16/fp16.
 *
 * Reading of the pages: section 2.3 of the JIT-argument page converts the
 * accumulator to the C type and then applies the epilogue; this oracle applies
 * the epilogue in binary64 and rounds once.  For identity and ReLU the two
 * orders give the same value; for SiLU they differ by at most an output ulp.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_IDENTITY = 0, OR_RELU = 1, OR_SILU = 2 };

/* ---------------- exact widening of stored inputs to binary64 ---------------- */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double widen_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0x1f)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1.f) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32 word. */
static double widen_bf16(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double widen(const void *base, int dtype, int64_t idx)
{
    switch (dtype) {
    case OR_F32: return (double)((const float *)base)[idx];
    case OR_F16: return widen_f16(((const uint16_t *)base)[idx]);
    default:     return widen_bf16(((const uint16_t *)base)[idx]);
    }
}

/* ---------------- the epilogue, in binary64 ---------------- */

double oracle_epilogue(double x, int epilogue)
{
    switch (epilogue) {
    case OR_RELU: return (x > 0.0) ? x : 0.0;
    case OR_SILU: return x / (1.0 + exp(-x));
    default:      return x;
    }
}

/* ---------------- single rounding binary64 -> narrow format ----------------
 *
 * A finite binary format with p significand bits (hidden bit included),
 * minimum normal exponent emin and maximum exponent emax.  The representable
 * numbers near |x| are multiples of the quantum 2^(max(e, emin) - p + 1),
 * where e = floor(log2 |x|).  Dividing by that power of two is exact in
 * binary64, rint() rounds to the nearest integer with ties to even (the
 * default rounding mode), and multiplying back is exact again.
 */
static double round_to_format(double x, int p, int emin, int emax)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);            /* ax = f * 2^e, f in [0.5, 1) */
    e -= 1;                   /* now ax in [2^e, 2^(e+1)) */
    if (e < emin)
        e = emin;
    int qexp = e - (p - 1);
    double q = rint(ldexp(ax, -qexp));
    double r = ldexp(q, qexp);
    /* largest finite: (2 - 2^(1-p)) * 2^emax; anything that rounds above it
     * overflows to infinity */
    double maxfin = ldexp(ldexp(1.0, p) - 1.0, emax - (p - 1));
    if (r > maxfin)
        r = INFINITY;
    return x < 0 ? -r : r;
}

static uint16_t encode_f16(double r)
{
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isnan(r)) return 0x7e00;
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    e -= 1;
    if (e < -14)              /* subnormal: a = f * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    int frac = (int)(ldexp(a, 10 - e) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)frac;
}

static uint16_t encode_bf16(double r)
{
    /* r is exactly representable in bfloat16, hence in binary32 */
    float f = (float)r;
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    if (isnan(r)) return 0x7fc0;
    return (uint16_t)(w >> 16);
}

/* Round n binary64 values once to dtype and store their bit patterns. */
void oracle_round(const double *in, void *out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = in[i];
        switch (dtype) {
        case OR_F32:
            ((float *)out)[i] = (float)round_to_format(x, 24, -126, 127);
            break;
        case OR_F16:
            ((uint16_t *)out)[i] = encode_f16(round_to_format(x, 11, -14, 15));
            break;
        default:
            ((uint16_t *)out)[i] = encode_bf16(round_to_format(x, 8, -126, 127));
            break;
        }
    }
}

/* Widen n stored values of dtype to binary64 (exact). */
void oracle_widen(const void *in, double *out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = widen(in, dtype, i);
}

/* ---------------- the GEMM ---------------- */

static double dot_row(const void *A, const void *B, int dtype,
                      int64_t a_off, int64_t b_off, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += widen(A, dtype, a_off + k) * widen(B, dtype, b_off + k);
    return acc;
}

/*
 * Full GEMM: C64 receives epilogue(sum) in binary64, shape [L][M][N].
 * nthreads <= 0 means the OpenMP default.  Returns the thread count used.
 */
int oracle_gemm(const void *A, const void *B, double *C64,
                int64_t M, int64_t N, int64_t K, int64_t L,
                int dtype, int epilogue, int nthreads)
{
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    used = omp_get_max_threads();
#endif
    int64_t rows = L * M;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t l = r / M, m = r % M;
        for (int64_t n = 0; n < N; ++n) {
            double acc = dot_row(A, B, dtype, (l * M + m) * K, (l * N + n) * K, K);
            C64[(l * M + m) * N + n] = oracle_epilogue(acc, epilogue);
        }
    }
    return used;
}

/*
 * Grouped GEMM (the variable-M grouped matrix product named on
 * "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制", section 5; the layout is
 * the plainest reading): group g owns rows [offs[g - 1], offs[g]) of A
 * ([total_m][K]) and of C64 ([total_m][N]), with offs[-1] = 0, and its own
 * B[g] ([G][N][K]).  For every row r of group g and every n:
 *
 *   C64[r][n] = epilogue( sum_k A[r][k] * B[g][n][k] )
 *
 * with the same binary64 sum as oracle_gemm.  Rows in no group are not
 * written.  The offsets must be non-decreasing in [0, total_m]; otherwise
 * nothing is written and -1 is returned.
 */
int oracle_gemm_grouped(const void *A, const void *B, double *C64, const int32_t *offs,
                        int64_t G, int64_t total_m, int64_t N, int64_t K,
                        int dtype, int epilogue, int nthreads)
{
    int64_t prev = 0;
    for (int64_t g = 0; g < G; ++g) {
        if (offs[g] < prev || offs[g] > total_m)
            return -1;
        prev = offs[g];
    }
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    used = omp_get_max_threads();
#endif
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < total_m; ++r) {
        /* the group of row r: the first g whose end lies past r */
        int64_t g = 0;
        while (g < G && offs[g] <= r)
            ++g;
        if (g == G)
            continue;
        for (int64_t n = 0; n < N; ++n) {
            double acc = dot_row(A, B, dtype, r * K, (g * N + n) * K, K);
            C64[r * N + n] = oracle_epilogue(acc, epilogue);
        }
    }
    return used;
}

/*
 * RMSNorm over the last axis (the worked example of "一个可定制的编译器，用于为
 * AI模型生成高效的融合GPU内核": torch.nn.RMSNorm over rows of hidden size H,
 * whose loop nest squares and sums a row, scales the sum by 1/H, adds eps,
 * takes the reciprocal square root, and multiplies each element by it and by
 * the weight).  For every row r and column j of x ([rows][H]):
 *
 *   ms  = (sum_{j'} x[r][j']^2) / H
 *   y64[r][j] = (x[r][j] * (1 / sqrt(ms + eps))) * w[j]
 *
 * all in binary64 (squares summed in ascending j from +0.0), left unrounded:
 * oracle_round rounds the result once to the output type.  eps is taken as
 * given (the caller passes the value the GPU adds).
 */
int oracle_rms_norm(const void *x, const void *w, double *y64, int64_t rows, int64_t H,
                    double eps, int dtype, int nthreads)
{
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    used = omp_get_max_threads();
#endif
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = widen(x, dtype, r * H + j);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t j = 0; j < H; ++j)
            y64[r * H + j] = (widen(x, dtype, r * H + j) * inv) * widen(w, dtype, j);
    }
    return used;
}

/*
 * Selected entries only: for i < count, out64[i] = C64[l[i]][m[i]][n[i]] of the
 * full GEMM above.  Used to check very large problems on sampled outputs.
 */
int oracle_gemm_entries(const void *A, const void *B,
                        int64_t M, int64_t N, int64_t K, int64_t L,
                        int dtype, int epilogue,
                        const int64_t *li, const int64_t *mi, const int64_t *ni,
                        int64_t count, double *out64, int nthreads)
{
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    used = omp_get_max_threads();
#endif
    (void)L;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double acc = dot_row(A, B, dtype, (li[i] * M + mi[i]) * K,
                             (li[i] * N + ni[i]) * K, K);
        out64[i] = oracle_epilogue(acc, epilogue);
    }
    return used;
}

/* Number of OpenMP threads the oracle's parallel loops use (1 without OpenMP). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
