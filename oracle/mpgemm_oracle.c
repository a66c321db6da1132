/*
 * mpgemm_oracle.c -- plain CPU reference for D = alpha * op(A) * op(B) + beta * C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or calls this
 * file, and this file includes nothing from the GPU library.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it.
 *
 * What it computes, and where each step comes from:
 *
 *   - The operation is the GEMM statement of "Programming Tensor Cores in CUDA 9"
 *     (makelele.cn/d/1827294.html): sections "Tensor Cores in CUDA libraries / how to use
 *     Tensor Cores in cuBLAS" (the cublasGemmEx call: transa, transb, m, n, k, alpha, lda,
 *     ldb, beta, ldc, input and compute types) and "Finishing" (the result is scaled by
 *     alpha and the existing C, scaled by beta, is added).
 *   - Products of FP16 inputs are formed at full precision and summed at FP32 or wider
 *     (same page, section "What are Tensor Cores?", Figure 2).  The oracle forms every
 *     product exactly in double and sums in double.
 *   - INT8 inputs are multiplied and summed into a 32-bit integer, the DP4A dot product of
 *     "Mixed-Precision Programming with CUDA 8" (m.ruidan.com/infomation/detail/138780),
 *     section "High-performance low-precision integers" and Figure 2.  The oracle sums in
 *     64-bit integers and reduces modulo 2^32 at the end.
 *   - Floating-point formats are decoded from their IEEE-754 field definitions (FP16 =
 *     1 sign, 5 exponent, 10 fraction bits; FP32 = 1/8/23; the CUDA 8 page, section "Floating
 *     point precision", Figure 1).  BF16 is the upper half of an FP32 pattern (1/8/7).
 *   - The output is rounded once, to nearest with ties to even, as the final step of the
 *     Tensor Core rounding model ("NVIDIA Tensor Core mixed-precision computing: principles
 *     and applications", jsqmd.com/news/1087138, section 2.3).
 *
 * Exactness: an FP16 x FP16 product has at most 22 significant bits and a BF16 x BF16
 * product at most 16, so every product is exact in double.  The double sum of k terms
 * differs from the exact sum by at most (k-1) * 2^-53 * sum|a*b|; integer-valued (or
 * common-dyadic-scale) inputs whose absolute sums stay below 2^53 are summed exactly.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no -ffast-math: it would
 * flush subnormals and reassociate).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* Element type codes, private to the oracle (the Python wrapper maps names to them). */
enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_F32 = 3, ORC_I32 = 4 };

/* Field widths (exponent bits, fraction bits) of the floating formats. */
static int ebits_of(int t) { return t == ORC_F16 ? 5 : 8; }
static int mbits_of(int t) { return t == ORC_F16 ? 10 : (t == ORC_BF16 ? 7 : 23); }

/*
 * Decode a binary floating-point pattern from its field definition:
 *   exponent field all ones    -> infinity (fraction 0) or NaN,
 *   exponent field 0           -> (-1)^s * 2^(1-bias) * f / 2^mbits   (zero / subnormal),
 *   otherwise                  -> (-1)^s * 2^(e-bias) * (1 + f / 2^mbits).
 */
double oracle_decode(uint64_t bits, int ebits, int mbits)
{
    const uint64_t fmask = (1ull << mbits) - 1;
    const uint64_t emask = (1ull << ebits) - 1;
    const int bias = (1 << (ebits - 1)) - 1;
    const uint64_t f = bits & fmask;
    const uint64_t e = (bits >> mbits) & emask;
    const int s = (int)((bits >> (mbits + ebits)) & 1);
    double mag;
    if (e == emask)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, 1 - bias - mbits);
    else
        mag = ldexp((double)(f | (1ull << mbits)), (int)e - bias - mbits);
    return s ? -mag : mag;
}

/*
 * Round a double to the binary format (ebits, mbits), to nearest, ties to even, and return
 * the bit pattern.  Finite values at or beyond the rounding threshold of the largest finite
 * value become infinity; values below half the smallest subnormal become signed zero.
 * Any NaN becomes the canonical quiet NaN with the input's sign.
 */
uint64_t oracle_encode_rne(double v, int ebits, int mbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const uint64_t emax_field = (1ull << ebits) - 1;
    const uint64_t sbit = (uint64_t)(signbit(v) ? 1 : 0) << (ebits + mbits);
    if (isnan(v))
        return sbit | (emax_field << mbits) | (1ull << (mbits - 1));
    const double a = fabs(v);
    if (isinf(a))
        return sbit | (emax_field << mbits);
    if (a == 0.0)
        return sbit;

    /* Binade of a: a lies in [2^x, 2^(x+1)); below the normal range the spacing stays at
     * the subnormal quantum 2^(emin - mbits). */
    int e2;
    (void)frexp(a, &e2);
    int x = e2 - 1;
    if (x < emin)
        x = emin;
    const double quantum = ldexp(1.0, x - mbits);
    const double n = a / quantum;           /* exact: division by a power of two */
    const double whole = floor(n);
    const double frac = n - whole;          /* exact */
    uint64_t r = (uint64_t)whole;
    if (frac > 0.5 || (frac == 0.5 && (r & 1)))
        r += 1;                             /* round half to even */
    if (r == (2ull << mbits)) {             /* rounded up into the next binade */
        r >>= 1;
        x += 1;
    }
    if (r < (1ull << mbits))                /* subnormal (x == emin here) */
        return sbit | r;
    if (x > bias)                           /* overflow */
        return sbit | (emax_field << mbits);
    return sbit | ((uint64_t)(x + bias) << mbits) | (r - (1ull << mbits));
}

/* Exact widening of every pattern of a 16-bit input format, built from oracle_decode. */
static void fill_table16(double *tab, int t)
{
    for (uint32_t b = 0; b < 65536u; ++b)
        tab[b] = oracle_decode(b, ebits_of(t), mbits_of(t));
}

/* C element (FP32 or FP16/BF16) widened to double. */
static double c_elem(const void *C, int ctype, int64_t idx)
{
    if (ctype == ORC_F32)
        return oracle_decode(((const uint32_t *)C)[idx], 8, 23);
    return oracle_decode(((const uint16_t *)C)[idx], ebits_of(ctype), mbits_of(ctype));
}

/* Storage index of op(A)(i, p) and op(B)(p, j) in row-major buffers (transpose flag 1 means
 * the buffer holds the transpose of the operand). */
static int64_t a_index(int transa, int64_t lda, int64_t i, int64_t p)
{
    return transa ? p * lda + i : i * lda + p;
}
static int64_t b_index(int transb, int64_t ldb, int64_t p, int64_t j)
{
    return transb ? j * ldb + p : p * ldb + j;
}

/*
 * One output element of the floating-point GEMM:
 *   s = sum_p a(i,p) * b(p,j)          (double; every product exact)
 *   S = sum_p |a(i,p) * b(p,j)|        (double; feeds the error bound)
 *   v = alpha * s            if beta == 0 (C is not read),
 *   v = alpha * s + beta * c otherwise.
 */
static void fp_point(const double *tab_a, const double *tab_b, int transa, int transb,
                     int64_t k, double alpha, const uint16_t *A, int64_t lda,
                     const uint16_t *B, int64_t ldb, double beta, const void *C, int ctype,
                     int64_t ldc, int64_t i, int64_t j, double *v, double *S, double *bc)
{
    double s = 0.0, sa = 0.0;
    for (int64_t p = 0; p < k; ++p) {
        const double prod = tab_a[A[a_index(transa, lda, i, p)]] *
                            tab_b[B[b_index(transb, ldb, p, j)]];
        s += prod;
        sa += fabs(prod);
    }
    double betac = 0.0;
    double out;
    if (beta == 0.0) {
        out = alpha * s;
    } else {
        betac = beta * c_elem(C, ctype, i * ldc + j);
        out = alpha * s + betac;
    }
    *v = out;
    *S = sa;
    *bc = betac;
}

/*
 * Floating-point GEMM at a list of output points (ii[t], jj[t]).
 * atype, btype: ORC_F16 or ORC_BF16 (same for both).  ctype: ORC_F32, ORC_F16 or ORC_BF16
 * (only read when beta != 0).  Outputs, per point: v (reference value before output
 * rounding), S (sum of |products|), bc (beta * c, 0 when beta == 0).
 * Returns 0, or -1 on an unsupported type.
 */
int oracle_gemm_fp_points(int transa, int transb, int64_t m, int64_t n, int64_t k,
                          double alpha, const void *A, int atype, int64_t lda,
                          const void *B, int btype, int64_t ldb, double beta,
                          const void *C, int ctype, int64_t ldc, int64_t npts,
                          const int64_t *ii, const int64_t *jj, double *v, double *S,
                          double *bc)
{
    (void)m; (void)n;
    if ((atype != ORC_F16 && atype != ORC_BF16) || (btype != ORC_F16 && btype != ORC_BF16))
        return -1;
    if (ctype != ORC_F32 && ctype != ORC_F16 && ctype != ORC_BF16)
        return -1;
    double *tab_a = malloc(65536 * sizeof(double));
    double *tab_b = malloc(65536 * sizeof(double));
    if (!tab_a || !tab_b) {
        free(tab_a);
        free(tab_b);
        return -2;
    }
    fill_table16(tab_a, atype);
    fill_table16(tab_b, btype);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < npts; ++t)
        fp_point(tab_a, tab_b, transa, transb, k, alpha, (const uint16_t *)A, lda,
                 (const uint16_t *)B, ldb, beta, C, ctype, ldc, ii[t], jj[t], &v[t], &S[t],
                 &bc[t]);
    free(tab_a);
    free(tab_b);
    return 0;
}

/* Floating-point GEMM over the whole m x n output (row-major v, S, bc with stride n). */
int oracle_gemm_fp_full(int transa, int transb, int64_t m, int64_t n, int64_t k,
                        double alpha, const void *A, int atype, int64_t lda, const void *B,
                        int btype, int64_t ldb, double beta, const void *C, int ctype,
                        int64_t ldc, double *v, double *S, double *bc)
{
    if ((atype != ORC_F16 && atype != ORC_BF16) || (btype != ORC_F16 && btype != ORC_BF16))
        return -1;
    if (ctype != ORC_F32 && ctype != ORC_F16 && ctype != ORC_BF16)
        return -1;
    double *tab_a = malloc(65536 * sizeof(double));
    double *tab_b = malloc(65536 * sizeof(double));
    if (!tab_a || !tab_b) {
        free(tab_a);
        free(tab_b);
        return -2;
    }
    fill_table16(tab_a, atype);
    fill_table16(tab_b, btype);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            fp_point(tab_a, tab_b, transa, transb, k, alpha, (const uint16_t *)A, lda,
                     (const uint16_t *)B, ldb, beta, C, ctype, ldc, i, j, &v[i * n + j],
                     &S[i * n + j], &bc[i * n + j]);
    free(tab_a);
    free(tab_b);
    return 0;
}

/*
 * One output element of the integer GEMM: s = sum_p a(i,p) * b(p,j) with a, b signed bytes,
 * then alpha * s (+ beta * c when beta != 0), all modulo 2^64 (unsigned arithmetic, so
 * wrap-around is defined); the caller reduces modulo 2^32 for the INT32 output.  Since 2^32
 * divides 2^64, the result modulo 2^32 equals the one of an INT32 accumulator that wraps.
 */
static uint64_t int_point(int transa, int transb, int64_t k, int64_t alpha,
                          const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                          int64_t beta, const int32_t *C, int64_t ldc, int64_t i, int64_t j)
{
    int64_t s = 0;
    for (int64_t p = 0; p < k; ++p)
        s += (int64_t)A[a_index(transa, lda, i, p)] * (int64_t)B[b_index(transb, ldb, p, j)];
    uint64_t out = (uint64_t)alpha * (uint64_t)s;
    if (beta != 0)
        out += (uint64_t)beta * (uint64_t)(int64_t)C[i * ldc + j];
    return out;
}

int oracle_gemm_int_points(int transa, int transb, int64_t m, int64_t n, int64_t k,
                           int64_t alpha, const int8_t *A, int64_t lda, const int8_t *B,
                           int64_t ldb, int64_t beta, const int32_t *C, int64_t ldc,
                           int64_t npts, const int64_t *ii, const int64_t *jj, int32_t *d)
{
    (void)m; (void)n;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < npts; ++t)
        d[t] = (int32_t)(uint32_t)int_point(transa, transb, k, alpha, A, lda, B, ldb, beta, C,
                                            ldc, ii[t], jj[t]);
    return 0;
}

int oracle_gemm_int_full(int transa, int transb, int64_t m, int64_t n, int64_t k,
                         int64_t alpha, const int8_t *A, int64_t lda, const int8_t *B,
                         int64_t ldb, int64_t beta, const int32_t *C, int64_t ldc, int32_t *d)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            d[i * n + j] = (int32_t)(uint32_t)int_point(transa, transb, k, alpha, A, lda, B,
                                                        ldb, beta, C, ldc, i, j);
    return 0;
}

/* Round an array of doubles to the output format (ORC_F32, ORC_F16 or ORC_BF16). */
int oracle_round_array(const double *v, int64_t count, int otype, void *out)
{
    if (otype == ORC_F32) {
        for (int64_t t = 0; t < count; ++t)
            ((uint32_t *)out)[t] = (uint32_t)oracle_encode_rne(v[t], 8, 23);
        return 0;
    }
    if (otype == ORC_F16 || otype == ORC_BF16) {
        for (int64_t t = 0; t < count; ++t)
            ((uint16_t *)out)[t] =
                (uint16_t)oracle_encode_rne(v[t], ebits_of(otype), mbits_of(otype));
        return 0;
    }
    return -1;
}

/* Threads the OpenMP loops above run on. */
int oracle_num_threads(void) { return omp_get_max_threads(); }
