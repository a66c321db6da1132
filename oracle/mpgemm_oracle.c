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
#include <limits.h>
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

/* Threads the OpenMP loops above run on, and a way to set them (n >= 1) for timing runs. */
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { if (n >= 1) omp_set_num_threads(n); }

/* ======================================================================================
 * Block-FMA model of matrix-core FP16/BF16 accumulation (bit-exact reference).
 *
 * "NVIDIA Tensor Core mixed-precision computing: principles and applications"
 * (jsqmd.com/news/1087138) models a matrix core's product-sum as a chain of block FMAs
 * (sections 2.2.1, 2.2.2, 2.3 and 4.2.1): the N_FMA products of a block are formed exactly,
 * aligned to the block's largest exponent in an accumulator with a fixed number of fraction
 * bits, the bits below it are dropped (truncation), and the running FP32 value is updated
 * once per block, rounding to nearest-even.  The page gives the parameters of NVIDIA parts
 * (for A100 FP16/BF16: 8 products per block and a 2+23+1-bit accumulator) and measures them
 * with the test-vector method of its section 3.1.  This function is that model with the
 * block size and the fraction width as arguments:
 *
 *   blocks       products of k = 0..nblk-1, then nblk..2 nblk-1, ... (a last, shorter block
 *                holds the remainder);
 *   alignment    emax = max over the block's products with both operands nonzero of
 *                E(a) + E(b), E(x) = the unbiased exponent of x's field, the format's
 *                minimum normal exponent for subnormals; zero operands take no part;
 *   window       every term is cut at 2^(emax - frac): products toward zero, the running
 *                FP32 value toward minus infinity;
 *   sum width    the exact sum of the cut terms keeps sum_bits bits, counted down from the
 *                leading bit of its magnitude (from 2^-126 when it lies below FP32's normal
 *                range), and is cut toward minus infinity below them (sum_bits = 0: no limit);
 *   update       running value = RNE_fp32(that sum), subnormal results kept, overflow to
 *                infinity; a block whose products are all zero leaves it as is;
 *   specials     a product whose exact magnitude reaches 2^128 is infinite; NaN operands,
 *                Inf x 0 and opposite infinities give NaN, other infinities propagate.
 *
 * The page leaves open the cut directions, the exponent a subnormal or zero operand stands
 * for, and overflow; the choices above are those that GNFT-style feature-detection vectors
 * find on gfx950's v_mfma_f32_16x16x32_{f16,bf16} (kept as GPU tests in
 * tests/test_gpu_numerics.py and tests/test_gpu_bitexact.py), and so is the sum width, which
 * the page does not model.  With nblk = 8, frac = 24 (the 2+23+1
 * accumulator) and sum_bits = 32 the model reproduces that instruction; other values give
 * the page's other models (V100: nblk = 4, frac = 22).
 *
 * Epilogue (the pages fix only D = alpha * AB + beta * C): FP32 arithmetic,
 * v = alpha * acc when beta == 0, else v = fma(alpha, acc, beta * c); then one RNE to the
 * output format.
 *
 * Exactness: every term is an integer multiple of 2^(emax - frac) held in a 128-bit
 * integer (sum_bits cuts it to a coarser multiple); products are below 2^(frac + 2) such units and the running value is shifted by
 * at most 64 bits (beyond that it is returned unchanged, see mfma_block).
 * ====================================================================================== */

typedef __int128 i128;

/* A decoded input: x = sign * mant * 2^(expo - mbits); kind 0 finite, 1 Inf, 2 NaN. */
typedef struct { uint32_t mant; int16_t expo; uint8_t neg, kind; } fp_parts;

static fp_parts parts16(uint16_t bits, int t)
{
    const int eb = ebits_of(t), mb = mbits_of(t);
    const int bias = (1 << (eb - 1)) - 1;
    const uint32_t f = bits & ((1u << mb) - 1);
    const uint32_t e = (bits >> mb) & ((1u << eb) - 1);
    fp_parts p = { 0, 0, (uint8_t)((bits >> (eb + mb)) & 1), 0 };
    if (e == (1u << eb) - 1) {
        p.kind = f ? 2 : 1;
    } else if (e == 0) {
        p.expo = (int16_t)(1 - bias);   /* subnormal (or zero): the minimum normal exponent */
        p.mant = f;
    } else {
        p.expo = (int16_t)((int)e - bias);
        p.mant = f | (1u << mb);
    }
    return p;
}

/* Number of significant bits of u (0 for u == 0). */
static int bitlen128(unsigned __int128 u)
{
    const uint64_t hi = (uint64_t)(u >> 64), lo = (uint64_t)u;
    if (hi)
        return 128 - __builtin_clzll(hi);
    return lo ? 64 - __builtin_clzll(lo) : 0;
}

/* S * 2^g rounded to FP32: nearest-even, subnormals kept, overflow to infinity. */
static float fp32_from_scaled(i128 S, int g)
{
    if (S == 0)
        return 0.0f;
    const int neg = S < 0;
    unsigned __int128 u = neg ? -(unsigned __int128)S : (unsigned __int128)S;
    const int e = g + bitlen128(u) - 1;           /* exponent of the leading bit */
    int q = e < -126 ? -149 : e - 23;              /* FP32 spacing at this magnitude */
    const int sh = q - g;
    if (sh > 0) {
        const unsigned __int128 rem = u & (((unsigned __int128)1 << sh) - 1);
        const unsigned __int128 half = (unsigned __int128)1 << (sh - 1);
        u >>= sh;
        if (rem > half || (rem == half && (u & 1)))
            u += 1;
    } else {
        q = g;
    }
    double mag = ldexp((double)(uint64_t)u, q);    /* u <= 2^24: exact */
    if (mag >= 0x1p128)
        mag = INFINITY;
    return (float)(neg ? -mag : mag);
}

/* x * 2^(*g) rounded to `bits` significant bits, ties to even; *g moves to the new grid. */
static i128 round_to_bits(i128 x, int *g, int bits)
{
    const unsigned __int128 u = x < 0 ? -(unsigned __int128)x : (unsigned __int128)x;
    const int sh = bitlen128(u) - bits;
    if (sh <= 0)
        return x;
    unsigned __int128 q = u >> sh;
    const unsigned __int128 r = u - (q << sh), half = (unsigned __int128)1 << (sh - 1);
    if (r > half || (r == half && (q & 1)))
        q += 1;
    *g += sh;
    return x < 0 ? -(i128)q : (i128)q;
}

/* x cut at 2^s (s > 0 bits dropped from an integer): toward zero / toward minus infinity. */
static i128 cut_toward_zero(i128 x, int s)
{
    if (s >= 120)
        return 0;
    return x >= 0 ? (x >> s) : -((-x) >> s);
}
static i128 cut_floor(i128 x, int s)
{
    if (s >= 120)
        return x >= 0 ? 0 : -1;
    return x >= 0 ? (x >> s) : -(((-x) + (((i128)1 << s) - 1)) >> s);
}

/* One block update of the running FP32 value acc with the products a[t] * b[t], t < cnt. */
static float mfma_block(float acc, const fp_parts *a, const fp_parts *b, int cnt, int mb,
                        int frac, int sum_bits)
{
    /* special values first: NaN, infinite operands, products overflowing FP32 */
    int nan = isnan(acc), pinf = isinf(acc) && acc > 0, ninf = isinf(acc) && acc < 0;
    int have = 0, emax = 0;
    for (int t = 0; t < cnt; ++t) {
        const int neg = a[t].neg ^ b[t].neg;
        if (a[t].kind == 2 || b[t].kind == 2) {
            nan = 1;
        } else if (a[t].kind == 1 || b[t].kind == 1) {
            const int other_zero = (a[t].kind == 1 ? (b[t].kind == 0 && b[t].mant == 0)
                                                   : (a[t].mant == 0));
            if (other_zero)
                nan = 1;
            else if (neg)
                ninf = 1;
            else
                pinf = 1;
        } else if (a[t].mant && b[t].mant) {
            const uint64_t pm = (uint64_t)a[t].mant * b[t].mant;
            const int e = a[t].expo + b[t].expo;
            if (bitlen128(pm) - 1 + e - 2 * mb >= 128) {
                if (neg)
                    ninf = 1;
                else
                    pinf = 1;
            }
            if (!have || e > emax)
                emax = e;
            have = 1;
        }
    }
    if (nan || (pinf && ninf))
        return NAN;
    if (pinf)
        return INFINITY;
    if (ninf)
        return -INFINITY;
    if (!have)
        return acc;

    const int g = emax - frac;                     /* the window's last bit is 2^g */
    i128 S = 0;
    for (int t = 0; t < cnt; ++t) {
        if (!a[t].mant || !b[t].mant)
            continue;
        const i128 pm = (i128)((uint64_t)a[t].mant * b[t].mant);
        const int sh = a[t].expo + b[t].expo - 2 * mb - g;   /* product = pm * 2^(sh + g) */
        const i128 term = sh >= 0 ? (pm << sh) : cut_toward_zero(pm, -sh);
        S += (a[t].neg ^ b[t].neg) ? -term : term;
    }
    if (acc != 0.0f) {
        /* acc = +-M * 2^(E - 23) from its FP32 fields (E = -126 for subnormals) */
        union { float f; uint32_t u; } fa = { acc };
        const uint32_t ef = (fa.u >> 23) & 0xFFu, fr = fa.u & 0x7FFFFFu;
        const int E = ef ? (int)ef - 127 : -126;
        const i128 M = ef ? (i128)(fr | 0x800000u) : (i128)fr;
        const int sa = E - 23 - g;
        if (sa > 64)
            return acc;   /* |products| < 2^(g + frac + 2 + 5) is below a quarter of acc's spacing */
        const i128 sM = acc < 0 ? -M : M;
        S += sa >= 0 ? sM * ((i128)1 << sa) : cut_floor(sM, -sa);   /* no shift of a negative */
    }
    if (sum_bits > 0 && S != 0) {
        /* keep sum_bits bits from the leading one, or from 2^-126 below FP32's normal range */
        int lead = g + bitlen128(S < 0 ? -(unsigned __int128)S : (unsigned __int128)S) - 1;
        if (lead < -126)
            lead = -126;
        const int drop = lead - (sum_bits - 1) - g;
        if (drop > 0)
            S = cut_floor(S, drop) * ((i128)1 << drop);
    }
    return fp32_from_scaled(S, g);
}

static float elem_f32(const void *C, int ctype, int64_t idx)
{
    return (float)c_elem(C, ctype, idx);       /* FP16/BF16/FP32 -> float: exact */
}

/* The FP32 accumulator of one output element under the block model, from the decoded row
 * of op(A) and column of op(B) (k entries each). */
static float mfma_dot(const fp_parts *row, const fp_parts *col, int64_t k, int mb, int nblk,
                      int frac, int sum_bits)
{
    float acc = 0.0f;
    for (int64_t k0 = 0; k0 < k; k0 += nblk) {
        const int cnt = (int)(k - k0 < nblk ? k - k0 : nblk);
        acc = mfma_block(acc, row + k0, col + k0, cnt, mb, frac, sum_bits);
    }
    return acc;
}

/* Epilogue: alpha * acc when beta == 0 (C not read), else fma(alpha, acc, beta * c). */
static float mfma_epilogue(float acc, float alpha, float beta, const void *C, int ctype,
                           int64_t ldc, int64_t i, int64_t j)
{
    if (beta == 0.0f)
        return alpha * acc;
    return fmaf(alpha, acc, beta * elem_f32(C, ctype, i * ldc + j));
}

/* Decode row i of op(A) and column j of op(B) into k entries each. */
static void decode_row(fp_parts *out, const uint16_t *A, int transa, int64_t lda, int64_t i,
                       int64_t k, int t)
{
    for (int64_t p = 0; p < k; ++p)
        out[p] = parts16(A[a_index(transa, lda, i, p)], t);
}
static void decode_col(fp_parts *out, const uint16_t *B, int transb, int64_t ldb, int64_t j,
                       int64_t k, int t)
{
    for (int64_t p = 0; p < k; ++p)
        out[p] = parts16(B[b_index(transb, ldb, p, j)], t);
}

static void store_out(void *D, int otype, int64_t idx, float v)
{
    if (otype == ORC_F32) {
        union { float f; uint32_t u; } c = { v };
        ((uint32_t *)D)[idx] = c.u;
    } else {
        ((uint16_t *)D)[idx] = (uint16_t)oracle_encode_rne((double)v, ebits_of(otype),
                                                          mbits_of(otype));
    }
}

static int mfma_args_ok(int atype, int btype, int ctype, int otype, int nblk, int frac,
                        int sum_bits)
{
    if ((atype != ORC_F16 && atype != ORC_BF16) || btype != atype)
        return 0;
    if (ctype != ORC_F32 && ctype != ORC_F16 && ctype != ORC_BF16)
        return 0;
    if (otype != ORC_F32 && otype != ORC_F16 && otype != ORC_BF16)
        return 0;
    return nblk >= 1 && nblk <= 64 && frac >= 2 * mbits_of(atype) && frac <= 40 &&
           (sum_bits == 0 || (sum_bits >= 25 && sum_bits <= 100));
}

/*
 * Block-model GEMM at the points (ii[t], jj[t]); D[t] receives the output pattern (uint32
 * for ORC_F32, uint16 for ORC_F16/ORC_BF16).  Returns 0, or -1 on unsupported arguments
 * (input types must match; 1 <= nblk <= 64; 2 * fraction bits of the input <= frac <= 40;
 * sum_bits 0 or 25..100).
 */
int oracle_gemm_mfma_points(int transa, int transb, int64_t m, int64_t n, int64_t k,
                            float alpha, const void *A, int atype, int64_t lda, const void *B,
                            int btype, int64_t ldb, float beta, const void *C, int ctype,
                            int64_t ldc, int otype, int nblk, int frac, int sum_bits,
                            int64_t npts, const int64_t *ii, const int64_t *jj, void *D)
{
    (void)m; (void)n;
    if (!mfma_args_ok(atype, btype, ctype, otype, nblk, frac, sum_bits))
        return -1;
    const int mb = mbits_of(atype);
    int failed = 0;
#pragma omp parallel
    {
        fp_parts *row = malloc((size_t)(k > 0 ? k : 1) * sizeof(fp_parts));
        fp_parts *col = malloc((size_t)(k > 0 ? k : 1) * sizeof(fp_parts));
        if (!row || !col) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < npts; ++t) {
            if (!row || !col)
                continue;
            decode_row(row, (const uint16_t *)A, transa, lda, ii[t], k, atype);
            decode_col(col, (const uint16_t *)B, transb, ldb, jj[t], k, atype);
            const float acc = mfma_dot(row, col, k, mb, nblk, frac, sum_bits);
            store_out(D, otype, t, mfma_epilogue(acc, alpha, beta, C, ctype, ldc, ii[t], jj[t]));
        }
        free(row);
        free(col);
    }
    return failed ? -2 : 0;
}

/* Block-model GEMM over the whole m x n output (row-major D with stride n).  Every row of
 * op(A) and column of op(B) is decoded once. */
int oracle_gemm_mfma_full(int transa, int transb, int64_t m, int64_t n, int64_t k,
                          float alpha, const void *A, int atype, int64_t lda, const void *B,
                          int btype, int64_t ldb, float beta, const void *C, int ctype,
                          int64_t ldc, int otype, int nblk, int frac, int sum_bits,
                          void *D)
{
    if (!mfma_args_ok(atype, btype, ctype, otype, nblk, frac, sum_bits))
        return -1;
    const int mb = mbits_of(atype);
    const size_t kk = (size_t)(k > 0 ? k : 1);
    fp_parts *rows = malloc((size_t)(m > 0 ? m : 1) * kk * sizeof(fp_parts));
    fp_parts *cols = malloc((size_t)(n > 0 ? n : 1) * kk * sizeof(fp_parts));
    if (!rows || !cols) {
        free(rows);
        free(cols);
        return -2;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        decode_row(rows + i * kk, (const uint16_t *)A, transa, lda, i, k, atype);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        decode_col(cols + j * kk, (const uint16_t *)B, transb, ldb, j, k, atype);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            const float acc = mfma_dot(rows + i * kk, cols + j * kk, k, mb, nblk, frac, sum_bits);
            store_out(D, otype, i * n + j, mfma_epilogue(acc, alpha, beta, C, ctype, ldc, i, j));
        }
    free(rows);
    free(cols);
    return 0;
}

/* ======================================================================================
 * FP32 operands for the three-product BF16 GEMM (multiword emulation).
 *
 * "NVIDIA Tensor Core mixed-precision computing: principles and applications", section
 * 5.1: a high-precision operand is decomposed into pieces the matrix cores take and the
 * partial products are summed.  An FP32 value x becomes x_hi = RN_bf16(x) and
 * x_lo = RN_bf16(x - x_hi) (x - x_hi is exact in double), with x_lo = 0 when x_hi is
 * infinite or NaN.  The GEMM on the pieces is the block model above (or the exact sum).
 * ====================================================================================== */
int oracle_split_bf16(const float *x, int64_t count, uint16_t *hi, uint16_t *lo)
{
    for (int64_t t = 0; t < count; ++t) {
        const double v = (double)x[t];
        const uint64_t h = oracle_encode_rne(v, 8, 7);
        const double hv = oracle_decode(h, 8, 7);
        hi[t] = (uint16_t)h;
        lo[t] = isfinite(hv) ? (uint16_t)oracle_encode_rne(v - hv, 8, 7) : 0;
    }
    return 0;
}

/* Reference FP32 GEMM in double: v = alpha * sum a*b (+ beta * c), S = sum |a*b|, at the
 * points (ii[t], jj[t]).  An FP32 x FP32 product is exact in double. */
int oracle_gemm_f32_points(int transa, int transb, int64_t k, double alpha, const float *A,
                           int64_t lda, const float *B, int64_t ldb, double beta,
                           const float *C, int64_t ldc, int64_t npts, const int64_t *ii,
                           const int64_t *jj, double *v, double *S)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < npts; ++t) {
        double s = 0.0, sa = 0.0;
        for (int64_t p = 0; p < k; ++p) {
            const double prod = (double)A[a_index(transa, lda, ii[t], p)] *
                                (double)B[b_index(transb, ldb, p, jj[t])];
            s += prod;
            sa += fabs(prod);
        }
        v[t] = beta == 0.0 ? alpha * s : alpha * s + beta * (double)C[ii[t] * ldc + jj[t]];
        S[t] = sa;
    }
    return 0;
}

/* ======================================================================================
 * FP8 inputs.  "NVIDIA Tensor Core mixed-precision computing: principles and applications",
 * section 4.3.1, names the two FP8 formats, E4M3 (narrower range, more precision) and E5M2;
 * their fields are read here as the OCP definitions: E5M2 is IEEE-style (5 exponent bits,
 * bias 15, 2 fraction bits, infinities and NaNs at exponent 31), E4M3 has 4 exponent bits,
 * bias 7, 3 fraction bits, no infinities, and only S.1111.111 as NaN (exponent 15 is an
 * ordinary binade, up to 448).  Products of two FP8 values are exact in double.
 * ====================================================================================== */
enum { ORC_E4M3 = 5, ORC_E5M2 = 6 };

double oracle_decode_e4m3(uint32_t bits)
{
    const int s = (bits >> 7) & 1, e = (bits >> 3) & 15, f = bits & 7;
    double mag;
    if (e == 15 && f == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)f, 1 - 7 - 3);
    else
        mag = ldexp((double)(f | 8), e - 7 - 3);
    return s ? -mag : mag;
}

static double decode8(uint32_t bits, int t)
{
    return t == ORC_E4M3 ? oracle_decode_e4m3(bits) : oracle_decode(bits, 5, 2);
}

static void fp8_point(const double *tab_a, const double *tab_b, int transa, int transb,
                      int64_t k, double alpha, const uint8_t *A, int64_t lda,
                      const uint8_t *B, int64_t ldb, double beta, const void *C, int ctype,
                      int64_t ldc, int64_t i, int64_t j, double *v, double *S, double *bc)
{
    double s = 0.0, sa = 0.0;
    for (int64_t p = 0; p < k; ++p) {
        const double prod = tab_a[A[a_index(transa, lda, i, p)]] * tab_b[B[b_index(transb, ldb, p, j)]];
        s += prod;
        sa += fabs(prod);
    }
    double betac = 0.0, out;
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

static int fp8_types_ok(int atype, int btype, int ctype)
{
    return (atype == ORC_E4M3 || atype == ORC_E5M2) && (btype == ORC_E4M3 || btype == ORC_E5M2) &&
           (ctype == ORC_F32 || ctype == ORC_BF16 || ctype == ORC_F16);
}

/* FP8 GEMM at the points (ii[t], jj[t]): as oracle_gemm_fp_points, for FP8 A and B. */
int oracle_gemm_fp8_points(int transa, int transb, int64_t m, int64_t n, int64_t k,
                           double alpha, const void *A, int atype, int64_t lda, const void *B,
                           int btype, int64_t ldb, double beta, const void *C, int ctype,
                           int64_t ldc, int64_t npts, const int64_t *ii, const int64_t *jj,
                           double *v, double *S, double *bc)
{
    (void)m; (void)n;
    if (!fp8_types_ok(atype, btype, ctype))
        return -1;
    double tab_a[256], tab_b[256];
    for (uint32_t b = 0; b < 256; ++b) {
        tab_a[b] = decode8(b, atype);
        tab_b[b] = decode8(b, btype);
    }
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < npts; ++t)
        fp8_point(tab_a, tab_b, transa, transb, k, alpha, (const uint8_t *)A, lda,
                  (const uint8_t *)B, ldb, beta, C, ctype, ldc, ii[t], jj[t], &v[t], &S[t], &bc[t]);
    return 0;
}

/* FP8 GEMM over the whole m x n output (row-major v, S, bc with stride n). */
int oracle_gemm_fp8_full(int transa, int transb, int64_t m, int64_t n, int64_t k,
                         double alpha, const void *A, int atype, int64_t lda, const void *B,
                         int btype, int64_t ldb, double beta, const void *C, int ctype,
                         int64_t ldc, double *v, double *S, double *bc)
{
    if (!fp8_types_ok(atype, btype, ctype))
        return -1;
    double tab_a[256], tab_b[256];
    for (uint32_t b = 0; b < 256; ++b) {
        tab_a[b] = decode8(b, atype);
        tab_b[b] = decode8(b, btype);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            fp8_point(tab_a, tab_b, transa, transb, k, alpha, (const uint8_t *)A, lda,
                      (const uint8_t *)B, ldb, beta, C, ctype, ldc, i, j, &v[i * n + j],
                      &S[i * n + j], &bc[i * n + j]);
    return 0;
}

/* ======================================================================================
 * 2:4 structured-sparse A (the page "稀疏张量核心加速模板计算的技术解析", sparse tensor cores for
 * stencil computation, sections 1.2.1 and
 * 1.3.2: at most two nonzeros per group of 4 consecutive k, kept values plus 2 bits of
 * metadata each).  D(i, c) = alpha * sum_j Ac(i, j) * B(4 (j / 2) + idx(i, j), c)
 * (+ beta * C(i, c)), idx(i, j) = bits 2 (j % 4) .. +1 of meta byte (i, j / 4).
 * ====================================================================================== */
static void sp24_point(const double *tab, int transb, int64_t k, double alpha,
                       const uint16_t *Ac, int64_t lda, const uint8_t *meta, int64_t ld_meta,
                       const uint16_t *B, int64_t ldb, double beta, const void *C, int ctype,
                       int64_t ldc, int64_t i, int64_t c, double *v, double *S, double *bc)
{
    double s = 0.0, sa = 0.0;
    for (int64_t j = 0; j < k / 2; ++j) {
        const int idx = (meta[i * ld_meta + j / 4] >> (2 * (j % 4))) & 3;
        const int64_t kk = 4 * (j / 2) + idx;
        const double prod = tab[Ac[i * lda + j]] * tab[B[b_index(transb, ldb, kk, c)]];
        s += prod;
        sa += fabs(prod);
    }
    double betac = 0.0, out;
    if (beta == 0.0) {
        out = alpha * s;
    } else {
        betac = beta * c_elem(C, ctype, i * ldc + c);
        out = alpha * s + betac;
    }
    *v = out;
    *S = sa;
    *bc = betac;
}

int oracle_gemm_sp24_points(int transb, int64_t k, double alpha, const void *Ac, int atype,
                            int64_t lda, const void *meta, int64_t ld_meta, const void *B,
                            int64_t ldb, double beta, const void *C, int ctype, int64_t ldc,
                            int64_t npts, const int64_t *ii, const int64_t *jj, double *v,
                            double *S, double *bc)
{
    if (atype != ORC_F16 && atype != ORC_BF16)
        return -1;
    double *tab = malloc(65536 * sizeof(double));
    if (!tab)
        return -2;
    fill_table16(tab, atype);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < npts; ++t)
        sp24_point(tab, transb, k, alpha, (const uint16_t *)Ac, lda, (const uint8_t *)meta,
                   ld_meta, (const uint16_t *)B, ldb, beta, C, ctype, ldc, ii[t], jj[t], &v[t],
                   &S[t], &bc[t]);
    free(tab);
    return 0;
}

/* Block-model result of the 2:4 sparse GEMM at the points: the kept products
 * Ac(i, j) * B(4 (j / 2) + idx(i, j), c), in kept order j, go through the same block-FMA
 * accumulation as the dense model (blocks of nblk kept products), then the dense epilogue. */
int oracle_gemm_sp24_mfma_points(int transb, int64_t k, float alpha, const void *Ac, int atype,
                                 int64_t lda, const void *meta, int64_t ld_meta, const void *B,
                                 int64_t ldb, float beta, const void *C, int ctype, int64_t ldc,
                                 int otype, int nblk, int frac, int sum_bits, int64_t npts,
                                 const int64_t *ii, const int64_t *jj, void *D)
{
    if (!mfma_args_ok(atype, atype, ctype, otype, nblk, frac, sum_bits) || k % 4)
        return -1;
    const int mb = mbits_of(atype);
    const int64_t kh = k / 2;
    int failed = 0;
#pragma omp parallel
    {
        fp_parts *row = malloc((size_t)(kh > 0 ? kh : 1) * sizeof(fp_parts));
        fp_parts *col = malloc((size_t)(kh > 0 ? kh : 1) * sizeof(fp_parts));
        if (!row || !col) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < npts; ++t) {
            if (!row || !col)
                continue;
            const int64_t i = ii[t], c = jj[t];
            for (int64_t j = 0; j < kh; ++j) {
                const int idx = (((const uint8_t *)meta)[i * ld_meta + j / 4] >> (2 * (j % 4))) & 3;
                row[j] = parts16(((const uint16_t *)Ac)[i * lda + j], atype);
                col[j] = parts16(((const uint16_t *)B)[b_index(transb, ldb, 4 * (j / 2) + idx, c)],
                                 atype);
            }
            const float acc = mfma_dot(row, col, kh, mb, nblk, frac, sum_bits);
            store_out(D, otype, t, mfma_epilogue(acc, alpha, beta, C, ctype, ldc, i, c));
        }
        free(row);
        free(col);
    }
    return failed ? -2 : 0;
}

/* INT8 2:4 sparse A: D(i, c) = alpha * sum_j Ac(i, j) * B(4 (j / 2) + idx(i, j), c)
 * + beta * C(i, c), exact in int64, then wrapped modulo 2^32 like the dense INT8 oracle. */
int oracle_gemm_sp24_int_points(int transb, int64_t k, int64_t alpha, const int8_t *Ac,
                                int64_t lda, const uint8_t *meta, int64_t ld_meta,
                                const int8_t *B, int64_t ldb, int64_t beta, const int32_t *C,
                                int64_t ldc, int64_t npts, const int64_t *ii, const int64_t *jj,
                                int32_t *d)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < npts; ++t) {
        const int64_t i = ii[t], c = jj[t];
        int64_t s = 0;
        for (int64_t j = 0; j < k / 2; ++j) {
            const int idx = (meta[i * ld_meta + j / 4] >> (2 * (j % 4))) & 3;
            s += (int64_t)Ac[i * lda + j] * (int64_t)B[b_index(transb, ldb, 4 * (j / 2) + idx, c)];
        }
        uint64_t out = (uint64_t)alpha * (uint64_t)s;
        if (beta != 0)
            out += (uint64_t)beta * (uint64_t)(int64_t)C[i * ldc + c];
        d[t] = (int32_t)(uint32_t)out;
    }
    return 0;
}

/* FP8 (E4M3 / E5M2, either pairing) 2:4 sparse A: as oracle_gemm_sp24_points, the kept
 * products exact in double, with separate decode tables for A's and B's formats. */
int oracle_gemm_sp24_fp8_points(int transb, int64_t k, double alpha, const void *Ac, int atype,
                                int64_t lda, const void *meta, int64_t ld_meta, const void *B,
                                int btype, int64_t ldb, double beta, const void *C, int ctype,
                                int64_t ldc, int64_t npts, const int64_t *ii, const int64_t *jj,
                                double *v, double *S, double *bc)
{
    if (!fp8_types_ok(atype, btype, ctype))
        return -1;
    double tab_a[256], tab_b[256];
    for (uint32_t b = 0; b < 256; ++b) {
        tab_a[b] = decode8(b, atype);
        tab_b[b] = decode8(b, btype);
    }
    const uint8_t *a8 = (const uint8_t *)Ac, *b8 = (const uint8_t *)B, *m8 = (const uint8_t *)meta;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < npts; ++t) {
        const int64_t i = ii[t], c = jj[t];
        double s = 0.0, sa = 0.0;
        for (int64_t j = 0; j < k / 2; ++j) {
            const int idx = (m8[i * ld_meta + j / 4] >> (2 * (j % 4))) & 3;
            const double prod = tab_a[a8[i * lda + j]] * tab_b[b8[b_index(transb, ldb, 4 * (j / 2) + idx, c)]];
            s += prod;
            sa += fabs(prod);
        }
        double betac = 0.0, out;
        if (beta == 0.0) {
            out = alpha * s;
        } else {
            betac = beta * c_elem(C, ctype, i * ldc + c);
            out = alpha * s + betac;
        }
        v[t] = out;
        S[t] = sa;
        bc[t] = betac;
    }
    return 0;
}

/* ======================================================================================
 * Block model of the FP8 matrix-core accumulation (the numerics page's block-FMA model,
 * sections 2.2-2.3 and 4.2.1, in two levels).  One instruction covers `kinst` consecutive k:
 *   1. groups of `nblk` consecutive products: each group with a nonzero product has
 *      e_g = max(E(a) + E(b)) over its nonzero products (a subnormal operand counts with its
 *      format's minimum normal exponent); every product is cut toward zero to 2^(e_g - frac)
 *      and the group's products are summed exactly;
 *   2. blocks of `sblk` consecutive k (whole groups), in k order, each meets the FP32
 *      accumulator: for a block with a nonzero product, E = max e_g over its groups; its
 *      group sums are cut toward -infinity to 2^(E - wide) and added exactly into the block's
 *      total; where 2^(E - wide) is coarser than the accumulator's grid, the accumulator is cut
 *      toward -infinity to it, or dropped when its leading bit lies two or more places below
 *      that grid (the cut would borrow a whole unit from nothing); where the block lies so far
 *      below the accumulator that 2^(lead - accw) (lead: the accumulator's leading bit) is
 *      coarser than the block's grid, the total is cut once more, toward -infinity, to that;
 *      then accumulator + total, exactly, rounded to FP32, to nearest even.
 * The accumulator is the carried FP32 value throughout: instructions only delimit the k range
 * of one call.  Measured on gfx950: operands spread over 12 and 24 binades decide the rounding
 * after each block and the accumulator's window (wide = 24, accw = 31) bit for bit, probe
 * vectors the accumulator's cut and drop; narrow ranges and the probe vectors of the group
 * window and the blocks fix the rest.
 * ====================================================================================== */
static fp_parts parts8(uint8_t bits, int t)
{
    const int e4 = t == ORC_E4M3;
    const int eb = e4 ? 4 : 5, mb = e4 ? 3 : 2, bias = e4 ? 7 : 15;
    const uint32_t f = bits & ((1u << mb) - 1), e = (bits >> mb) & ((1u << eb) - 1);
    fp_parts p = { 0, 0, (uint8_t)(bits >> 7), 0 };
    if (e4 && e == 15 && f == 7) {
        p.kind = 2;                                /* E4M3: S.1111.111 is NaN, no infinities */
    } else if (!e4 && e == 31) {
        p.kind = f ? 2 : 1;                        /* E5M2: IEEE-style infinities and NaNs */
    } else if (e == 0) {
        p.expo = (int16_t)(1 - bias);
        p.mant = f;
    } else {
        p.expo = (int16_t)((int)e - bias);
        p.mant = f | (1u << mb);
    }
    return p;
}

#define FP8_MAX_GROUPS 64

static float fp8_inst(float acc, const fp_parts *a, const fp_parts *b, int mba, int mbb, int cnt,
                      int nblk, int sblk, int frac, int wide, int accw)
{
    int nan = isnan(acc), pinf = isinf(acc) && acc > 0, ninf = isinf(acc) && acc < 0;
    for (int t = 0; t < cnt; ++t) {
        const int neg = a[t].neg ^ b[t].neg;
        if (a[t].kind == 2 || b[t].kind == 2) {
            nan = 1;
        } else if (a[t].kind == 1 || b[t].kind == 1) {
            const int other_zero = a[t].kind == 1 ? (b[t].kind == 0 && b[t].mant == 0)
                                                  : (a[t].mant == 0);
            if (other_zero)
                nan = 1;
            else if (neg)
                ninf = 1;
            else
                pinf = 1;
        }
    }
    if (nan || (pinf && ninf))
        return NAN;
    if (pinf)
        return INFINITY;
    if (ninf)
        return -INFINITY;

    /* level 1: group sums, group q exact on the grid 2^(eg[q] - frac) */
    i128 gsum[FP8_MAX_GROUPS];
    int eg[FP8_MAX_GROUPS], ng = 0, have = 0, E = 0;
    for (int b0 = 0; b0 < cnt && ng < FP8_MAX_GROUPS; b0 += nblk, ++ng) {
        const int n = cnt - b0 < nblk ? cnt - b0 : nblk;
        int e = 0, any = 0;
        for (int t = b0; t < b0 + n; ++t)
            if (a[t].mant && b[t].mant) {
                const int x = a[t].expo + b[t].expo;
                if (!any || x > e)
                    e = x;
                any = 1;
            }
        gsum[ng] = 0;
        eg[ng] = any ? e : INT_MIN;
        if (!any)
            continue;
        if (!have || e > E)
            E = e;
        have = 1;
        const int g = e - frac;
        for (int t = b0; t < b0 + n; ++t) {
            if (!a[t].mant || !b[t].mant)
                continue;
            const i128 pm = (i128)((uint64_t)a[t].mant * b[t].mant);
            const i128 sp = (a[t].neg ^ b[t].neg) ? -pm : pm;       /* signed product */
            const int sh = a[t].expo + b[t].expo - mba - mbb - g;   /* = sp * 2^(sh + g) */
            gsum[ng] += sh >= 0 ? sp * ((i128)1 << sh) : cut_toward_zero(sp, -sh);
        }
    }
    if (!have)
        return acc;
    (void)E;
    /* level 2: blocks of sblk / nblk groups, in k order, each added to the running FP32 value
     * (the accumulator, S * 2^G exactly) and the result rounded to FP32 */
    const int per = sblk / nblk;
    i128 S = 0;
    int G = 0, started = 0;
    if (acc != 0.0f) {
        union { float f; uint32_t u; } fa = { acc };
        const uint32_t ef = (fa.u >> 23) & 0xFFu, fr = fa.u & 0x7FFFFFu;
        const i128 M = ef ? (i128)(fr | 0x800000u) : (i128)fr;
        S = acc < 0 ? -M : M;
        G = (ef ? (int)ef - 127 : -126) - 23;
        started = 1;
    }
    for (int q0 = 0; q0 < ng; q0 += per) {
        int Eb = INT_MIN;
        for (int q = q0; q < q0 + per && q < ng; ++q)
            if (eg[q] != INT_MIN && eg[q] > Eb)
                Eb = eg[q];
        if (Eb == INT_MIN)
            continue;
        const int Gb = Eb - wide;
        /* a block far below the accumulator: its total is cut once more, toward -infinity,
         * to accw bits below the accumulator's leading bit (accw = 0: no such cut) */
        int Gt = INT_MIN;
        if (started && S != 0 && accw > 0) {
            const unsigned __int128 us = S < 0 ? -(unsigned __int128)S : (unsigned __int128)S;
            const int Ga = G + bitlen128(us) - 1 - accw;
            if (Ga > Gb)
                Gt = Ga;
        }
        if (!started) {
            G = Gb;
            started = 1;
        } else if (Gb > G) {
            /* cut toward -infinity to the block's grid; an accumulator whose leading bit lies
             * two or more places below that grid is dropped instead (no borrow of one unit) */
            const unsigned __int128 us = S < 0 ? -(unsigned __int128)S : (unsigned __int128)S;
            if (G + bitlen128(us) - 1 <= Gb - 2)
                S = 0;
            else
                S = cut_floor(S, Gb - G);
            G = Gb;
        } else if (Gb < G) {
            S = S * ((i128)1 << (G - Gb));
            G = Gb;
        }
        /* the block's total T on its grid 2^Gb (= 2^G now): group sums cut toward -infinity */
        i128 T = 0;
        for (int q = q0; q < q0 + per && q < ng; ++q) {
            if (eg[q] == INT_MIN)
                continue;
            const int d = eg[q] - frac - G;        /* group grid relative to 2^G */
            T += d >= 0 ? gsum[q] * ((i128)1 << d) : cut_floor(gsum[q], -d);
        }
        if (Gt != INT_MIN)
            T = cut_floor(T, Gt - G) * ((i128)1 << (Gt - G));
        S += T;
        /* the block's result is an FP32 value: 24 significant bits, ties to even (FP8 sums
         * stay far above FP32's subnormal range and below its overflow) */
        S = round_to_bits(S, &G, 24);
    }
    return fp32_from_scaled(S, G);
}

/* FP8 GEMM through the instruction model at the points; D[t] gets the output pattern. */
int oracle_gemm_fp8_mfma_points(int transa, int transb, int64_t k, float alpha, const void *A,
                                int atype, int64_t lda, const void *B, int btype, int64_t ldb,
                                float beta, const void *C, int ctype, int64_t ldc, int otype,
                                int kinst, int nblk, int sblk, int frac, int wide, int accw,
                                int64_t npts, const int64_t *ii, const int64_t *jj, void *D)
{
    if (!fp8_types_ok(atype, btype, ctype) || (otype != ORC_F32 && otype != ORC_BF16) ||
        kinst < 1 || nblk < 1 || kinst > nblk * FP8_MAX_GROUPS || sblk < nblk ||
        sblk % nblk || frac < 4 || frac > 40 || wide < frac || wide > 60 || accw < 0 || accw > 90)
        return -1;
    const int mba = atype == ORC_E4M3 ? 3 : 2, mbb = btype == ORC_E4M3 ? 3 : 2;
    int failed = 0;
#pragma omp parallel
    {
        fp_parts *row = malloc((size_t)(k > 0 ? k : 1) * sizeof(fp_parts));
        fp_parts *col = malloc((size_t)(k > 0 ? k : 1) * sizeof(fp_parts));
        if (!row || !col) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < npts; ++t) {
            if (!row || !col)
                continue;
            for (int64_t p = 0; p < k; ++p) {
                row[p] = parts8(((const uint8_t *)A)[a_index(transa, lda, ii[t], p)], atype);
                col[p] = parts8(((const uint8_t *)B)[b_index(transb, ldb, p, jj[t])], btype);
            }
            float acc = 0.0f;
            for (int64_t k0 = 0; k0 < k; k0 += kinst) {
                const int cnt = (int)(k - k0 < kinst ? k - k0 : kinst);
                acc = fp8_inst(acc, row + k0, col + k0, mba, mbb, cnt, nblk, sblk, frac, wide, accw);
            }
            store_out(D, otype, t, mfma_epilogue(acc, alpha, beta, C, ctype, ldc, ii[t], jj[t]));
        }
        free(row);
        free(col);
    }
    return failed ? -2 : 0;
}

/* The FP8 block model over the kept products of a 2:4 sparse A, in kept order: instructions of
 * `kinst` kept products, as oracle_gemm_fp8_mfma_points. */
int oracle_gemm_sp24_fp8_mfma_points(int transb, int64_t k, float alpha, const void *Ac, int atype,
                                     int64_t lda, const void *meta, int64_t ld_meta,
                                     const void *B, int btype, int64_t ldb, float beta,
                                     const void *C, int ctype, int64_t ldc, int otype, int kinst,
                                     int nblk, int sblk, int frac, int wide, int accw,
                                     int64_t npts, const int64_t *ii, const int64_t *jj, void *D)
{
    if (!fp8_types_ok(atype, btype, ctype) || (otype != ORC_F32 && otype != ORC_BF16) ||
        kinst < 1 || nblk < 1 || kinst > nblk * FP8_MAX_GROUPS || sblk < nblk ||
        sblk % nblk || frac < 4 || frac > 40 || wide < frac || wide > 60 || accw < 0 ||
        accw > 90 || k % 4)
        return -1;
    const int mba = atype == ORC_E4M3 ? 3 : 2, mbb = btype == ORC_E4M3 ? 3 : 2;
    const int64_t kh = k / 2;
    int failed = 0;
#pragma omp parallel
    {
        fp_parts *row = malloc((size_t)(kh > 0 ? kh : 1) * sizeof(fp_parts));
        fp_parts *col = malloc((size_t)(kh > 0 ? kh : 1) * sizeof(fp_parts));
        if (!row || !col) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < npts; ++t) {
            if (!row || !col)
                continue;
            const int64_t i = ii[t], c = jj[t];
            for (int64_t j = 0; j < kh; ++j) {
                const int idx = (((const uint8_t *)meta)[i * ld_meta + j / 4] >> (2 * (j % 4))) & 3;
                row[j] = parts8(((const uint8_t *)Ac)[i * lda + j], atype);
                col[j] = parts8(((const uint8_t *)B)[b_index(transb, ldb, 4 * (j / 2) + idx, c)], btype);
            }
            float acc = 0.0f;
            for (int64_t j0 = 0; j0 < kh; j0 += kinst) {
                const int cnt = (int)(kh - j0 < kinst ? kh - j0 : kinst);
                acc = fp8_inst(acc, row + j0, col + j0, mba, mbb, cnt, nblk, sblk, frac, wide, accw);
            }
            store_out(D, otype, t, mfma_epilogue(acc, alpha, beta, C, ctype, ldc, i, c));
        }
        free(row);
        free(col);
    }
    return failed ? -2 : 0;
}
