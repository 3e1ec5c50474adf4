/*
 * gemm_oracle.c -- plain CPU reference for the dense matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * GPU path.
 *
 * What it computes (page "10. Tensor Cores, shapes, and tile alignment",
 * section "Shape the operation", the problem statement C(MxN) = A(MxK) B(KxN)
 * and the FLOPs equation): every output is the full K-term dot product of a
 * row of A with a column of B.  Inputs are decoded once to binary64, the
 * products and their sums are formed in binary64 by a plain i-k-j triple loop,
 * and the result is multiplied by alpha (1 for bf16, s_A*s_B for E4M3 with
 * per-tensor scales).  The same loop also forms
 *     W[i][j] = |alpha| * sum_k |a(i,k) b(k,j)|,
 * the magnitude the parity tolerance is scaled by.
 *
 * Products of two bf16 (8-bit significands) or two E4M3 (4-bit significands)
 * values are exact in binary64; the only rounding is in the binary64 sums
 * (at most K * 2^-53 * W), so for every shape used here the result is the
 * exact product to far below any tolerance that is applied to it.
 *
 * Element formats (decoded from their definitions, not from any library):
 *   bf16  : the upper 16 bits of an IEEE-754 binary32 value.
 *   E4M3  : the OCP 8-bit float "E4M3FN": 1 sign, 4 exponent (bias 7) and
 *           3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6);
 *           S.1111.111 is NaN; there is no infinity; the largest finite
 *           magnitude is 1.75 * 2^8 = 448.
 *   E5M2  : the OCP 8-bit float "E5M2": 1 sign, 5 exponent (bias 15) and
 *           2 mantissa bits; exponent field 0 is subnormal (m/4 * 2^-14);
 *           exponent field 31 is infinity (m = 0) or NaN; the largest finite
 *           magnitude is 1.75 * 2^15 = 57344.
 *   The low-precision input table on page "The Tensor Core" lists E4M3 and
 *   E5M2 as the Hopper-row FP8 inputs.  A and B may use different formats.
 *
 * Operand addressing (leading dimensions as in that page's WMMA example):
 *   a_colmajor = 0 : a(i,k) = A[i*lda + k]   (A row-major, M rows of K)
 *   a_colmajor = 1 : a(i,k) = A[k*lda + i]   (A column-major)
 *   b_rowmajor = 0 : b(k,j) = B[j*ldb + k]   (B column-major, N columns of K)
 *   b_rowmajor = 1 : b(k,j) = B[k*ldb + j]   (B row-major)
 * C and W are dense row-major M x N binary64 arrays owned by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_E4M3 = 1, ORACLE_E5M2 = 2 };

static double decode_bf16(uint16_t code)
{
    uint32_t bits = (uint32_t)code << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double decode_e4m3(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);            /* (m/8) * 2^(1-7) */
    else
        mag = ldexp(8.0 + (double)m, e - 10);  /* (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

static double decode_e5m2(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 2) & 0x1F;
    int m = code & 0x3;
    double mag;
    if (e == 0x1F)
        mag = m == 0 ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m, -16);           /* (m/4) * 2^(1-15) */
    else
        mag = ldexp(4.0 + (double)m, e - 17);  /* (1 + m/4) * 2^(e-15) */
    return sign ? -mag : mag;
}

static double decode(const void *base, int64_t idx, int fmt)
{
    if (fmt == ORACLE_BF16)
        return decode_bf16(((const uint16_t *)base)[idx]);
    if (fmt == ORACLE_E5M2)
        return decode_e5m2(((const uint8_t *)base)[idx]);
    return decode_e4m3(((const uint8_t *)base)[idx]);
}

static int64_t a_index(int64_t i, int64_t k, int64_t lda, int a_colmajor)
{
    return a_colmajor ? k * lda + i : i * lda + k;
}

static int64_t b_index(int64_t k, int64_t j, int64_t ldb, int b_rowmajor)
{
    return b_rowmajor ? k * ldb + j : j * ldb + k;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full product.  Returns the number of multiply-adds executed (M*N*K when
 * every term is formed), or -1 if a scratch allocation failed.
 */
int64_t oracle_gemm(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda, int a_colmajor,
                    const void *B, int64_t ldb, int b_rowmajor,
                    int fmt_a, int fmt_b, double alpha, double *C, double *W)
{
    int64_t i, j, k, macs = 0;
    double *a = NULL, *b = NULL;

    if (M <= 0 || N <= 0) return 0;
    a = (double *)malloc(sizeof(double) * (size_t)(M * (K > 0 ? K : 1)));
    b = (double *)malloc(sizeof(double) * (size_t)((K > 0 ? K : 1) * N));
    if (!a || !b) { free(a); free(b); return -1; }

    /* decode once: a as dense M x K, b as dense K x N (both row-major) */
    for (i = 0; i < M; ++i)
        for (k = 0; k < K; ++k)
            a[i * K + k] = decode(A, a_index(i, k, lda, a_colmajor), fmt_a);
    for (k = 0; k < K; ++k)
        for (j = 0; j < N; ++j)
            b[k * N + j] = decode(B, b_index(k, j, ldb, b_rowmajor), fmt_b);

#pragma omp parallel for schedule(static) private(j, k) reduction(+ : macs)
    for (i = 0; i < M; ++i) {
        double *c = C + i * N;
        double *w = W ? W + i * N : NULL;
        for (j = 0; j < N; ++j) c[j] = 0.0;
        if (w) for (j = 0; j < N; ++j) w[j] = 0.0;
        for (k = 0; k < K; ++k) {
            const double aik = a[i * K + k];
            const double *bk = b + k * N;
            if (w) {
                for (j = 0; j < N; ++j) {
                    const double p = aik * bk[j];
                    c[j] += p;
                    w[j] += fabs(p);
                }
            } else {
                for (j = 0; j < N; ++j) c[j] += aik * bk[j];
            }
            macs += N;
        }
        for (j = 0; j < N; ++j) c[j] *= alpha;
        if (w) for (j = 0; j < N; ++j) w[j] *= fabs(alpha);
    }
    free(a);
    free(b);
    return macs;
}

/*
 * Selected entries only: c[t] = C[ii[t]][jj[t]] and w[t] = W[ii[t]][jj[t]]
 * of the same product, each formed as its own K-term dot product.  Used where
 * the full product is too large for the CPU.  Returns the multiply-adds done.
 */
int64_t oracle_gemm_entries(int64_t K,
                            const void *A, int64_t lda, int a_colmajor,
                            const void *B, int64_t ldb, int b_rowmajor,
                            int fmt_a, int fmt_b, double alpha,
                            int64_t n, const int64_t *ii, const int64_t *jj,
                            double *c, double *w)
{
    int64_t t, macs = 0;
#pragma omp parallel for schedule(static) reduction(+ : macs)
    for (t = 0; t < n; ++t) {
        double s = 0.0, sa = 0.0;
        int64_t k;
        for (k = 0; k < K; ++k) {
            const double p = decode(A, a_index(ii[t], k, lda, a_colmajor), fmt_a) *
                             decode(B, b_index(k, jj[t], ldb, b_rowmajor), fmt_b);
            s += p;
            sa += fabs(p);
        }
        c[t] = alpha * s;
        if (w) w[t] = fabs(alpha) * sa;
        macs += K;
    }
    return macs;
}

/* Element decoders exposed for the codec pins. */
double oracle_decode_bf16(uint16_t code) { return decode_bf16(code); }
double oracle_decode_e4m3(uint8_t code) { return decode_e4m3(code); }
double oracle_decode_e5m2(uint8_t code) { return decode_e5m2(code); }
