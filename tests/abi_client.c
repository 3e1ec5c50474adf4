/*
 * A C program that uses libgemm355 through its C interface alone: device
 * memory from hipMalloc, a stream from hipStreamCreate, and no other GPU
 * runtime in the process.  Operands hold small integers, so every product
 * is an exact integer in fp32 whatever the summation order (|C| < 2^24),
 * and the check against a host int64 loop is bit-exact.
 *
 * Covers gemm355_gemm (automatic plan, forced split-K with its combine pass,
 * persistent grid), gemm355_gemm_ex (E4M3 operands, bf16 output, batch with
 * per-entry scales, a caller workspace), gemm355_gemm_noalloc, gemm355_plan,
 * the convolution entry points (output size, plan, automatic and split-K
 * runs), the per-tensor quantiser (fp32 and bf16 sources, both 8-bit
 * formats), K == 0, and an argument error.  Prints one line per case; exit status 0
 * when all agree.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gemm355.h"

static int failures = 0;

#define HIP_OK(call)                                                          \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,   \
                    hipGetErrorString(e_));                                   \
            exit(3);                                                          \
        }                                                                     \
    } while (0)

static void expect_status(const char *name, gemm355_status got, gemm355_status want)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d\n", name, (int)got,
                gemm355_status_string(got), (int)want);
        ++failures;
    }
}

/* Small integers in [-4, 4] from a fixed linear congruential sequence. */
static uint32_t lcg_state = 12345u;
static int next_small(void)
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (int)((lcg_state >> 16) % 9u) - 4;
}

static uint16_t bf16_of_int(int v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);   /* exact: |v| <= 4 has few mantissa bits */
}

/* OCP E4M3FN codes of -4 .. 4 (bias 7; 3 = 1.5 * 2). */
static uint8_t e4m3_of_int(int v)
{
    static const uint8_t mag[5] = {0x00, 0x38, 0x40, 0x44, 0x48};
    uint8_t c = mag[v < 0 ? -v : v];
    return (uint8_t)(v < 0 ? (c | 0x80) : c);
}

/* OCP E5M2 codes of -4 .. 4 (bias 15; 3 = 1.5 * 2). */
static uint8_t e5m2_of_int(int v)
{
    static const uint8_t mag[5] = {0x00, 0x3C, 0x40, 0x42, 0x44};
    uint8_t c = mag[v < 0 ? -v : v];
    return (uint8_t)(v < 0 ? (c | 0x80) : c);
}

/* fp32 -> bf16, round to nearest even (finite inputs). */
static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ref[g][i][j] = sum_k a[g][i][k] * b[g][j][k] (A row-major, B column-major). */
static void reference(int64_t batch, int64_t M, int64_t N, int64_t K,
                      const int8_t *a, const int8_t *b, int64_t *ref)
{
    for (int64_t g = 0; g < batch; ++g)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                int64_t s = 0;
                for (int64_t k = 0; k < K; ++k)
                    s += (int64_t)a[(g * M + i) * K + k] * b[(g * N + j) * K + k];
                ref[(g * M + i) * N + j] = s;
            }
}

static void check_f32(const char *name, const float *c, const int64_t *ref,
                      int64_t count, double alpha)
{
    int64_t bad = 0;
    for (int64_t e = 0; e < count; ++e)
        if (c[e] != (float)(alpha * (double)ref[e])) {
            if (bad < 3)
                fprintf(stderr, "%s: element %lld = %.9g, expected %.9g\n", name,
                        (long long)e, (double)c[e], alpha * (double)ref[e]);
            ++bad;
        }
    if (bad) {
        fprintf(stderr, "%s: %lld of %lld elements differ\n", name, (long long)bad,
                (long long)count);
        ++failures;
    } else {
        printf("case %s ok (%lld elements)\n", name, (long long)count);
    }
}

int main(void)
{
    const int64_t M = 300, N = 200, K = 520, BATCH = 2;
    int ndev = 0;
    HIP_OK(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        fprintf(stderr, "no device\n");
        return 3;
    }
    HIP_OK(hipSetDevice(0));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    int8_t *a = malloc((size_t)(BATCH * M * K));
    int8_t *b = malloc((size_t)(BATCH * N * K));
    int64_t *ref = malloc(sizeof(int64_t) * (size_t)(BATCH * M * N));
    uint16_t *a16 = malloc(2 * (size_t)(M * K));
    uint16_t *b16 = malloc(2 * (size_t)(N * K));
    uint8_t *a8 = malloc((size_t)(BATCH * M * K));
    uint8_t *b8 = malloc((size_t)(BATCH * N * K));
    float *c = malloc(sizeof(float) * (size_t)(BATCH * M * N));
    uint16_t *c16 = malloc(2 * (size_t)(M * N));
    if (!a || !b || !ref || !a16 || !b16 || !a8 || !b8 || !c || !c16) {
        fprintf(stderr, "host allocation failed\n");
        return 3;
    }
    for (int64_t e = 0; e < BATCH * M * K; ++e) a[e] = (int8_t)next_small();
    for (int64_t e = 0; e < BATCH * N * K; ++e) b[e] = (int8_t)next_small();
    for (int64_t e = 0; e < M * K; ++e) a16[e] = bf16_of_int(a[e]);
    for (int64_t e = 0; e < N * K; ++e) b16[e] = bf16_of_int(b[e]);
    for (int64_t e = 0; e < BATCH * M * K; ++e) a8[e] = e4m3_of_int(a[e]);
    for (int64_t e = 0; e < BATCH * N * K; ++e) b8[e] = e4m3_of_int(b[e]);
    reference(BATCH, M, N, K, a, b, ref);

    void *dA, *dB, *dC, *dA8, *dB8, *dWs, *dScale;
    const size_t ws_bytes = (size_t)64 << 20;
    HIP_OK(hipMalloc(&dA, 2 * (size_t)(M * K)));
    HIP_OK(hipMalloc(&dB, 2 * (size_t)(N * K)));
    HIP_OK(hipMalloc(&dC, sizeof(float) * (size_t)(BATCH * M * N)));
    HIP_OK(hipMalloc(&dA8, (size_t)(BATCH * M * K)));
    HIP_OK(hipMalloc(&dB8, (size_t)(BATCH * N * K)));
    HIP_OK(hipMalloc(&dWs, ws_bytes));
    HIP_OK(hipMalloc(&dScale, 4 * sizeof(float)));
    HIP_OK(hipMemcpy(dA, a16, 2 * (size_t)(M * K), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dB, b16, 2 * (size_t)(N * K), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dA8, a8, (size_t)(BATCH * M * K), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dB8, b8, (size_t)(BATCH * N * K), hipMemcpyHostToDevice));
    /* scale_a = {0.5, 2}, scale_b = {2, 0.25}: alpha = {1, 0.5}, exact. */
    const float scales[4] = {0.5f, 2.0f, 2.0f, 0.25f};
    HIP_OK(hipMemcpy(dScale, scales, sizeof scales, hipMemcpyHostToDevice));
    const size_t c_bytes = sizeof(float) * (size_t)(M * N);

    /* bf16 -> fp32 through the short entry point: automatic, forced split-K
     * (partials plus the combine kernel), persistent grid. */
    static const struct { const char *name; int32_t split, persistent; } modes[] = {
        {"gemm_bf16_auto", 0, -1}, {"gemm_bf16_split4", 4, 0}, {"gemm_bf16_persistent", 1, 1}};
    for (size_t m = 0; m < sizeof modes / sizeof modes[0]; ++m) {
        HIP_OK(hipMemsetAsync(dC, 0xFF, c_bytes, stream));   /* NaN fill */
        expect_status(modes[m].name,
                      gemm355_gemm(M, N, K, dA, K, dB, K, dC, N, GEMM355_BF16_F32,
                                   GEMM355_A_ROW_B_COL, modes[m].split, modes[m].persistent,
                                   (void *)stream),
                      GEMM355_OK);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(c, dC, c_bytes, hipMemcpyDeviceToHost));
        check_f32(modes[m].name, c, ref, M * N, 1.0);
    }

    /* The plan of the forced split-K call agrees with what it asked for. */
    gemm355_args args;
    memset(&args, 0, sizeof args);
    args.M = M; args.N = N; args.K = K;
    args.A = dA; args.lda = K; args.B = dB; args.ldb = K; args.C = dC; args.ldc = N;
    args.batch = 1; args.dtype = GEMM355_BF16_F32; args.layout = GEMM355_A_ROW_B_COL;
    args.split_k = 4; args.persistent = 0; args.tile = -1;
    gemm355_plan_t plan;
    expect_status("plan", gemm355_plan(&args, &plan), GEMM355_OK);
    if (plan.split < 2 || plan.units != plan.G * plan.split || plan.workspace_bytes == 0 ||
        plan.eta_pad_num <= 0 || plan.eta_pad_num > plan.eta_pad_den) {
        fprintf(stderr, "plan: split %d units %lld G %lld workspace %zu\n", plan.split,
                (long long)plan.units, (long long)plan.G, plan.workspace_bytes);
        ++failures;
    } else {
        printf("case plan ok (tile %d, split %d, %lld units)\n", plan.tile, plan.split,
               (long long)plan.units);
    }

    /* E4M3 -> bf16 with the full argument set and a caller workspace: the
     * bf16 output is the exact integer rounded to nearest even. */
    args.A = dA8; args.B = dB8; args.dtype = GEMM355_E4M3_BF16; args.split_k = 3;
    args.workspace = dWs; args.workspace_bytes = ws_bytes;
    HIP_OK(hipMemsetAsync(dC, 0xFF, c_bytes, stream));
    expect_status("gemm_ex_e4m3_bf16", gemm355_gemm_ex(&args, (void *)stream), GEMM355_OK);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(c16, dC, 2 * (size_t)(M * N), hipMemcpyDeviceToHost));
    {
        int64_t bad = 0;
        for (int64_t e = 0; e < M * N; ++e)
            if (c16[e] != bf16_rne((float)ref[e])) ++bad;
        if (bad) {
            fprintf(stderr, "gemm_ex_e4m3_bf16: %lld elements differ\n", (long long)bad);
            ++failures;
        } else {
            printf("case gemm_ex_e4m3_bf16 ok (%lld elements)\n", (long long)(M * N));
        }
    }

    /* Batch of two E4M3 products with per-entry scales, through the entry
     * point that allocates nothing, split along K. */
    args.dtype = GEMM355_E4M3_F32; args.batch = BATCH;
    args.stride_a = M * K; args.stride_b = N * K; args.stride_c = M * N;
    args.scale_a = (const float *)dScale; args.scale_b = (const float *)dScale + 2;
    args.workspace = NULL; args.workspace_bytes = 0; args.split_k = 2;
    HIP_OK(hipMemsetAsync(dC, 0xFF, 2 * c_bytes, stream));
    expect_status("gemm_noalloc_batch", gemm355_gemm_noalloc(&args, (void *)stream), GEMM355_OK);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(c, dC, 2 * c_bytes, hipMemcpyDeviceToHost));
    check_f32("gemm_noalloc_batch_0", c, ref, M * N, 1.0);
    check_f32("gemm_noalloc_batch_1", c + M * N, ref + M * N, M * N, 0.5);

    /* Convolution (bf16 NHWC images, KRSC filters, fp32 NPQK output) with
     * padding, stride and dilation, automatic and split along K, against a
     * direct loop over the window. */
    {
        gemm355_conv_args cv;
        memset(&cv, 0, sizeof cv);
        cv.N = 2; cv.H = 9; cv.W = 11; cv.C = 64; cv.K = 40; cv.R = 3; cv.S = 2;
        cv.pad_h = 1; cv.pad_w = 1; cv.stride_h = 2; cv.stride_w = 1; cv.dil_h = 1; cv.dil_w = 2;
        cv.dtype = GEMM355_BF16_F32; cv.tile = -1; cv.persistent = -1;
        int64_t P = 0, Q = 0;
        expect_status("conv_out_size", gemm355_conv2d_out_size(&cv, &P, &Q), GEMM355_OK);
        if (P != 5 || Q != 11) {
            fprintf(stderr, "conv_out_size: P %lld Q %lld, expected 5 and 11\n", (long long)P, (long long)Q);
            ++failures;
        }
        const int64_t nx = cv.N * cv.H * cv.W * cv.C, nw = cv.K * cv.R * cv.S * cv.C;
        const int64_t ny = cv.N * P * Q * cv.K;
        int8_t *x = malloc((size_t)nx), *w = malloc((size_t)nw);
        uint16_t *x16 = malloc(2 * (size_t)nx), *w16 = malloc(2 * (size_t)nw);
        int64_t *yref = malloc(sizeof(int64_t) * (size_t)ny);
        float *y = malloc(sizeof(float) * (size_t)ny);
        if (!x || !w || !x16 || !w16 || !yref || !y) {
            fprintf(stderr, "host allocation failed\n");
            return 3;
        }
        for (int64_t e = 0; e < nx; ++e) { x[e] = (int8_t)next_small(); x16[e] = bf16_of_int(x[e]); }
        for (int64_t e = 0; e < nw; ++e) { w[e] = (int8_t)next_small(); w16[e] = bf16_of_int(w[e]); }
        for (int64_t n = 0; n < cv.N; ++n)
            for (int64_t p = 0; p < P; ++p)
                for (int64_t q = 0; q < Q; ++q)
                    for (int64_t k = 0; k < cv.K; ++k) {
                        int64_t acc = 0;
                        for (int64_t r = 0; r < cv.R; ++r)
                            for (int64_t t = 0; t < cv.S; ++t) {
                                const int64_t h = p * cv.stride_h - cv.pad_h + r * cv.dil_h;
                                const int64_t v = q * cv.stride_w - cv.pad_w + t * cv.dil_w;
                                if (h < 0 || h >= cv.H || v < 0 || v >= cv.W) continue;
                                for (int64_t c = 0; c < cv.C; ++c)
                                    acc += (int64_t)x[((n * cv.H + h) * cv.W + v) * cv.C + c] *
                                           w[((k * cv.R + r) * cv.S + t) * cv.C + c];
                            }
                        yref[((n * P + p) * Q + q) * cv.K + k] = acc;
                    }
        void *dx, *dw, *dy;
        HIP_OK(hipMalloc(&dx, 2 * (size_t)nx));
        HIP_OK(hipMalloc(&dw, 2 * (size_t)nw));
        HIP_OK(hipMalloc(&dy, sizeof(float) * (size_t)ny));
        HIP_OK(hipMemcpy(dx, x16, 2 * (size_t)nx, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dw, w16, 2 * (size_t)nw, hipMemcpyHostToDevice));
        cv.x = dx; cv.w = dw; cv.y = dy;
        gemm355_plan_t cplan;
        expect_status("conv_plan", gemm355_conv2d_plan(&cv, &cplan), GEMM355_OK);
        static const struct { const char *name; int32_t split; } cmodes[] = {
            {"conv_auto", 0}, {"conv_split3", 3}};
        for (size_t m = 0; m < sizeof cmodes / sizeof cmodes[0]; ++m) {
            cv.split_k = cmodes[m].split;
            HIP_OK(hipMemsetAsync(dy, 0xFF, sizeof(float) * (size_t)ny, stream));
            expect_status(cmodes[m].name, gemm355_conv2d(&cv, (void *)stream), GEMM355_OK);
            HIP_OK(hipStreamSynchronize(stream));
            HIP_OK(hipMemcpy(y, dy, sizeof(float) * (size_t)ny, hipMemcpyDeviceToHost));
            check_f32(cmodes[m].name, y, yref, ny, 1.0);
        }
        HIP_OK(hipFree(dx)); HIP_OK(hipFree(dw)); HIP_OK(hipFree(dy));
        free(x); free(w); free(x16); free(w16); free(yref); free(y);
    }

    /* Per-tensor quantiser, fp32 and bf16 sources, both formats: each of the
     * two tensors holds the format's largest finite magnitude once (+ in
     * tensor 0, - in tensor 1) and small integers elsewhere, so its scale
     * is amax / max = 1 exactly and every code is the exact encoding. */
    {
        const int64_t nq = 1000, bq = 2;
        float *xf = malloc(sizeof(float) * (size_t)(nq * bq));
        uint16_t *xb = malloc(2 * (size_t)(nq * bq));
        int8_t *xi = malloc((size_t)(nq * bq));
        uint8_t *qh = malloc((size_t)(nq * bq));
        if (!xf || !xb || !xi || !qh) {
            fprintf(stderr, "host allocation failed\n");
            return 3;
        }
        void *dxf, *dxb, *dq, *dsc;
        HIP_OK(hipMalloc(&dxf, sizeof(float) * (size_t)(nq * bq)));
        HIP_OK(hipMalloc(&dxb, 2 * (size_t)(nq * bq)));
        HIP_OK(hipMalloc(&dq, (size_t)(nq * bq)));
        HIP_OK(hipMalloc(&dsc, 2 * sizeof(float)));
        static const struct { const char *name; gemm355_fp8 fmt; float max; uint8_t max_code; } fmts[] = {
            {"e4m3", GEMM355_FP8_E4M3, 448.0f, 0x7E}, {"e5m2", GEMM355_FP8_E5M2, 57344.0f, 0x7B}};
        for (size_t f = 0; f < 2; ++f) {
            const int64_t at[2] = {17, nq + 911};   /* +max in tensor 0, -max in tensor 1 */
            for (int64_t e = 0; e < nq * bq; ++e) xi[e] = (int8_t)next_small();
            for (int64_t e = 0; e < nq * bq; ++e) xf[e] = (float)xi[e];
            xf[at[0]] = fmts[f].max;
            xf[at[1]] = -fmts[f].max;
            for (int64_t e = 0; e < nq * bq; ++e) {
                uint32_t u;
                memcpy(&u, &xf[e], 4);
                xb[e] = (uint16_t)(u >> 16);   /* exact: the values have few mantissa bits */
            }
            HIP_OK(hipMemcpy(dxf, xf, sizeof(float) * (size_t)(nq * bq), hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(dxb, xb, 2 * (size_t)(nq * bq), hipMemcpyHostToDevice));
            for (int src = 0; src < 2; ++src) {
                char name[48];
                snprintf(name, sizeof name, "quantize_%s_%s", src ? "bf16" : "f32", fmts[f].name);
                HIP_OK(hipMemsetAsync(dq, 0xAA, (size_t)(nq * bq), stream));
                HIP_OK(hipMemsetAsync(dsc, 0xFF, 2 * sizeof(float), stream));
                expect_status(name,
                              gemm355_quantize(src ? dxb : dxf, nq, bq, src ? GEMM355_SRC_BF16 : GEMM355_SRC_F32,
                                               fmts[f].fmt, dq, (float *)dsc, (void *)stream),
                              GEMM355_OK);
                HIP_OK(hipStreamSynchronize(stream));
                float sc[2];
                HIP_OK(hipMemcpy(sc, dsc, sizeof sc, hipMemcpyDeviceToHost));
                HIP_OK(hipMemcpy(qh, dq, (size_t)(nq * bq), hipMemcpyDeviceToHost));
                int64_t bad = 0;
                for (int64_t e = 0; e < nq * bq; ++e) {
                    uint8_t want = f == 0 ? e4m3_of_int(xi[e]) : e5m2_of_int(xi[e]);
                    if (e == at[0]) want = fmts[f].max_code;
                    if (e == at[1]) want = (uint8_t)(fmts[f].max_code | 0x80);
                    if (qh[e] != want) ++bad;
                }
                if (sc[0] != 1.0f || sc[1] != 1.0f || bad) {
                    fprintf(stderr, "%s: scales %.9g %.9g, %lld codes differ\n", name, (double)sc[0],
                            (double)sc[1], (long long)bad);
                    ++failures;
                } else {
                    printf("case %s ok (%lld codes)\n", name, (long long)(nq * bq));
                }
            }
        }
        HIP_OK(hipFree(dxf)); HIP_OK(hipFree(dxb)); HIP_OK(hipFree(dq)); HIP_OK(hipFree(dsc));
        free(xf); free(xb); free(xi); free(qh);
    }

    /* K == 0 writes zeros; a negative extent is an argument error. */
    HIP_OK(hipMemsetAsync(dC, 0xFF, c_bytes, stream));
    expect_status("gemm_k0", gemm355_gemm(M, N, 0, dA, 1, dB, 1, dC, N, GEMM355_BF16_F32,
                                         GEMM355_A_ROW_B_COL, 0, -1, (void *)stream),
                  GEMM355_OK);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(c, dC, c_bytes, hipMemcpyDeviceToHost));
    {
        int64_t bad = 0;
        for (int64_t e = 0; e < M * N; ++e)
            if (c[e] != 0.0f || signbit(c[e])) ++bad;
        if (bad) {
            fprintf(stderr, "gemm_k0: %lld elements not +0\n", (long long)bad);
            ++failures;
        } else {
            printf("case gemm_k0 ok\n");
        }
    }
    expect_status("gemm_negative_m",
                  gemm355_gemm(-1, N, K, dA, K, dB, K, dC, N, GEMM355_BF16_F32,
                               GEMM355_A_ROW_B_COL, 0, -1, (void *)stream),
                  GEMM355_EINVAL);
    if (!gemm355_status_string(GEMM355_EINVAL) || !*gemm355_status_string(GEMM355_EINVAL)) {
        fprintf(stderr, "status string empty\n");
        ++failures;
    }

    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(dA)); HIP_OK(hipFree(dB)); HIP_OK(hipFree(dC));
    HIP_OK(hipFree(dA8)); HIP_OK(hipFree(dB8)); HIP_OK(hipFree(dWs)); HIP_OK(hipFree(dScale));
    free(a); free(b); free(ref); free(a16); free(b16); free(a8); free(b8); free(c); free(c16);
    printf("%s\n", failures ? "FAILED" : "all cases ok");
    return failures ? 1 : 0;
}
