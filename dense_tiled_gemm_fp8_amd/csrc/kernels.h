/*
 * kernels.h -- launch interface between the host side of libgemm355 and its
 * gfx950 kernels.  Internal; not part of the C ABI.
 */
#ifndef GEMM355_KERNELS_H
#define GEMM355_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sched.h"

namespace g355 {

/* Main loop.  A and B are K-contiguous: row r of the A tile (column r of B)
 * starts lda (ldb) bytes after row r-1; both 16-byte aligned. */
struct GemmParams {
    const uint8_t *A;
    const uint8_t *B;
    void *C;
    float *ws;                    /* partial slots [slot][TM*TN] fp32      */
    int64_t lda, ldb;             /* bytes                                  */
    int64_t stride_a, stride_b;   /* bytes between batch entries            */
    int64_t ldc, stride_c;        /* elements of C                          */
    const float *scale_a, *scale_b;
    int32_t M, N, Kb;             /* Kb: K in bytes rounded up to 16        */
    int32_t Kv;                   /* K in bytes when rows are read in place
                                     and K is not a whole number of 16-byte
                                     chunks (the bytes of the last chunk past
                                     Kv are cleared in LDS); else 0          */
    int32_t out_bf16;
    int32_t c_vec;                /* 1: C rows can take 16-byte stores (base,
                                     row pitch and batch stride multiples
                                     of 16 bytes)                           */
    uint64_t *stamps;             /* per-unit start/end clock or null       */
    /* block scales (MX tiles), regrouped: dword [batch][K-tile][row] holds
     * a row's four E8M0 scales of one K-tile of 128 values */
    const uint8_t *bsa, *bsb;
    int64_t ktp_a, ktp_b;         /* bytes between K-tiles: 4 M, 4 N        */
    int64_t stride_bsa, stride_bsb;   /* bytes between batch entries        */
    /* convolution tiles: A row m = (n, p, q) gathers x[n][p*sh - ph + r*dh]
     * [q*sw - pw + s*dw][c] for K-tile (r, s, 64-channel block) */
    int32_t cv_H, cv_W, cv_C, cv_S, cv_P, cv_Q;
    int32_t cv_ph, cv_pw, cv_sh, cv_sw, cv_dh, cv_dw;
    Sched s;
};

struct ReduceParams {
    const float *ws;
    void *C;
    int64_t ldc, stride_c;
    const float *scale_a, *scale_b;
    int32_t M, N, TM, TN;
    int32_t out_bf16;
    int32_t tail;                 /* 1: reduce the tail tiles, 0: all tiles */
    int32_t sg_log2, chunks;      /* set by launch_reduce                   */
    Sched s;
};

struct PackParams {
    const void *src;
    uint8_t *dst;
    int64_t ld, stride;           /* source, elements                       */
    int64_t ldd_bytes;            /* destination row pitch, multiple of 16  */
    int64_t dst_stride_bytes;
    int32_t rows, K, batch, esize;
    int32_t kmajor;               /* 1: source K-contiguous                 */
};

/* Block scales [batch][rows][nK * 4] bytes -> [batch][nK][rows] dwords. */
struct ScalePackParams {
    const uint8_t *src;
    uint32_t *dst;
    int32_t rows, nK, batch;
};

/* Per-tensor quantisation to 8 bits (quant.hip). */
struct QuantParams {
    const void *x;                /* batch tensors of n elements            */
    uint8_t *q;                   /* codes, same layout                     */
    float *scale;                 /* [batch] dequantisation factors         */
    float *maxima;                /* scratch [batch * parts]                */
    int64_t n, batch;
    int32_t parts;                /* blocks per tensor (1 .. 4096)          */
    int32_t src;                  /* 0 fp32, 1 bf16                         */
    int32_t fmt;                  /* 0 E4M3, 1 E5M2                         */
    int32_t vec;                  /* 1: 8-element vector path (x 16-byte and
                                     q 8-byte aligned, n % 8 == 0)          */
};

hipError_t launch_quantize(const QuantParams &qp, hipStream_t stream);

/* fmt: operand formats of an 8-bit tile (0 E4M3 x E4M3, 1 E5M2 x E5M2,
 * 2 E4M3 x E5M2), with or without block scales; 0 for bf16 tiles */
hipError_t launch_gemm(int32_t tile, int32_t fmt, const GemmParams &p, hipStream_t stream);
const void *gemm_kernel_symbol(int32_t tile);
hipError_t launch_reduce(const ReduceParams &r, int32_t tiles, hipStream_t stream);
/* repack n (1 or 2) operands in one launch */
hipError_t launch_pack(const PackParams *pk, int n, hipStream_t stream);
hipError_t launch_pack_scales(const ScalePackParams &sp, hipStream_t stream);
hipError_t launch_zero(void *C, int32_t M, int32_t N, int64_t ldc, int64_t stride_c,
                       int32_t batch, int32_t esize, hipStream_t stream);

} /* namespace g355 */

#endif
