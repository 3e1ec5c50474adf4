/*
 * plan.h -- the host planner of libgemm355 (internal).
 */
#ifndef GEMM355_PLAN_H
#define GEMM355_PLAN_H

#include <stddef.h>
#include <stdint.h>

#include "../../include/gemm355.h"
#include "sched.h"

namespace g355 {

struct Plan {
    gemm355_plan_t pub;
    Sched s;
    int32_t esize;              /* input element bytes (2 bf16, 1 8-bit)    */
    int32_t out_esize;          /* 4 fp32, 2 bf16                           */
    int32_t Kb;                 /* K bytes seen by the main loop            */
    int32_t Kv;                 /* K bytes when an operand is read in place
                                   and K ends inside a 16-byte chunk; else 0 */
    int32_t pack_a, pack_b;
    /* operand views the main loop reads (bytes) */
    int64_t lda_b, ldb_b, stride_a_b, stride_b_b;
    /* workspace carve-up (byte offsets) */
    size_t ws_partial_off, ws_partial_bytes;
    size_t ws_pack_a_off, ws_pack_a_bytes;
    size_t ws_pack_b_off, ws_pack_b_bytes;
    /* MX: block scales regrouped K-tile-major, [batch][nK][rows] dwords */
    size_t ws_scale_a_off, ws_scale_a_bytes;
    size_t ws_scale_b_off, ws_scale_b_bytes;
    int32_t reduce_tiles;       /* blocks of the combine kernel (0: none)   */
    int32_t reduce_tail;        /* 1: combine the tail tiles                */
};

/* Element-type queries.  Dtypes come in pairs (fp32 C, bf16 C). */
constexpr int kNumDtypes = 20;
/* 8-bit inputs, with or without block scales */
inline bool dtype_fp8(gemm355_dtype d) { return d >= GEMM355_E4M3_F32 && d <= GEMM355_MXE4M3_E5M2_BF16; }
/* block-scaled 4-bit (E2M1) inputs */
inline bool dtype_fp4(gemm355_dtype d) { return d == GEMM355_MXFP4_F32 || d == GEMM355_MXFP4_BF16; }
/* block-scaled 6-bit (E2M3 or E3M2) inputs */
inline bool dtype_fp6(gemm355_dtype d) { return d >= GEMM355_MXFP6_E2M3_F32 && d <= GEMM355_MXFP6_E3M2_BF16; }
/* block-scaled inputs (8-, 6- or 4-bit) */
inline bool dtype_mx(gemm355_dtype d)
{
    return (d >= GEMM355_MXE4M3_F32 && d <= GEMM355_MXE4M3_E5M2_BF16) || dtype_fp4(d) || dtype_fp6(d);
}
/* bits per input element */
inline int32_t dtype_ebits(gemm355_dtype d)
{
    return dtype_fp4(d) ? 4 : dtype_fp6(d) ? 6 : dtype_fp8(d) ? 8 : 16;
}
inline bool dtype_out_bf16(gemm355_dtype d) { return ((int)d & 1) != 0; }
/* tile-table class: 0 bf16, 1 8-bit, 2 block-scaled 8-bit, 3 block-scaled
 * FP4, 4 block-scaled FP6 */
inline int32_t dtype_class_of(gemm355_dtype d)
{
    return dtype_fp6(d) ? 4 : dtype_fp4(d) ? 3 : dtype_mx(d) ? 2 : dtype_fp8(d) ? 1 : 0;
}
/* format codes of the MFMA operands relative to the element class: 0 E4M3
 * (FP6: E2M3), 1 E5M2 (FP6: E3M2) */
inline int32_t dtype_fmt_a(gemm355_dtype d)
{
    return (d == GEMM355_E5M2_F32 || d == GEMM355_E5M2_BF16 || d == GEMM355_MXE5M2_F32 ||
            d == GEMM355_MXE5M2_BF16 || d == GEMM355_MXFP6_E3M2_F32 || d == GEMM355_MXFP6_E3M2_BF16) ? 1 : 0;
}
inline int32_t dtype_fmt_b(gemm355_dtype d)
{
    return ((d >= GEMM355_E5M2_F32 && d <= GEMM355_E4M3_E5M2_BF16) ||
            (d >= GEMM355_MXE5M2_F32 && d <= GEMM355_MXE4M3_E5M2_BF16) || d == GEMM355_MXFP6_E3M2_F32 ||
            d == GEMM355_MXFP6_E3M2_BF16) ? 1 : 0;
}

/* A convolution planned as its implicit product (conv != null below): the
 * product's A is not a matrix in memory, so its pointer checks and repack
 * decisions come from here. */
struct ConvShape {
    int64_t N, H, W, C, R, S, P, Q;
    int64_t pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
};

/* Validate `a` and plan it for S compute units.  Never touches a device. */
gemm355_status make_plan(const gemm355_args &a, int32_t S, Plan &out, const ConvShape *conv = nullptr);

/* Null, alignment and overlap checks of the pointers in `a` (run on every
 * call, also when the plan comes from the cache). */
gemm355_status check_pointers(const gemm355_args &a, const ConvShape *conv = nullptr);

/* Exact rational -> nearest binary64 (ties to even). */
double rational_to_double(uint64_t num, uint64_t den);

/* Resident workgroups per compute unit for a tile-table entry. */
int32_t resident_workgroups(int32_t tile);

} /* namespace g355 */

#endif
