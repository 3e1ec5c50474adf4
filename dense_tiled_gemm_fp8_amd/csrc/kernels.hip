/*
 * kernels.hip -- gfx950 kernels of libgemm355.
 *
 *   gemm_tile_kernel  the MFMA main loop over work units (tile x K-range):
 *                     LDS-staged A/B tiles (and block scales) in a ring fed
 *                     by direct-to-LDS buffer loads, fp32 accumulators,
 *                     epilogue to C or to a split-K partial slot; also the
 *                     implicit-GEMM convolution (A gathered from images)
 *   reduce_kernel     the split-K combine: sums a tile's partial slots in
 *                     ascending slice order, scales, converts, stores C
 *   pack_kernel       repack A and/or B (one launch) into the K-contiguous,
 *                     16-byte aligned layout the main loop reads
 *                     (misaligned rows or K not a multiple of 16 bytes;
 *                     the three other operand layouts)
 *   pack_scales_kernel
 *                     regroup block scales (MX) K-tile-major
 *   zero_kernel       C = 0 for K == 0
 *
 * Source pages: "10. Tensor Cores, shapes, and tile alignment" (tile grid,
 * split-K, persistent loop) and "The Tensor Core" (stage A and B tiles in
 * on-chip memory once and feed many matrix-unit operations from them; low
 * precision inputs with a wide accumulator; the precision table's FP8 and
 * microscaled rows; convolutions as GEMM).
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.h"
#include "sched.h"
#include "tiles.h"

namespace g355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

/* Buffer loads whose offset is past num_records return zero (and write zero
 * to LDS for the direct-to-LDS form): rows beyond M or N and K-chunks beyond
 * K are read through offset kOOB. */
constexpr uint32_t kNumRecords = 0x7FFFFF00u;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base)
{
    /* word 3: 32-bit data format, the gfx9-family raw-buffer setting */
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)kNumRecords,
                                             0x00020000);
}

/* The four dwords of a raw buffer resource: 48-bit base, stride 0,
 * num_records, and the gfx9-family word 3 (32-bit data format). */
__device__ __forceinline__ i32x4 rsrc_words(const void *base)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF),
                 (int)kNumRecords, 0x00020000};
}

/* The lane's index in its wavefront, counted from the execution mask
 * (every lane active): needs no register held since the kernel's start. */
__device__ __forceinline__ int lane_id()
{
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

/* 32-bit LDS address of a __shared__ object. */
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

/* Compile-time unrolling: f(integral_constant<int, t>) for t = 0 .. N-1. */
template <int... T, class F>
__device__ __forceinline__ void unroll_seq(std::integer_sequence<int, T...>, F &&f)
{
    (f(std::integral_constant<int, T>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F &&f)
{
    unroll_seq(std::make_integer_sequence<int, N>{}, static_cast<F &&>(f));
}

/* One direct-to-LDS copy: each lane fetches 16 bytes at voffset from the
 * buffer and the wavefront writes them to LDS at lds_base + OFF .. + 1023
 * (lane l at + 16 l).  Issued as inline assembly so that the compiler neither
 * waits for it before unrelated LDS reads nor counts it (completion is
 * awaited explicitly), and so that the LDS address is formed in M0 right at
 * the load from one base register and an immediate. */
template <int OFF>
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t lds_base, uint32_t voffset)
{
    /* s_add writes SCC: declared clobbered, or the compiler could keep a
     * comparison result in SCC across this statement */
    int m0_out;
    asm volatile("s_add_u32 m0, %2, %4\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds"
                 : "={m0}"(m0_out)
                 : "v"(voffset), "s"(lds_base), "s"(rsrc), "n"(OFF)
                 : "memory", "scc");
    (void)m0_out;
}

/* One direct-to-LDS dword copy: lane l fetches 4 bytes at voffset and the
 * wavefront writes them to LDS at lds_addr + 4 l (256 bytes). */
__device__ __forceinline__ void dma4(const i32x4 &rsrc, uint32_t lds_addr_, uint32_t voffset)
{
    int m0_out;
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %1, %3, 0 offen lds"
                 : "={m0}"(m0_out)
                 : "v"(voffset), "s"(lds_addr_), "s"(rsrc)
                 : "memory");
    (void)m0_out;
}

/* All of this wave's direct-to-LDS copies have landed, then the workgroup
 * meets; the asm statements keep the compiler from moving LDS accesses
 * across. */
__device__ __forceinline__ void stage_barrier()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

/* Wait until at most N vector-memory operations of this wave are
 * outstanding (loads complete in issue order). */
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int V> using IC = std::integral_constant<int, V>;

template <bool FP8> struct FragType { typedef bf16x8 type; };
template <> struct FragType<true> { typedef i32x8 type; };
/* accumulator of one MI x MI MFMA block: MI * MI / 64 fp32 per lane */
template <int MI> struct AccType { typedef f32x16 type; };
template <> struct AccType<16> { typedef f32x4 type; };

__device__ __forceinline__ float unit_alpha(const GemmParams &p, int32_t batch)
{
    float a = 1.0f;
    if (p.scale_a) a *= p.scale_a[batch];
    if (p.scale_b) a *= p.scale_b[batch];
    return a;
}

/*
 * One workgroup of WGM x WGN wavefronts (4, 8 or 16) computes a TM x TN
 * tile; wavefront (wm, wn) owns a (TM/WGM) x (TN/WGN) block made of MI x MI
 * MFMA blocks (32 or 16).  With 8 wavefronts two share each SIMD, so one
 * issues MFMAs while the other waits on LDS or at the barrier.  A K-tile is
 * RB bytes of K per row (64 or 128: 32/64 bf16, 64/128 8-bit, 256 FP4 or 128
 * FP6 values); the LDS holds a ring of STAGES K-tiles.  Template knobs
 * beyond the shape: EL, the element class (bf16, 8-bit, block-scaled 8-, 4-
 * and 6-bit); SPREAD, the copy schedule (0-5, tiles.h); OP, the operation
 * (matrix product, or a convolution whose A rows are gathered from NHWC
 * images); FMT, the operand-format pair of the 8- and 6-bit classes.
 *
 * LDS layout of one stage of A (B alike): TM rows of RB bytes.  The LDS
 * serves a 128-bit read 16 lanes at a time from 64 four-byte banks, i.e. one
 * 256-byte line holding RPL = 256 / RB consecutive rows, so the 16 rows read
 * together by a fragment load must land on 16 different 16-byte slots of it.
 * Row r's 16-byte chunk c (of CPR = RB / 16) is stored at chunk position
 * c ^ ((r / RPL) % CPR): rows with different r % RPL use different parts of
 * the line, and the 16 / RPL = CPR rows sharing r % RPL get distinct chunks.
 * A direct-to-LDS load writes 1024 contiguous bytes per wavefront (lane l at
 * bytes 16 l .. 16 l + 15), i.e. 1024 / RB rows; lane l fetches row l / CPR
 * of its group and the logical chunk that belongs at position l % CPR.
 *
 * Pipeline: a ring of STAGES K-tiles.  Within a K-tile the fragments of MFMA
 * K-step ks+1 are read while the MFMAs of step ks run (fragments double
 * buffered in registers).  One barrier per K-tile, before its last step:
 * by then every wave has read all of this stage and the copy of the next
 * K-tile has landed; right after it, the copy of the K-tile STAGES ahead is
 * issued into the stage just freed, and the last step's MFMAs overlap the
 * reads of the next tile's first fragments.
 */
template <int TM, int TN, int EL, int MINB, int RB, int STAGES, int WGM, int WGN, int SPREAD, int OP, int MI, int FMT>
__global__ __launch_bounds__((WGM * WGN + (SPREAD == 3 ? 4 : 0)) * 64, MINB) void gemm_tile_kernel(GemmParams p)
{
    /* element class: 0 bf16, 1 8-bit, 2 8-bit with E8M0 block scales, 3 FP4
     * (E2M1, two per byte) with E8M0 block scales, 4 FP6 (E2M3 or E3M2, four
     * per three bytes) with E8M0 block scales.  FP8 marks the f8f6f4 matrix
     * instructions (classes 1-4). */
    constexpr bool FP8 = EL != 0, MX = EL >= 2, FP4 = EL == 3, FP6 = EL == 4;
    /* OP 1: convolution, A gathered from NHWC images (kernels.h) */
    constexpr bool CONV = OP == 1;
    /* operand formats (instruction format codes: 0 E4M3, 1 E5M2, 2 E2M3,
     * 3 E3M2, 4 E2M1): FMT 0 E4M3 x E4M3, 1 E5M2 x E5M2, 2 E4M3 x E5M2
     * (A x B), and for FP6 E2M3 / E3M2 in the same places; FP4 both 4 */
    constexpr int FA = FP4 ? 4 : (FP6 ? 2 : 0) + (FMT == 1 ? 1 : 0);
    constexpr int FB = FP4 ? 4 : (FP6 ? 2 : 0) + (FMT >= 1 ? 1 : 0);
    constexpr int NW = WGM * WGN, WN = WGN;
    /* SPREAD 3 (warp specialisation): four more wavefronts, one per SIMD,
     * issue every copy and run no MFMA; the NW MFMA wavefronts only read LDS.
     * CW wavefronts copy. */
    constexpr int NP = SPREAD == 3 ? 4 : 0, CW = SPREAD == 3 ? NP : NW;
    constexpr int WTM = TM / WGM, WTN = TN / WGN;
    constexpr int FM = WTM / MI, FN = WTN / MI;
    constexpr int CPR = RB / 16, RPL = 256 / RB, ROWS_PER_DMA = 1024 / RB;
    constexpr int A_BYTES = TM * RB, B_BYTES = TN * RB;
    /* MX: a K-tile of RB bytes holds RB * VPB values per row, i.e. SW
     * dwords of four E8M0 scales (one per 32-value block) per row of A and
     * B (SW = 1 for 8-bit, 2 for FP4).  A stage keeps them after the operand
     * rows as SW planes of TM + TN dwords (plane w: A's rows, then B's),
     * copied 64 rows per direct-to-LDS dword load, SC loads per wavefront. */
    constexpr int VPB = FP4 ? 2 : 1;
    /* values per row per K-tile, and the bytes they take in global memory
     * (FP6: 128 values in 96 bytes, staged in 128-byte LDS rows whose last
     * 32 bytes are not read) */
    constexpr int VPT = FP6 ? 128 : RB * VPB;
    constexpr int KTB = FP6 ? 96 : RB;
    constexpr int SW = MX ? VPT / 128 : 0;
    constexpr int SCA_OFF = A_BYTES + B_BYTES, SCB_OFF = SCA_OFF + TM * 4, SPLANE = (TM + TN) * 4;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SW * SPLANE;
    constexpr int SC = SW * (TM + TN) / 64 / NW;
    constexpr int A_LOADS = TM / ROWS_PER_DMA / CW, B_LOADS = TN / ROWS_PER_DMA / CW;
    constexpr int LOADS = A_LOADS + B_LOADS + SC;
    /* bytes of K per MFMA step: 32 x 32 blocks take 16 bf16, 64 E4M3 or 64
     * FP4 values, 16 x 16 blocks twice that; CPS 16-byte chunks */
    constexpr int KB_STEP = FP6 ? 64 : (FP8 && !FP4 ? 64 : 32) * (MI == 32 ? 1 : 2);
    constexpr int CPS = KB_STEP / 16;
    constexpr int KSTEPS = RB / KB_STEP;
    constexpr int ACC_N = MI * MI / 64;
    using Frag = typename FragType<FP8>::type;
    using Acc = typename AccType<MI>::type;
    static_assert(MI == 32 || MI == 16, "MFMA block");
    static_assert(RB % KB_STEP == 0, "K-tile holds whole MFMA steps");
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && FM >= 1 && FN >= 1 && KSTEPS >= 1, "tile");
    static_assert(STAGES >= 2 && (STAGES - 1) * LOADS < 64, "ring depth");
    static_assert(SPREAD != 1 || STAGES >= 3, "spread copies need a third stage");
    /* SPREAD 2: fragments read two K-steps ahead, one barrier per K-tile
     * before its second-to-last step, copies over its last two steps */
    static_assert(SPREAD != 2 || (KSTEPS == 4 && STAGES == 2 && LOADS % 2 == 0), "two-step prefetch schedule");
    static_assert(SPREAD != 3 || STAGES >= 3, "producer wavefronts run two K-tiles ahead");
    static_assert(!CONV || (!FP8 && SPREAD == 0 && RB == 128), "convolution: bf16, 64-channel K-tiles copied in one step");
    static_assert(!FP6 || (RB == 128 && MI == 32), "FP6: 128-value K-tiles in 128-byte rows, 32 x 32 blocks");
    /* SPREAD 4: copies as in schedule 0; A's fragments single-buffered, each
     * row's next fragment read into its own registers right after the row's
     * last MFMA (B's double-buffered), so the fragments take FM fewer
     * registers */
    static_assert(SPREAD != 4 || (!FP8 && !CONV && FM + FN - 1 <= 15), "in-place A fragments: bf16 matrix products");
    static_assert(A_LOADS * CW * ROWS_PER_DMA == TM && B_LOADS * CW * ROWS_PER_DMA == TN, "whole copies");
    static_assert(!MX || (SPREAD == 0 && RB == 128 && MI == 32 && TM % 64 == 0 && SC * 64 * NW == SW * (TM + TN)),
                  "block scales: whole dwords per row and K-tile, whole 64-row copies per wavefront");
    constexpr int NB = SPREAD == 2 ? 4 : 2;     /* fragment buffers */
    /* SPREAD 5: schedule 0 with B's ring one stage deeper than A's, the
     * spare LDS of a two-stage 256 x 256 tile.  A's stages sit at s A_BYTES,
     * B's at B_BASE + t B_BYTES.  B's copies of K-tile kt+2 then go in the
     * first K-step of K-tile kt (B's stage of kt-1 is free since the barrier
     * in kt-1's middle) and A's in its last step, as in schedule 0: half the
     * copies per step, each with at least a K-tile to land.  Otherwise B
     * follows A in each stage. */
    static_assert(SPREAD != 5 || (!MX && !FP6 && !CONV && STAGES == 2 && KSTEPS == 2),
                  "deeper B ring: two stages of two K-steps");
    /* SPREAD 6: schedule 5's rings and copies in a ping-pong loop, the
     * alternative to producer wavefronts (schedule 3) that keeps every
     * wavefront an MFMA wavefront (page "10. Tensor Cores, shapes, and tile
     * alignment", section "Warp specialization is not ordinary occupancy",
     * splits copies and MMA between warps).  The wavefronts of block row 1
     * run one phase behind those of block row 0, and each wavefront
     * alternates a phase of MFMAs only with a phase of fragment reads and
     * copies, so each SIMD (which holds one wavefront of each block row)
     * has one wavefront issuing MFMAs while the other feeds the next step.
     * Four barriers per K-tile keep the phases aligned. */
    static_assert(SPREAD != 6 || (!MX && !FP6 && !CONV && STAGES == 2 && KSTEPS == 2 && WGM == 2 && WGN == 4),
                  "ping-pong: two block rows of four wavefronts, two stages of two K-steps");
    constexpr bool DEEP_B = SPREAD == 5 || SPREAD == 6;
    constexpr int BST = DEEP_B ? STAGES + 1 : STAGES;
    constexpr int B_BASE = DEEP_B ? STAGES * A_BYTES : A_BYTES;
    constexpr int LDS_BYTES = DEEP_B ? STAGES * A_BYTES + BST * B_BYTES : STAGES * STAGE_BYTES;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    /* this wavefront's index among the CW copying ones (SPREAD 3: the
     * producers NW .. NW+3) */
    const bool producer = SPREAD == 3 && wave >= NW;
    const int cw = SPREAD == 3 ? wave - NW : wave;
    constexpr bool TWO = (4 * CW) % CPR != 0;
    const uint32_t smem_base = lds_addr(smem);

    int32_t first = blockIdx.x;
    if (p.s.xcd_remap) first = xcd_remap(first, p.s.grid);

    for (int32_t u = first; u < p.s.units; u += p.s.grid) {
        /* Lane-derived addresses are formed per unit from a lane index the
         * compiler cannot see through: otherwise it hoists them out of the
         * persistent loop and holds (or spills) them across every unit. */
        int lane_u = lane_id();
        asm volatile("" : "+v"(lane_u));
        const int drow = lane_u / CPR;
        /* Copy d of a stage part is copy group d * CW + cw; the lane's row
         * is r = (d * CW + cw) * ROWS_PER_DMA + drow, and ROWS_PER_DMA =
         * 4 RPL, so (r / RPL) % CPR = (4 (d CW + cw) + drow / RPL) % CPR:
         * with 4 CW a multiple of CPR it is the same for every d, otherwise
         * (CPR = 8, CW odd) it alternates with the parity of d.
         * lchunk[d & 1] is the logical chunk the lane fetches. */
        int lchunk[2];
        lchunk[0] = (lane_u % CPR) ^ ((4 * cw + drow / RPL) % CPR);
        lchunk[1] = (lane_u % CPR) ^ ((4 * (CW + cw) + drow / RPL) % CPR);
        /* fragment lanes: lane l reads row l % MI of the block and K-chunk
         * group l / MI of the step */
        const int frow = lane_u % MI, hi = lane_u / MI, sw = (frow / RPL) % CPR;
        uint64_t stamp0 = 0, clk0 = 0;
        if (p.stamps) {
            stamp0 = __builtin_amdgcn_s_memrealtime();
            clk0 = __builtin_amdgcn_s_memtime();
        }
        const Unit un = decode_unit(p.s, u);
        const int32_t m0 = un.tile_m * TM, n0 = un.tile_n * TN;
        /* convolution: A's offsets are taken from the first image */
        const i32x4 ra = rsrc_words(CONV ? p.A : p.A + (int64_t)un.batch * p.stride_a + (int64_t)m0 * p.lda);
        const i32x4 rb = rsrc_words(p.B + (int64_t)un.batch * p.stride_b + (int64_t)n0 * p.ldb);

        uint32_t aoff[A_LOADS], boff[B_LOADS];
        /* convolution: the lane's output pixel (n, p, q) per A copy, as the
         * window's top-left input position (ch0, cw0) and the byte offset of
         * that position plus the lane's chunk (negative while the window
         * starts in the padding; only in-image taps are read) */
        int32_t ch0[CONV ? A_LOADS : 1], cw0[CONV ? A_LOADS : 1];
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int r = (i * CW + cw) * ROWS_PER_DMA + drow;
            if constexpr (CONV) {
                const int32_t m = m0 + r, pq_n = p.cv_P * p.cv_Q;
                if (m < p.M) {
                    const int32_t n = m / pq_n, pq = m - n * pq_n, pp = pq / p.cv_Q, qq = pq - pp * p.cv_Q;
                    ch0[i] = pp * p.cv_sh - p.cv_ph;
                    cw0[i] = qq * p.cv_sw - p.cv_pw;
                    aoff[i] = (uint32_t)(((n * p.cv_H + ch0[i]) * p.cv_W + cw0[i]) * p.cv_C * 2 +
                                         lchunk[TWO ? i & 1 : 0] * 16);
                } else {
                    ch0[i] = -(1 << 29);
                    cw0[i] = 0;
                    aoff[i] = 0;
                }
            } else {
                aoff[i] = (m0 + r < p.M) ? (uint32_t)(r * p.lda + lchunk[TWO ? i & 1 : 0] * 16) : kOOB;
            }
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int r = (i * CW + cw) * ROWS_PER_DMA + drow;
            boff[i] = (n0 + r < p.N) ? (uint32_t)(r * p.ldb + lchunk[TWO ? i & 1 : 0] * 16) : kOOB;
        }
        /* MX: scale copy q of this wavefront moves the dwords of 64 rows,
         * group g = q NW + wave: rows 64 g .. 64 g + 63 of A if g < TM / 64,
         * else rows 64 (g - TM / 64) .. of B; lane l takes the group's row l
         * (the scales are regrouped K-tile-major, so the 64 dwords are
         * contiguous).  Rows past M or N read zero (scale 2^-127 on zero
         * operands). */
        i32x4 srs[SC > 0 ? SC : 1];
        uint32_t soff[SC > 0 ? SC : 1], sdst[SC > 0 ? SC : 1], stp[SC > 0 ? SC : 1];
        if constexpr (MX) {
            const uint8_t *sa0 = p.bsa + (int64_t)un.batch * p.stride_bsa + (int64_t)m0 * 4;
            const uint8_t *sb0 = p.bsb + (int64_t)un.batch * p.stride_bsb + (int64_t)n0 * 4;
            unroll<SC>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                /* group g: plane w = g / G1, then A's or B's 64-row group */
                constexpr int G1 = (TM + TN) / 64;
                const int g = q * NW + wave;
                const int w = g / G1, g1 = g % G1;
                const bool in_a = g1 < TM / 64;
                const int r = (in_a ? g1 : g1 - TM / 64) * 64 + lane_u;
                const uint32_t plane = (uint32_t)(in_a ? p.ktp_a : p.ktp_b);
                srs[q] = rsrc_words(in_a ? sa0 : sb0);
                soff[q] = (in_a ? m0 + r < p.M : n0 + r < p.N) ? (uint32_t)(r * 4) + w * plane : kOOB;
                sdst[q] = (uint32_t)(SCA_OFF + g * 256);
                stp[q] = SW * plane;
            });
        }

        /* Copy of K-tile kt into the stage at LDS byte offset so: chunks past
         * K, and every chunk of a K-tile past the unit's range, read zero, so
         * copies can be issued unconditionally (a masked copy only rewrites
         * LDS rows this wave owns and nobody reads before they are copied
         * again). */
        /* per parity class of the copy index (one class unless TWO) */
        struct KV {
            bool v[2];
            bool tile;   /* the K-tile is in the unit's range (block scales:
                            whole dwords, whatever the lane's chunk) */
        };
        /* iteration i of the unit's loop works on K-tile kt_begin + i */
        const int32_t nkt = un.kt_end - un.kt_begin;
        auto ktile = [&](int32_t i) __attribute__((always_inline)) { return un.kt_begin + i; };
        /* copies of iteration i; iterations past the range read zero */
        /* chunks of a row that belong to the K-tile (FP6: 6 of the 8; the
         * last two would be the next K-tile's bytes and are not read) */
        constexpr int KCH = KTB / 16;
        auto kvalid = [&](int32_t i) __attribute__((always_inline)) {
            const uint32_t kb = (uint32_t)ktile(i) * KTB;
            KV k;
            k.v[0] = ((int32_t)(kb + lchunk[0] * 16) < p.Kb) && (i < nkt) && lchunk[0] < KCH;
            k.v[1] = TWO ? ((int32_t)(kb + lchunk[1] * 16) < p.Kb) && (i < nkt) && lchunk[1] < KCH : k.v[0];
            k.tile = ((int32_t)kb < p.Kb) && (i < nkt);
            return k;
        };
        /* convolution: filter tap and channel block of the next K-tile to
         * be copied (K-tiles are copied once each, in order); ctap holds the
         * one whose copies are being issued */
        struct Tap {
            int32_t rd, sd;   /* r dh, s dw */
            uint32_t off;     /* byte offset of the tap and channel block */
        };
        int32_t t_cb = 0, t_s = 0, t_r = 0;
        const int32_t n_cb = CONV ? p.cv_C / 64 : 1;
        if constexpr (CONV) {
            const int32_t rs = un.kt_begin / n_cb;
            t_cb = un.kt_begin - rs * n_cb;
            t_r = rs / p.cv_S;
            t_s = rs - t_r * p.cv_S;
        }
        Tap ctap{0, 0, 0u};
        auto next_tap = [&]() __attribute__((always_inline)) {
            if constexpr (CONV) {
                ctap.rd = t_r * p.cv_dh;
                ctap.sd = t_s * p.cv_dw;
                ctap.off = (uint32_t)((ctap.rd * p.cv_W + ctap.sd) * p.cv_C * 2 + t_cb * 128);
                if (++t_cb == n_cb) {
                    t_cb = 0;
                    if (++t_s == p.cv_S) {
                        t_s = 0;
                        ++t_r;
                    }
                }
            }
        };
        /* copy d of a K-tile into the stage whose A part is at byte so and B
         * part at byte sob */
        auto dma = [&](auto dc, uint32_t so, uint32_t sob, uint32_t kb, const KV &kv) __attribute__((always_inline)) {
            constexpr int d = decltype(dc)::value;
            constexpr int di = d < A_LOADS ? d : d - A_LOADS;
            const bool ok = kv.v[TWO ? di & 1 : 0];
            const uint32_t dst = smem_base + so + cw * 1024;
            if constexpr (d < A_LOADS && CONV) {
                /* only taps inside the image are read; the rest are zero */
                const bool in = ok && (uint32_t)(ch0[d] + ctap.rd) < (uint32_t)p.cv_H &&
                                (uint32_t)(cw0[d] + ctap.sd) < (uint32_t)p.cv_W;
                dma16<d * CW * 1024>(ra, dst, in ? aoff[d] + ctap.off : kOOB);
            } else if constexpr (d < A_LOADS) {
                dma16<d * CW * 1024>(ra, dst, ok ? aoff[d] + kb : kOOB);
            } else if constexpr (d < A_LOADS + B_LOADS) {
                dma16<(d - A_LOADS) * CW * 1024>(rb, smem_base + sob + cw * 1024, ok ? boff[di] + kb : kOOB);
            } else {
                /* K-tile kb / KTB of the regrouped scales */
                constexpr int q = d - A_LOADS - B_LOADS;
                dma4(srs[q], smem_base + so + sdst[q], kv.tile ? soff[q] + (kb / KTB) * stp[q] : kOOB);
            }
        };
        /* Rows read in place whose K ends inside a 16-byte chunk: the chunk
         * also brought the next bytes of memory (the next row's first
         * elements, or whatever follows the operand).  Once the copies of
         * iteration i (in the stage at so) have landed, each lane that
         * fetched such a chunk clears its bytes past K in LDS, before the
         * barrier that shows the stage to the other waves.  Only copy
         * schedules 0, 4 and 5 (tile and prologue waits below) take this
         * path. */
        auto zero_tail = [&](uint32_t so, uint32_t sob, int32_t i) __attribute__((always_inline)) {
            if constexpr (!FP6 && !MX && !CONV && (SPREAD == 0 || SPREAD == 4 || DEEP_B)) {
                const int32_t kb = ktile(i) * KTB;
                if (p.Kv > 0 && i < nkt && kb + KTB > p.Kv) {
                    unroll<A_LOADS + B_LOADS>([&](auto dc) __attribute__((always_inline)) {
                        constexpr int d = decltype(dc)::value;
                        constexpr int di = d < A_LOADS ? d : d - A_LOADS;
                        const int32_t v = p.Kv - (kb + lchunk[TWO ? di & 1 : 0] * 16);
                        if (v > 0 && v < 16) {
                            const uint32_t doff = d < A_LOADS ? so + d * CW * 1024 : sob + (d - A_LOADS) * CW * 1024;
                            i32x4 *c = (i32x4 *)(smem + doff + cw * 1024 + lane_u * 16);
                            i32x4 w = *c;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int32_t vb = v - 4 * j;
                                const uint32_t keep = vb >= 4 ? 0xFFFFFFFFu : (vb <= 0 ? 0u : (1u << (8 * vb)) - 1u);
                                w[j] = (int)((uint32_t)w[j] & keep);
                            }
                            *c = w;
                        }
                    });
                    /* the cleared bytes are in LDS before the barrier */
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            }
        };
        auto copy_tile = [&](uint32_t so, uint32_t sob, int32_t i) __attribute__((always_inline)) {
            const KV kv = kvalid(i);
            const uint32_t kb = (uint32_t)ktile(i) * KTB;
            next_tap();
            unroll<LOADS>([&](auto dc) __attribute__((always_inline)) { dma(dc, so, sob, kb, kv); });
        };

        /* Fragment of MFMA K-step ks for block blk of this wave, from the
         * operand rows starting at `rows` (A or B part of a stage). */
        auto frag = [&](const uint8_t *rows, int ks, int blk) __attribute__((always_inline)) -> Frag {
            const uint8_t *row = rows + (blk * MI + frow) * RB;
            if constexpr (!FP8) {
                return *(const bf16x8 *)(row + (((CPS * ks + hi) ^ sw) * 16));
            } else if constexpr (FP6) {
                /* 32 values (one block, 24 bytes) per lane group: bytes
                 * 48 ks + 24 hi .. + 23 of the row, i.e. chunks 3 ks (all)
                 * and 3 ks + 1 (first half) for lane group 0, chunks 3 ks + 1
                 * (second half) and 3 ks + 2 (all) for lane group 1.  Two
                 * whole-chunk reads per lane (its own chunk and the shared
                 * middle one) keep the 8-row read groups of the swizzle free
                 * of bank conflicts, which 8-byte reads of 16 rows are not. */
                const i32x4 f = *(const i32x4 *)(row + (((3 * ks + 2 * hi) ^ sw) << 4));
                const i32x4 m = *(const i32x4 *)(row + (((3 * ks + 1) ^ sw) << 4));
                return hi ? i32x8{m[2], m[3], f[0], f[1], f[2], f[3], 0, 0}
                          : i32x8{f[0], f[1], f[2], f[3], m[0], m[1], 0, 0};
            } else if constexpr (FP4) {
                /* 32 values (one block) per lane in the low four dwords */
                const i32x4 v = *(const i32x4 *)(row + (((CPS * ks + hi) ^ sw) * 16));
                return i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
            } else {
                /* the instruction takes K in 16-byte quarters: lane group
                 * hi's first and second halves are quarters hi and 2 + hi of
                 * the step, and the block scale of lane group hi covers
                 * quarters 2 hi and 2 hi + 1 (the first halves of both
                 * groups, or the second halves).  Without block scales any
                 * consistent order of A's and B's chunks gives the same
                 * products; with them, reading chunks hi and 2 + hi puts
                 * the step's 32-value block hi under scale byte hi. */
                const int c0 = MX ? CPS * ks + hi : CPS * ks + 2 * hi;
                const int c1 = MX ? CPS * ks + 2 + hi : CPS * ks + 2 * hi + 1;
                const i32x4 lo = *(const i32x4 *)(row + ((c0 ^ sw) * 16));
                const i32x4 up = *(const i32x4 *)(row + ((c1 ^ sw) * 16));
                return i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
            }
        };

        /* MX: the scale dwords of this wavefront's MFMA rows for the next
         * K-tile (read from LDS in the last K-step, after the next tile's
         * first fragments) and for the current one, shifted so that byte 0
         * holds the lane's first block (the instruction takes its scale
         * from byte 0) */
        constexpr int NSW = MX ? SW : 1;
        uint32_t nsa[NSW][MX ? FM : 1], nsb[NSW][MX ? FN : 1], csa[NSW][MX ? FM : 1], csb[NSW][MX ? FN : 1];
        auto read_scales = [&](const uint8_t *st) __attribute__((always_inline)) {
            if constexpr (MX) {
#pragma unroll
                for (int w = 0; w < SW; ++w) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        nsa[w][i] = *(const uint32_t *)(st + w * SPLANE + SCA_OFF + (wm * WTM + i * MI + frow) * 4);
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        nsb[w][j] = *(const uint32_t *)(st + w * SPLANE + SCB_OFF + (wn * WTN + j * MI + frow) * 4);
                }
            }
        };
        auto take_scales = [&]() __attribute__((always_inline)) {
            if constexpr (MX) {
#pragma unroll
                for (int w = 0; w < SW; ++w) {
#pragma unroll
                    for (int i = 0; i < FM; ++i) csa[w][i] = nsa[w][i] >> (8 * hi);
#pragma unroll
                    for (int j = 0; j < FN; ++j) csb[w][j] = nsb[w][j] >> (8 * hi);
                }
            }
        };

        Acc acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = Acc{};

        /* Fragments double-buffered by K-step parity (SPREAD 2: one buffer
         * per K-step of the tile). */
        Frag fa[NB][FM], fb[NB][FN];

        /* One K-step: the FM x FN MFMAs on buffer CUR, interleaved slot by
         * slot with the fragment reads of step nks of the stage whose A and
         * B parts are at `ns` and `nbs` into buffer CUR^1 and with copies
         * D0 .. D0+DN-1 of the K-tile at byte kb into the stage whose parts
         * are at byte offsets dso and dsob, copy j at slot j * SLOTS / DN.
         * The scheduling barriers keep this interleave as written. */
        auto step = [&](auto cur_c, auto d0_c, auto dn_c, const uint8_t *ns, const uint8_t *nbs, int nks,
                        uint32_t dso, uint32_t dsob, uint32_t kb, const KV &kv, auto ks_c)
                        __attribute__((always_inline)) {
            constexpr int CUR = decltype(cur_c)::value;
            /* K-step of the tile the MFMAs work on (MX: its blocks are bytes
             * 8 KS KB_STEP / 32 + 8 hi of the scale dwords) */
            constexpr int KS = decltype(ks_c)::value;
            /* buffer the reads of this step fill */
            constexpr int TGT = SPREAD == 2 ? (CUR + 2) % NB : CUR ^ 1;
            constexpr int D0 = decltype(d0_c)::value, DN = decltype(dn_c)::value;
            constexpr int NM = FM * FN, NR = FM + FN;
            /* MX: the last K-step, which reads the next tile's first
             * fragments, also reads its FM + FN scale dwords, after them */
            constexpr bool SCALES = MX && KS == KSTEPS - 1;
            constexpr int NS = SW * (FM + FN);        /* scale dwords read in that step */
            /* SPREAD 2 puts the copies after the reads: NR + DN slots at least */
            constexpr int SLOTS0 = SPREAD == 2 ? (NM > NR + DN ? NM : NR + DN)
                                               : NM > (NR > DN ? NR : DN) ? NM : (NR > DN ? NR : DN);
            constexpr int SLOTS = SCALES && SLOTS0 < NR + NS ? NR + NS : SLOTS0;
            if constexpr (SPREAD == 2) {
                /* this step's fragments (read two steps ago) are in; the NR
                 * reads of the previous step may still be outstanding */
                asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NR < 15 ? NR : 15) : "memory");
            } else if constexpr (SPREAD == 4) {
                /* waits per row, below */
            } else {
                /* this step's fragments (read during the previous step) are
                 * in; nothing else is outstanding on the LDS counter here */
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            /* A's fragment buffer (SPREAD 4: one) */
            constexpr int CA = SPREAD == 4 ? 0 : CUR;
            unroll<SLOTS>([&](auto tc) __attribute__((always_inline)) {
                constexpr int t = decltype(tc)::value;
                if constexpr (SPREAD == 4 && t < NM && t % FN == 0) {
                    /* row t / FN's A fragment (read after that row of the
                     * previous step) is in: newer reads are the later rows'
                     * (FM - 1 - row), and this step's B reads and earlier
                     * rows' A reads (FN + row) once row 0 has issued them */
                    constexpr int ROW = t / FN, NEWER = ROW == 0 ? FM - 1 : FM + FN - 1;
                    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NEWER) : "memory");
                }
                if constexpr (t < NM) {
                    constexpr int i = t / FN, j = t % FN;
                    if constexpr (!FP8 && MI == 32)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CA][i], fb[CUR][j], acc[i][j], 0, 0, 0);
                    else if constexpr (!FP8)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[CA][i], fb[CUR][j], acc[i][j], 0, 0, 0);
                    else if constexpr (MX) {
                        /* the step's first block: its plane and byte */
                        constexpr int B0 = KS * (FP6 ? 2 : KB_STEP * VPB / 32), DW = B0 / 4, SH = 8 * (B0 % 4);
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa[CUR][i], fb[CUR][j], acc[i][j], FA, FB, 0, (int)(csa[DW][i] >> SH), 0,
                            (int)(csb[DW][j] >> SH));
                    }
                    /* format fields FA / FB of the A and B operands; zero
                     * scales select the unscaled instruction */
                    else if constexpr (MI == 32)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa[CUR][i], fb[CUR][j], acc[i][j], FA, FB, 0, 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            fa[CUR][i], fb[CUR][j], acc[i][j], FA, FB, 0, 0, 0, 0);
                }
                if constexpr (SPREAD == 4) {
                    /* B's next fragments during row 0; row i's next A
                     * fragment right after its last MFMA */
                    if constexpr (t < FN)
                        fb[TGT][t] = frag(nbs + wn * WTN * RB, nks, t);
                    if constexpr (t < NM && t % FN == FN - 1)
                        fa[0][t / FN] = frag(ns + wm * WTM * RB, nks, t / FN);
                } else if constexpr (t < FM)
                    fa[TGT][t] = frag(ns + wm * WTM * RB, nks, t);
                else if constexpr (t < NR)
                    fb[TGT][t - FM] = frag(nbs + wn * WTN * RB, nks, t - FM);
                else if constexpr (SCALES && t < NR + NS) {
                    /* dword u of the step's scale reads: plane u / (FM + FN) */
                    constexpr int u = t - NR, w = u / (FM + FN), v = u % (FM + FN);
                    if constexpr (v < FM)
                        nsa[w][v] = *(const uint32_t *)(ns + w * SPLANE + SCA_OFF + (wm * WTM + v * MI + frow) * 4);
                    else
                        nsb[w][v - FM] =
                            *(const uint32_t *)(ns + w * SPLANE + SCB_OFF + (wn * WTN + (v - FM) * MI + frow) * 4);
                }
                if constexpr (DN > 0 && SPREAD == 2) {
                    /* copies after the fragment reads, spread over the rest
                     * of the step */
                    constexpr int FREE = SLOTS - NR;
                    unroll<DN>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        if constexpr (NR + (j * FREE) / DN == t)
                            dma(std::integral_constant<int, D0 + j>{}, dso, dsob, kb, kv);
                    });
                } else if constexpr (DN > 0) {
                    constexpr int j = (t * DN + SLOTS - 1) / SLOTS;
                    if constexpr (j < DN && (j * SLOTS) / DN == t)
                        dma(std::integral_constant<int, D0 + j>{}, dso, dsob, kb, kv);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        /* One K-tile in the stage at byte offset so; nso is the next tile's
         * stage.  Fragment buffers alternate by K-step; with an odd number of
         * K-steps per tile the parity P of the tile shifts them.
         *
         * Copies: without SPREAD, K-tile kt+STAGES goes into this tile's own
         * stage during its last step (the stage is free once the barrier
         * shows every wave has read it).  With SPREAD, K-tile kt+STAGES-1
         * goes into the stage dso of tile kt-1 (free since the previous
         * barrier), its copies spread evenly over all K-steps, so the copy
         * queue never receives a whole K-tile at once. */
        /* SPREAD 2, one K-tile of 4 K-steps in stage so (nso: the next
         * tile's stage).  Step ks runs its MFMAs on buffer ks and reads the
         * fragments of step ks+2 into buffer (ks+2) % 4: steps 0 and 1 read
         * steps 2 and 3 of this stage, steps 2 and 3 read steps 0 and 1 of
         * the next.  Before step 2 every wave has finished reading this stage
         * and the next stage has landed: one barrier, then the copies of
         * K-tile kt+2 into this stage over steps 2 and 3. */
        auto tile2 = [&](uint32_t so, uint32_t nso, int32_t kt) __attribute__((always_inline)) {
            const uint8_t *cs = smem + so;
            const KV kv0{{false, false}, false};
            step(IC<0>{}, IC<0>{}, IC<0>{}, cs, cs + A_BYTES, 2, so, so + A_BYTES, 0u, kv0, IC<0>{});
            step(IC<1>{}, IC<0>{}, IC<0>{}, cs, cs + A_BYTES, 3, so, so + A_BYTES, 0u, kv0, IC<1>{});
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            /* tile kt+1 landed (its copies are the only ones outstanding) */
            wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const KV kv = kvalid(kt + 2);
            const uint32_t kb = (uint32_t)ktile(kt + 2) * KTB;
            step(IC<2>{}, IC<0>{}, IC<LOADS / 2>{}, smem + nso, smem + nso + A_BYTES, 0, so, so + A_BYTES, kb, kv,
                 IC<2>{});
            step(IC<3>{}, IC<LOADS / 2>{}, IC<LOADS / 2>{}, smem + nso, smem + nso + A_BYTES, 1, so, so + A_BYTES, kb,
                 kv, IC<3>{});
        };

        auto tile = [&](auto pc, uint32_t so, uint32_t nso, uint32_t dso, int32_t kt) __attribute__((always_inline)) {
            /* kt: the iteration index within the unit */
            constexpr int P = decltype(pc)::value;
            constexpr bool SP1 = SPREAD == 1;
            constexpr int LPRE = SP1 ? (KSTEPS - 1) * LOADS / KSTEPS : 0;
            const uint8_t *cs = smem + so;
            KV kv{{false, false}, false};
            uint32_t kb = 0;
            take_scales();
            if constexpr (SP1) {
                kv = kvalid(kt + STAGES - 1);
                kb = (uint32_t)ktile(kt + STAGES - 1) * KTB;
            }
            unroll<KSTEPS - 1>([&](auto kc) __attribute__((always_inline)) {
                constexpr int ks = decltype(kc)::value;
                constexpr int D0 = SP1 ? ks * LOADS / KSTEPS : 0;
                constexpr int DN = SP1 ? (ks + 1) * LOADS / KSTEPS - D0 : 0;
                step(IC<(ks + P) & 1>{}, IC<D0>{}, IC<DN>{}, cs, cs + A_BYTES, ks + 1, dso, dso + A_BYTES, kb, kv,
                     IC<ks>{});
            });
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            /* tile kt+1 landed: later copies may still be in flight (SPREAD
             * 3: the producers have waited for it before this barrier) */
            if constexpr (SPREAD != 3)
                wait_vmcnt<SP1 ? (STAGES - 3) * LOADS + LPRE : (STAGES - 2) * LOADS>();
            /* K-tile kt+1 (stage nso) has landed */
            zero_tail(nso, nso + A_BYTES, kt + 1);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if constexpr (SP1) {
                step(IC<(KSTEPS - 1 + P) & 1>{}, IC<LPRE>{}, IC<LOADS - LPRE>{}, smem + nso, smem + nso + A_BYTES, 0, dso,
                     dso + A_BYTES, kb, kv, IC<KSTEPS - 1>{});
            } else if constexpr (SPREAD == 3) {
                step(IC<(KSTEPS - 1 + P) & 1>{}, IC<0>{}, IC<0>{}, smem + nso, smem + nso + A_BYTES, 0, so,
                     so + A_BYTES, 0u, kv, IC<KSTEPS - 1>{});
            } else {
                kv = kvalid(kt + STAGES);
                kb = (uint32_t)ktile(kt + STAGES) * KTB;
                next_tap();
                step(IC<(KSTEPS - 1 + P) & 1>{}, IC<0>{}, IC<LOADS>{}, smem + nso, smem + nso + A_BYTES, 0, so,
                     so + A_BYTES, kb, kv, IC<KSTEPS - 1>{});
            }
        };
        auto next_stage = [](uint32_t so) __attribute__((always_inline)) {
            return so + STAGE_BYTES == STAGES * STAGE_BYTES ? 0u : so + STAGE_BYTES;
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;

        if (producer && nkt > 0) {
            /* SPREAD 3 producer: K-tiles 0 .. STAGES-2 first; then, between
             * the MFMA wavefronts' barriers kt-1 and kt, K-tile kt+STAGES-1
             * into the stage of K-tile kt-1 (read by every wavefront before
             * barrier kt-1), and barrier kt only once K-tile kt+1 has
             * landed.  Same barrier count as the MFMA wavefronts. */
            unroll<STAGES - 1>([&](auto sc) __attribute__((always_inline)) {
                constexpr int st = decltype(sc)::value;
                copy_tile(st * STAGE_BYTES, st * STAGE_BYTES + A_BYTES, st);
            });
            wait_vmcnt<(STAGES - 2) * LOADS>();
            __builtin_amdgcn_s_barrier();
            uint32_t dso = (STAGES - 1) * STAGE_BYTES;
            for (int32_t kt = 0; kt < nkt; ++kt) {
                copy_tile(dso, dso + A_BYTES, kt + STAGES - 1);
                wait_vmcnt<(STAGES - 2) * LOADS>();
                __builtin_amdgcn_s_barrier();
                dso = next_stage(dso);
            }
        } else if (nkt > 0) {
            int32_t kt = 0;
            /* prologue: the first PRE K-tiles of the unit (SPREAD 3: issued
             * by the producers) */
            if constexpr (DEEP_B) {
                /* K-tiles 0 and 1: A in stages 0 and 1, B in B's stages 0 and 1 */
                copy_tile(0u, B_BASE, kt);
                copy_tile(A_BYTES, B_BASE + B_BYTES, kt + 1);
                wait_vmcnt<LOADS>();
                zero_tail(0u, B_BASE, kt);
            } else if constexpr (SPREAD != 3) {
                constexpr int PRE = SPREAD == 1 ? STAGES - 1 : STAGES;
                unroll<PRE>([&](auto sc) __attribute__((always_inline)) {
                    constexpr int st = decltype(sc)::value;
                    copy_tile(st * STAGE_BYTES, st * STAGE_BYTES + A_BYTES, kt + st);
                });
                wait_vmcnt<(PRE - 1) * LOADS>();
                zero_tail(0u, A_BYTES, kt);
            }
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            /* fragments of the first K-step (SPREAD 2: the first two) */
            unroll<SPREAD == 2 ? 2 : 1>([&](auto pc) __attribute__((always_inline)) {
                constexpr int b = decltype(pc)::value;
#pragma unroll
                for (int i = 0; i < FM; ++i) fa[b][i] = frag(smem + wm * WTM * RB, b, i);
#pragma unroll
                for (int j = 0; j < FN; ++j) fb[b][j] = frag(smem + B_BASE + wn * WTN * RB, b, j);
            });
            read_scales(smem);
            uint32_t so = 0, dso = (STAGES - 1) * STAGE_BYTES;
            if constexpr (SPREAD == 2) {
                for (; kt < nkt; ++kt) {
                    const uint32_t nso = next_stage(so);
                    tile2(so, nso, kt);
                    so = nso;
                }
            } else if constexpr (SPREAD == 5) {
                /* A's stage of K-tile kt at sa (two), B's at sb (three) */
                uint32_t sa = 0, sb = B_BASE;
                auto next_b = [](uint32_t b) __attribute__((always_inline)) {
                    return b + B_BYTES == B_BASE + BST * B_BYTES ? (uint32_t)B_BASE : b + B_BYTES;
                };
                for (; kt < nkt; ++kt) {
                    const uint32_t na = sa ^ (uint32_t)A_BYTES, nb = next_b(sb), db = next_b(nb);
                    /* step 0: B's copies of K-tile kt+2 into B's stage of kt-1 */
                    KV kv = kvalid(kt + 2);
                    const uint32_t kb = (uint32_t)ktile(kt + 2) * KTB;
                    step(IC<0>{}, IC<A_LOADS>{}, IC<B_LOADS>{}, smem + sa, smem + sb, 1, 0u, db, kb, kv, IC<0>{});
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    /* K-tile kt+1 landed: only this step's copies may be
                     * outstanding */
                    wait_vmcnt<B_LOADS>();
                    zero_tail(na, nb, kt + 1);
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    /* step 1: A's copies of K-tile kt+2 into this tile's A stage */
                    step(IC<1>{}, IC<0>{}, IC<A_LOADS>{}, smem + na, smem + nb, 0, sa, 0u, kb, kv, IC<1>{});
                    sa = na;
                    sb = nb;
                }
            } else if constexpr (SPREAD == 6) {
                /* Per K-tile kt, four phases, each closed by a barrier:
                 *   M0  the FM x FN MFMAs of K-step 0 (buffer 0)
                 *   R0  K-step 1's fragments of kt into buffer 1; B's copies
                 *       of kt+2 into B's stage of kt-1; then this wave's
                 *       copies of kt+1 have landed
                 *   M1  the MFMAs of K-step 1 (buffer 1)
                 *   R1  K-step 0's fragments of kt+1 into buffer 0; A's
                 *       copies of kt+2 into A's stage of kt
                 * Block row 1 passes one barrier more before the loop and
                 * block row 0 one more after it, so every wavefront passes
                 * the same number and each barrier closes a phase of one
                 * kind in block row 0 and of the other kind in block row 1.
                 * Stage use: R1 of either row reads kt+1 after the barrier
                 * that closes R0 of row 1 (row 0's R0 closed a phase
                 * earlier), so every copy of kt+1 has landed; A's stage of
                 * kt is last read in R0 of row 1, closed before row 0's R1
                 * copies into it; B's stage of kt-1 was last read in R0 of
                 * kt-1. */
                auto mma = [&](auto cur_c) __attribute__((always_inline)) {
                    constexpr int CUR = decltype(cur_c)::value;
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    unroll<FM * FN>([&](auto tc) __attribute__((always_inline)) {
                        constexpr int t = decltype(tc)::value, i = t / FN, j = t % FN;
                        if constexpr (!FP8 && MI == 32)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][i], fb[CUR][j], acc[i][j], 0, 0, 0);
                        else if constexpr (!FP8)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[CUR][i], fb[CUR][j], acc[i][j], 0, 0, 0);
                        else if constexpr (MI == 32)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[CUR][i], fb[CUR][j], acc[i][j],
                                                                                         FA, FB, 0, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[CUR][i], fb[CUR][j], acc[i][j],
                                                                                          FA, FB, 0, 0, 0, 0);
                    });
                    __builtin_amdgcn_sched_barrier(0);
                };
                /* fragments of step nks of the stage at ns / nbs into buffer
                 * TGT, with copies D0 .. D0+DN-1 spread over the reads */
                auto feed = [&](auto tgt_c, const uint8_t *ns, const uint8_t *nbs, int nks, auto d0_c, auto dn_c,
                                uint32_t dso, uint32_t dsob, uint32_t kb, const KV &kv) __attribute__((always_inline)) {
                    constexpr int TGT = decltype(tgt_c)::value;
                    constexpr int D0 = decltype(d0_c)::value, DN = decltype(dn_c)::value, NR = FM + FN;
                    unroll<NR>([&](auto tc) __attribute__((always_inline)) {
                        constexpr int t = decltype(tc)::value;
                        if constexpr (t < FM)
                            fa[TGT][t] = frag(ns + wm * WTM * RB, nks, t);
                        else
                            fb[TGT][t - FM] = frag(nbs + wn * WTN * RB, nks, t - FM);
                        constexpr int j = (t * DN + NR - 1) / NR;
                        if constexpr (j < DN && (j * NR) / DN == t)
                            dma(std::integral_constant<int, D0 + j>{}, dso, dsob, kb, kv);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                };
                auto phase_end = [&]() __attribute__((always_inline)) {
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                };
                uint32_t sa = 0, sb = B_BASE;
                auto next_b = [](uint32_t b) __attribute__((always_inline)) {
                    return b + B_BYTES == B_BASE + BST * B_BYTES ? (uint32_t)B_BASE : b + B_BYTES;
                };
                const bool lag = wm == 1;
                if (lag) phase_end();
                for (; kt < nkt; ++kt) {
                    const uint32_t na = sa ^ (uint32_t)A_BYTES, nb = next_b(sb), db = next_b(nb);
                    const KV kv = kvalid(kt + 2);
                    const uint32_t kb = (uint32_t)ktile(kt + 2) * KTB;
                    mma(IC<0>{});
                    phase_end();
                    feed(IC<1>{}, smem + sa, smem + sb, 1, IC<A_LOADS>{}, IC<B_LOADS>{}, 0u, db, kb, kv);
                    wait_vmcnt<B_LOADS>();
                    zero_tail(na, nb, kt + 1);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    phase_end();
                    mma(IC<1>{});
                    phase_end();
                    feed(IC<0>{}, smem + na, smem + nb, 0, IC<0>{}, IC<A_LOADS>{}, sa, 0u, kb, kv);
                    phase_end();
                    sa = na;
                    sb = nb;
                }
                if (!lag) phase_end();
            } else if constexpr (KSTEPS % 2 == 0) {
                /* one loop body; the stage advances around the ring */
                for (; kt < nkt; ++kt) {
                    const uint32_t nso = next_stage(so);
                    tile(P0{}, so, nso, dso, kt);
                    dso = so;
                    so = nso;
                }
            } else {
                for (;;) {
                    uint32_t nso = next_stage(so);
                    tile(P0{}, so, nso, dso, kt);
                    dso = so;
                    so = nso;
                    if (++kt >= nkt) break;
                    nso = next_stage(so);
                    tile(P1{}, so, nso, dso, kt);
                    dso = so;
                    so = nso;
                    if (++kt >= nkt) break;
                }
            }
        }

        /* Epilogue.  Accumulator layout of a 32 x 32 MFMA block: lane l holds
         * column l % 32, register 4 g + r holds row 8 g + 4 (l / 32) + r; of a
         * 16 x 16 block: lane l holds column l % 16, register r holds row
         * 4 (l / 16) + r.
         * Stores go through a buffer resource based at the tile's corner.
         * The lane index is re-materialised here so the compiler cannot
         * hoist the epilogue's addresses above the main loop and hold them
         * in registers across it. */
        /* per-unit clock hook: wave 0's main loop ends here */
        const uint64_t clk_loop = p.stamps ? __builtin_amdgcn_s_memtime() : 0;
        int el = lane_id();
        asm volatile("" : "+v"(el));
        const int ecol = el % MI, ehi = el / MI;
        /* row of accumulator register e relative to the lane's first row */
        auto erow = [](int e) __attribute__((always_inline)) { return MI == 32 ? (e >> 2) * 8 + (e & 3) : e; };
        const int32_t mrem = p.M - m0, nrem = p.N - n0;

        /* Staged epilogue: once the ring is idle, each MFMA wavefront writes
         * its WTM x WTN block of results (alpha applied, binary32) into its
         * own share of the LDS, FMP block rows per pass, then reads it back
         * as row segments and stores 16 bytes per lane (4 fp32 results, or 8
         * results rounded to bf16) instead of one 2- or 4-byte store per
         * result.  One write sequence serves both output types, so each
         * accumulator is read once.  A staged row is WTN fp32 plus 16 bytes
         * of padding (CWB bytes): the 64 / MI row groups one write
         * instruction covers (rows 4 apart) then start 16 banks apart, and
         * every staged address is the lane's base plus a constant.  Rows
         * past M and segments past N are not stored.  The columns of a
         * segment that straddles N, and every result when C's rows are not
         * 16-byte aligned (vec false), are stored element by element in a
         * second, rolled loop. */
        constexpr int WAVE_LDS = LDS_BYTES / NW;
        /* (no padding where a wave's share holds just one unpadded block row) */
        constexpr int CWB = WTN * 4 + (MI * (WTN * 4 + 16) <= WAVE_LDS ? 16 : 0), CW = WTN / 4;
        constexpr int FMP = [] {
            int f = FM;
            while (f > 0 && (FM % f != 0 || f * MI * CWB > WAVE_LDS)) --f;
            return f;
        }();
        static_assert(FMP > 0, "a wave's share of the LDS holds one block row of fp32 results");
        constexpr int PR = FMP * MI;
        /* output kind: 0 partial slot (fp32, pitch TN), 1 fp32 C, 2 bf16 C.
         * Staged: bf16 C, and fp32 C from 16 x 16 blocks (a store of one
         * register then covers only 64 bytes of each of 4 rows) when C's
         * rows are 16-byte aligned.  Direct fp32 stores from the
         * accumulators: partial slots (a split tail's slots often hold a few
         * valid rows), fp32 C from 32 x 32 blocks, whose stores already
         * cover 128 contiguous bytes of each of 2 rows, and fp32 C whose rows
         * are not 16-byte aligned. */
        const int kind = un.slot >= 0 ? 0 : (p.out_bf16 ? 2 : 1);
        const bool use_staged = kind == 2 || (kind == 1 && MI == 16 && p.c_vec);
        if (!producer && kind == 0) {
            /* partial slot: the tile's positions inside M x N only (the
             * combine pass reads no others) */
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.ws + (int64_t)un.slot * (TM * TN));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = wn * WTN + j * MI + ecol;
                    const int row0 = wm * WTM + i * MI + ehi * 4;
                    const uint32_t voff = (uint32_t)((row0 * TN + col) * 4);
#pragma unroll
                    for (int e = 0; e < ACC_N; ++e) {
                        /* copy the element out first: a bit_cast applied to
                         * a vector subscript directly was lowered to element
                         * 0 for every e */
                        const float v = acc[i][j][e];
                        const bool ok = (row0 + erow(e) < mrem) && (col < nrem);
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rw, ok ? voff : kOOB,
                                                              erow(e) * TN * 4, 0);
                    }
                    /* one block at a time keeps the epilogue's registers few */
                    __builtin_amdgcn_sched_barrier(0);
                }
        } else if (!producer && !use_staged) {
            /* fp32 C straight from the accumulators */
            const float alpha = unit_alpha(p, un.batch);
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc((const uint8_t *)p.C + ((int64_t)un.batch * p.stride_c + (int64_t)m0 * p.ldc + n0) * 4);
            const int32_t ldcb = (int32_t)p.ldc * 4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = wn * WTN + j * MI + ecol;
                    const int row0 = wm * WTM + i * MI + ehi * 4;
                    const uint32_t voff = (uint32_t)(row0 * ldcb + col * 4);
#pragma unroll
                    for (int e = 0; e < ACC_N; ++e) {
                        const int dr = erow(e);
                        const bool ok = (row0 + dr < mrem) && (col < nrem);
                        const float v = alpha * acc[i][j][e];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, ok ? voff : kOOB,
                                                              dr * ldcb, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        if (use_staged) {
            /* the ring is idle: every wave's copies (those of K-tiles past
             * the range included) have landed and its fragment reads are done */
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        if (!producer && use_staged) {
            uint8_t *region = smem + wave * WAVE_LDS;
            /* the lane's staged element of register 0 of block (0, 0) */
            uint8_t *lbase = region + ehi * 4 * CWB + ecol * 4;
            const int os = kind == 2 ? 2 : 4;
            const float alpha = unit_alpha(p, un.batch);
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc((const uint8_t *)p.C + ((int64_t)un.batch * p.stride_c + (int64_t)m0 * p.ldc + n0) * os);
            const int32_t ldcb = (int32_t)p.ldc * os;
            const bool vec = p.c_vec != 0;
            /* output elements per 16-byte segment */
            const int epc = 16 / os;
            /* this wave's columns end inside a segment of C */
            const int ncol = nrem - wn * WTN;
            const bool edge = ncol > 0 && ncol < WTN && ncol % epc != 0;
#pragma unroll
            for (int ps = 0; ps < FM / FMP; ++ps) {
#pragma unroll
                for (int ii = 0; ii < FMP; ++ii)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
#pragma unroll
                        for (int e = 0; e < ACC_N; ++e)
                            *(float *)(lbase + (ii * MI + erow(e)) * CWB + j * MI * 4) = alpha * acc[ps * FMP + ii][j][e];
                        /* one block at a time keeps the epilogue's registers few */
                        __builtin_amdgcn_sched_barrier(0);
                    }
                if (vec) {
                    if (kind == 2) {
                        /* segment q: staged row q / (CW/2), bf16 columns
                         * 8 (q % (CW/2)) .. + 7 from fp32 chunks 2c, 2c + 1 */
                        constexpr int NSEG = PR * CW / 2, IT = (NSEG + 63) / 64;
#pragma unroll
                        for (int it = 0; it < IT; ++it) {
                            const int q = it * 64 + el;
                            if (NSEG % 64 == 0 || q < NSEG) {
                                const int r = q / (CW / 2), c = q % (CW / 2);
                                const f32x4 lo = *(const f32x4 *)(region + r * CWB + 32 * c);
                                const f32x4 hi = *(const f32x4 *)(region + r * CWB + 32 * c + 16);
                                const int grow = wm * WTM + ps * PR + r, gcol = wn * WTN + 8 * c;
                                const bool full = grow < mrem && gcol + 8 <= nrem;
                                __attribute__((ext_vector_type(4))) uint32_t d;
                                d[0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo[0], (__bf16)lo[1]});
                                d[1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo[2], (__bf16)lo[3]});
                                d[2] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)hi[0], (__bf16)hi[1]});
                                d[3] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)hi[2], (__bf16)hi[3]});
                                __builtin_amdgcn_raw_buffer_store_b128(d, rc, full ? (uint32_t)(grow * ldcb + gcol * 2) : kOOB,
                                                                       0, 0);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
                        constexpr int NSEG = PR * CW, IT = (NSEG + 63) / 64;
#pragma unroll
                        for (int it = 0; it < IT; ++it) {
                            const int q = it * 64 + el;
                            if (NSEG % 64 == 0 || q < NSEG) {
                                const int r = q / CW, c = q % CW;
                                const i32x4 d = *(const i32x4 *)(region + r * CWB + 16 * c);
                                const int grow = wm * WTM + ps * PR + r, gcol = wn * WTN + 4 * c;
                                const bool full = grow < mrem && gcol + 4 <= nrem;
                                __builtin_amdgcn_raw_buffer_store_b128(
                                    __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, d), rc,
                                    full ? (uint32_t)(grow * ldcb + gcol * 4) : kOOB, 0, 0);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
                if (!vec || edge) {
                    /* element by element, 64 consecutive columns of a row
                     * per store instruction: every result when C's rows are
                     * not 16-byte aligned, else the columns of the segment
                     * that straddles N (those past the last whole segment) */
                    const int c0 = vec ? ncol - ncol % epc : 0, cn = vec ? ncol % epc : WTN;
                    for (int t = el; t < PR * cn; t += 64) {
                        const int r = t / cn, col = c0 + t % cn;
                        const int grow = wm * WTM + ps * PR + r, gcol = wn * WTN + col;
                        if (grow < mrem && gcol < nrem) {
                            const float v = *(const float *)(region + r * CWB + col * 4);
                            const uint32_t voff = (uint32_t)(grow * ldcb + gcol * os);
                            if (os == 2)
                                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), rc, voff,
                                                                      0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, voff, 0, 0);
                        }
                    }
                }
            }
        }
        if (use_staged) {
            /* every wave has read its staged results back before the next
             * unit's copies refill the ring */
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        if (p.stamps) {
            /* wave 0 has issued its epilogue's stores */
            const uint64_t clk_epi = __builtin_amdgcn_s_memtime();
            /* every wave's stores of this unit have completed */
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            const uint64_t stamp1 = __builtin_amdgcn_s_memrealtime();
            const uint64_t clk1 = __builtin_amdgcn_s_memtime();
            if (wave == 0 && lane_id() == 0) {
                uint64_t *st = p.stamps + 6 * (int64_t)u;
                st[0] = stamp0;
                st[1] = stamp1;
                st[2] = clk0;
                st[3] = clk1;
                st[4] = clk_loop;
                st[5] = clk_epi;
            }
        }
    }
}

/*
 * Split-K combine.  Block x = (reduce tile q, chunk of P float4 positions of
 * the tile); its 256 threads are SG slice groups of P = 256 / SG positions.
 * Group g sums slices [g nsl / SG, (g + 1) nsl / SG) of its position in
 * ascending order; the group sums are then added in ascending group order,
 * so the result is the same on every run.
 */
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams r)
{
    __shared__ f32x4 part[256];
    const int32_t q = blockIdx.x / r.chunks, chunk = blockIdx.x % r.chunks;
    int32_t tile, nsl;
    if (r.tail) {
        tile = r.s.tail_first + q;
        nsl = r.s.tail_split;
    } else {
        tile = q;
        nsl = r.s.split;
    }
    Unit un;
    tile_coords(r.s, tile, un);
    const int32_t m0 = un.tile_m * r.TM, n0 = un.tile_n * r.TN;
    const int32_t SG = 1 << r.sg_log2, P = 256 >> r.sg_log2;
    const int32_t g = (int32_t)threadIdx.x / P, pos = (int32_t)threadIdx.x % P;
    const int64_t tile_f4 = (int64_t)r.TM * r.TN / 4;
    const int64_t e4 = (int64_t)chunk * P + pos;
    /* positions outside M x N were not written by the main pass and are
     * not read here */
    const bool live = e4 < tile_f4 && m0 + (int32_t)(e4 * 4 / r.TN) < r.M && n0 + (int32_t)(e4 * 4 % r.TN) < r.N;
    const int32_t s_lo = (int32_t)((int64_t)g * nsl / SG), s_hi = (int32_t)((int64_t)(g + 1) * nsl / SG);
    /* the scales are fetched while the slices load */
    float alpha = 1.0f;
    if (r.scale_a) alpha *= r.scale_a[un.batch];
    if (r.scale_b) alpha *= r.scale_b[un.batch];
    f32x4 sum = f32x4{};
    if (live) {
        const f32x4 *src = (const f32x4 *)(r.ws + (int64_t)q * nsl * r.TM * r.TN) + e4;
        int32_t i = s_lo;
        for (; i + 4 <= s_hi; i += 4) {
            const f32x4 v0 = src[(int64_t)i * tile_f4], v1 = src[(int64_t)(i + 1) * tile_f4];
            const f32x4 v2 = src[(int64_t)(i + 2) * tile_f4], v3 = src[(int64_t)(i + 3) * tile_f4];
            sum += v0;
            sum += v1;
            sum += v2;
            sum += v3;
        }
        for (; i < s_hi; ++i) sum += src[(int64_t)i * tile_f4];
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    if (g != 0 || !live) return;
    /* the group sums in ascending order, read seven or eight at a time (SG
     * is a power of two): groups 1 .. 7, then 8 .. 15, ... */
    if (SG >= 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 1; j < 8; ++j) v[j] = part[j * P + pos];
#pragma unroll
        for (int j = 1; j < 8; ++j) sum += v[j];
        for (int32_t h = 8; h < SG; h += 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = part[(h + j) * P + pos];
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += v[j];
        }
    } else {
        for (int32_t h = 1; h < SG; ++h) sum += part[h * P + pos];
    }
    const int64_t e = e4 * 4;
    const int32_t row = m0 + (int32_t)(e / r.TN);
    const int32_t col0 = n0 + (int32_t)(e % r.TN);
    if (row >= r.M) return;
    const int64_t cbase = (int64_t)un.batch * r.stride_c + (int64_t)row * r.ldc;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int32_t col = col0 + c;
        if (col < r.N) {
            const float v = alpha * sum[c];
            if (r.out_bf16)
                ((__bf16 *)r.C)[cbase + col] = (__bf16)v;
            else
                ((float *)r.C)[cbase + col] = v;
        }
    }
}

/*
 * Repack one operand to K-contiguous rows of ldd_bytes (a multiple of 16),
 * zero-filled beyond K.  Source element (row, k) of batch entry g is at
 * src[g*stride + (kmajor ? row*ld + k : k*ld + row)] (elements of esize
 * bytes).  pack_kernel repacks up to two operands in one launch: blocks
 * [0, nb0) work on the first, the rest on the second.
 *
 * pack_rows (K-contiguous source whose rows are misaligned or whose K is
 * not a whole number of 16-byte chunks): one lane per 16-byte chunk of the
 * padded output, the chunks of consecutive rows numbered consecutively
 * (row r, chunk c is chunk r * cpr + c), 256 per workgroup, a workgroup
 * within one batch entry.  A chunk wholly inside the row is one 16-byte
 * load at its own byte offset (buffer loads take any byte address); the
 * chunk that holds the row's last n < 16 bytes loads the row's last 16
 * bytes instead (never past the row) and shifts them down by 16 - n; rows
 * shorter than 16 bytes are read element by element.  Bytes at or beyond
 * K are zero.
 */
__device__ __forceinline__ i32x4 pack_chunk(const i32x4 lo, const i32x4 hi, uint32_t q, uint32_t rb, uint32_t valid)
{
    const int w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    int o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        /* dword j of the chunk: bytes sh + 4j .. sh + 4j + 3 of the window,
         * i.e. (w[q + j + 1] : w[q + j]) >> (8 rb) */
        int d0 = w[j], d1 = w[j + 1];
        if (q == 1) { d0 = w[j + 1]; d1 = w[j + 2]; }
        if (q == 2) { d0 = w[j + 2]; d1 = w[j + 3]; }
        if (q == 3) { d0 = w[j + 3]; d1 = w[j + 4]; }
        o[j] = (int)__builtin_amdgcn_alignbyte((uint32_t)d1, (uint32_t)d0, rb);
    }
    if (valid < 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int32_t vb = (int32_t)valid - 4 * j;
            const uint32_t keep = vb >= 4 ? 0xFFFFFFFFu : (vb <= 0 ? 0u : (1u << (8 * vb)) - 1u);
            o[j] = (int)((uint32_t)o[j] & keep);
        }
    }
    return i32x4{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ void pack_rows(const PackParams &pk, int64_t blk)
{
    const int64_t cpr = pk.ldd_bytes / 16;
    const int64_t per_entry = (int64_t)pk.rows * cpr;
    const int64_t bpe = (per_entry + 255) / 256;
    const int64_t g = blk / bpe;
    /* the workgroup's first chunk and its row r0 (within batch entry g) */
    const int64_t q0 = (blk - g * bpe) * 256;
    const int64_t r0 = q0 / cpr;
    if (q0 + (int64_t)threadIdx.x >= per_entry) return;
    const uint32_t ql = (uint32_t)(q0 - r0 * cpr) + threadIdx.x;
    const uint32_t dr = ql / (uint32_t)cpr, c = ql - dr * (uint32_t)cpr;
    const int64_t r = r0 + dr;
    const int64_t ld_bytes = pk.ld * pk.esize;
    const uint8_t *entry = (const uint8_t *)pk.src + g * pk.stride * pk.esize;
    const uint32_t kbytes = (uint32_t)pk.K * (uint32_t)pk.esize;
    const uint32_t off = c * 16u;
    /* a buffer resource based at row r0 serves the whole workgroup while
     * the rows it spans (256 / cpr + 2 at most) stay within 31-bit offsets;
     * otherwise (short rows far apart) bytes are read one by one */
    const bool near = (256 / cpr + 2) * ld_bytes < ((int64_t)1 << 31);
    i32x4 out = i32x4{0, 0, 0, 0};
    if (near && kbytes >= 16u) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(entry + r0 * ld_bytes);
        const uint32_t rowoff = dr * (uint32_t)ld_bytes;
        if (off + 16u <= kbytes) {
            out = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, rowoff + off, 0, 0));
        } else if (off < kbytes) {
            const uint32_t n = kbytes - off, sh = 16u - n;
            const i32x4 w =
                __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, rowoff + kbytes - 16u, 0, 0));
            out = pack_chunk(w, i32x4{0, 0, 0, 0}, sh >> 2, sh & 3u, n);
        }
    } else if (off < kbytes) {
        const uint8_t *row = entry + r * ld_bytes;
        const uint32_t n = kbytes - off < 16u ? kbytes - off : 16u;
        uint32_t wd[4] = {0, 0, 0, 0};
        for (uint32_t b = 0; b < n; ++b) wd[b >> 2] |= (uint32_t)row[off + b] << (8 * (b & 3));
        out = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
    }
    *(i32x4 *)(pk.dst + g * pk.dst_stride_bytes + r * pk.ldd_bytes + off) = out;
}

/*
 * pack_transpose (source with rows contiguous along the operand's M or N
 * index, i.e. element (row, k) at k*ld + row): a workgroup moves a 64-row x
 * 64-k block through LDS: reads along rows (consecutive lanes, consecutive
 * rows), writes 16-byte chunks of the K-contiguous output.  Blocks along k
 * cover the whole padded row; k >= K reads as zero.
 */
__device__ __forceinline__ void pack_transpose(const PackParams &pk, int64_t bid, uint16_t (*tile)[65])
{
    const int32_t kblocks = (int32_t)((pk.ldd_bytes / pk.esize + 63) / 64);
    const int32_t rblocks = (pk.rows + 63) / 64;
    const int32_t kb = (int32_t)(bid % kblocks);
    const int64_t t2 = bid / kblocks;
    const int32_t rbk = (int32_t)(t2 % rblocks);
    const int64_t g = t2 / rblocks;
    const int32_t r0 = rbk * 64, k0 = kb * 64;
    const int t = threadIdx.x;
    const int rr = t & 63;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int kk = (t >> 6) + 4 * i;
        const int32_t row = r0 + rr, k = k0 + kk;
        uint16_t v = 0;
        if (row < pk.rows && k < pk.K) {
            const int64_t idx = g * pk.stride + (int64_t)k * pk.ld + row;
            v = pk.esize == 2 ? ((const uint16_t *)pk.src)[idx] : ((const uint8_t *)pk.src)[idx];
        }
        tile[kk][rr] = v;
    }
    __syncthreads();
    /* output: 64 rows x (64 esize) bytes = 64 x (8 or 4) chunks of 16 bytes */
    const int cpr = pk.esize == 2 ? 8 : 4;
    const int per = 16 / pk.esize;
    for (int idx = t; idx < 64 * cpr; idx += 256) {
        const int r = idx / cpr, qc = idx % cpr;
        const int32_t row = r0 + r;
        const int64_t boff = (int64_t)k0 * pk.esize + qc * 16;
        if (row >= pk.rows || boff >= pk.ldd_bytes) continue;
        uint8_t out[16];
        for (int e = 0; e < per; ++e) {
            const uint16_t v = tile[qc * per + e][r];
            if (pk.esize == 2) {
                out[2 * e] = (uint8_t)(v & 0xFF);
                out[2 * e + 1] = (uint8_t)(v >> 8);
            } else {
                out[e] = (uint8_t)v;
            }
        }
        i32x4 w;
        __builtin_memcpy(&w, out, 16);
        *(i32x4 *)(pk.dst + g * pk.dst_stride_bytes + (int64_t)row * pk.ldd_bytes + boff) = w;
    }
}

__global__ __launch_bounds__(256) void pack_kernel(PackParams p0, PackParams p1, uint32_t nb0)
{
    __shared__ uint16_t tile[64][65];
    const bool first = blockIdx.x < nb0;
    const PackParams &pk = first ? p0 : p1;
    const int64_t blk = first ? (int64_t)blockIdx.x : (int64_t)(blockIdx.x - nb0);
    if (pk.kmajor)
        pack_rows(pk, blk);
    else
        pack_transpose(pk, blk, tile);
}

/*
 * Block-scale regrouping for the MX tiles: src holds batch x rows x (4 nK)
 * E8M0 bytes (a row's four scales of K-tile kt are bytes 4 kt .. 4 kt + 3,
 * one dword); dst[b][kt][row] receives that dword.  Block (b, row block of
 * 64, K-tile block of 32) moves a 64 x 32 dword tile through LDS: reads of
 * 128 contiguous bytes per row, writes of 256 contiguous bytes per K-tile.
 */
__global__ __launch_bounds__(256) void pack_scales_kernel(ScalePackParams sp)
{
    __shared__ uint32_t t[64][33];
    const int32_t rblocks = (sp.rows + 63) / 64, kblocks = (sp.nK + 31) / 32;
    int32_t bid = blockIdx.x;
    const int32_t kb = bid % kblocks;
    bid /= kblocks;
    const int32_t rb = bid % rblocks;
    const int32_t b = bid / rblocks;
    const int32_t r0 = rb * 64, k0 = kb * 32;
    const uint32_t *src = (const uint32_t *)sp.src + (int64_t)b * sp.rows * sp.nK;
    uint32_t *dst = sp.dst + (int64_t)b * sp.rows * sp.nK;
    for (int32_t i = threadIdx.x; i < 64 * 32; i += 256) {
        const int32_t r = i / 32, k = i % 32;
        if (r0 + r < sp.rows && k0 + k < sp.nK) t[r][k] = src[(int64_t)(r0 + r) * sp.nK + k0 + k];
    }
    __syncthreads();
    for (int32_t i = threadIdx.x; i < 64 * 32; i += 256) {
        const int32_t k = i / 64, r = i % 64;
        if (r0 + r < sp.rows && k0 + k < sp.nK) dst[(int64_t)(k0 + k) * sp.rows + r0 + r] = t[r][k];
    }
}

__global__ __launch_bounds__(256) void zero_kernel(void *C, int32_t M, int32_t N, int64_t ldc,
                                                    int64_t stride_c, int32_t batch, int32_t esize)
{
    const int64_t total = (int64_t)batch * M * N;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t g = t / ((int64_t)M * N);
        const int64_t rem = t - g * M * N;
        const int64_t idx = g * stride_c + (rem / N) * ldc + rem % N;
        if (esize == 4)
            ((float *)C)[idx] = 0.0f;
        else
            ((uint16_t *)C)[idx] = 0;
    }
}

/* ------------------------------------------------------------------ launch */

template <int TM, int TN, int EL, int MINB, int RB, int STAGES, int WGM, int WGN, int SPREAD, int OP, int MI, int FMT>
static hipError_t launch_one(const GemmParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_tile_kernel<TM, TN, EL, MINB, RB, STAGES, WGM, WGN, SPREAD, OP, MI, FMT>), dim3(p.s.grid),
                       dim3((WGM * WGN + (SPREAD == 3 ? 4 : 0)) * 64), 0, stream, p);
    return hipGetLastError();
}

/* bf16 tiles have one instantiation; 8-bit tiles one per operand-format pair */
template <int TM, int TN, int EL, int MINB, int RB, int STAGES, int WGM, int WGN, int SPREAD, int OP, int MI>
static hipError_t launch_tile(int32_t fmt, const GemmParams &p, hipStream_t stream)
{
    if constexpr (EL == 3) {
        if (fmt != 0) return hipErrorInvalidValue;
        return launch_one<TM, TN, EL, MINB, RB, STAGES, WGM, WGN, SPREAD, OP, MI, 0>(p, stream);
    } else if constexpr (EL != 0) {
        switch (fmt) {
        case 0: return launch_one<TM, TN, EL, MINB, RB, STAGES, WGM, WGN, SPREAD, OP, MI, 0>(p, stream);
        case 1: return launch_one<TM, TN, EL, MINB, RB, STAGES, WGM, WGN, SPREAD, OP, MI, 1>(p, stream);
        case 2: return launch_one<TM, TN, EL, MINB, RB, STAGES, WGM, WGN, SPREAD, OP, MI, 2>(p, stream);
        default: return hipErrorInvalidValue;
        }
    } else {
        if (fmt != 0) return hipErrorInvalidValue;
        return launch_one<TM, TN, EL, MINB, RB, STAGES, WGM, WGN, SPREAD, OP, MI, 0>(p, stream);
    }
}

/* Instantiations, in tile-table order (csrc/tiles.h):
 * id, TM, TN, element class (false bf16, true 8-bit, 2 block-scaled 8-bit,
 * 3 block-scaled FP4, 4 block-scaled FP6),
 * groups per CU, K-tile bytes, stages, waves along M, N, copy schedule,
 * MFMA block edge, operation (0 matrix product, 1 convolution) */
#define GEMM355_TILES(X)                                                                          \
    X(0, 256, 256, false, 1, 128, 2, 2, 2, 0, 32, 0)                                                       \
    X(1, 128, 128, false, 2, 128, 2, 2, 2, 0, 32, 0)                                                       \
    X(2, 64, 64, false, 4, 128, 2, 2, 2, 0, 32, 0)                                                         \
    X(3, 256, 256, true, 1, 128, 2, 2, 2, 0, 32, 0)                                                        \
    X(4, 128, 128, true, 2, 128, 2, 2, 2, 0, 32, 0)                                                        \
    X(5, 64, 64, true, 4, 128, 2, 2, 2, 0, 32, 0)                                                          \
    X(6, 256, 256, false, 1, 64, 4, 2, 2, 0, 32, 0)                                                        \
    X(7, 256, 256, false, 1, 64, 5, 2, 2, 0, 32, 0)                                                        \
    X(8, 256, 256, true, 1, 64, 4, 2, 2, 0, 32, 0)                                                         \
    X(9, 256, 256, true, 1, 64, 5, 2, 2, 0, 32, 0)                                                         \
    X(10, 256, 256, false, 1, 128, 2, 2, 4, 0, 32, 0)                                                      \
    X(11, 256, 256, false, 1, 64, 4, 2, 4, 0, 32, 0)                                                       \
    X(12, 256, 256, true, 1, 128, 2, 2, 4, 0, 32, 0)                                                       \
    X(13, 256, 256, true, 1, 64, 4, 2, 4, 0, 32, 0)                                                        \
    X(14, 64, 64, false, 1, 128, 8, 2, 2, 0, 32, 0)                                                        \
    X(15, 64, 64, false, 2, 128, 4, 2, 2, 0, 32, 0)                                                        \
    X(16, 128, 128, false, 1, 128, 4, 2, 2, 0, 32, 0)                                                      \
    X(17, 64, 64, true, 1, 128, 8, 2, 2, 0, 32, 0)                                                         \
    X(18, 64, 64, true, 2, 128, 4, 2, 2, 0, 32, 0)                                                         \
    X(19, 128, 128, true, 1, 128, 4, 2, 2, 0, 32, 0)                                                       \
    X(20, 64, 64, false, 4, 128, 2, 1, 1, 0, 32, 0)                                                        \
    X(21, 64, 64, false, 2, 128, 4, 1, 1, 0, 32, 0)                                                        \
    X(22, 64, 64, true, 4, 128, 2, 1, 1, 0, 32, 0)                                                         \
    X(23, 64, 64, true, 2, 128, 4, 1, 1, 0, 32, 0)                                                         \
    X(24, 256, 256, false, 1, 64, 4, 2, 2, 1, 32, 0)                                                       \
    X(25, 256, 256, false, 1, 64, 5, 2, 2, 1, 32, 0)                                                       \
    X(26, 256, 256, false, 1, 64, 4, 2, 4, 1, 32, 0)                                                       \
    X(27, 256, 256, false, 1, 64, 5, 2, 4, 1, 32, 0)                                                       \
    X(28, 256, 256, true, 1, 64, 4, 2, 2, 1, 32, 0)                                                        \
    X(29, 256, 256, true, 1, 64, 5, 2, 2, 1, 32, 0)                                                        \
    X(30, 256, 256, true, 1, 64, 4, 2, 4, 1, 32, 0)                                                        \
    X(31, 256, 256, true, 1, 64, 5, 2, 4, 1, 32, 0)                                                        \
    X(32, 256, 256, false, 1, 128, 2, 4, 4, 0, 32, 0)                                                      \
    X(33, 256, 256, false, 1, 64, 4, 4, 4, 0, 32, 0)                                                       \
    X(34, 256, 256, false, 1, 64, 4, 4, 4, 1, 32, 0)                                                   \
    X(35, 256, 256, false, 1, 128, 2, 2, 2, 0, 16, 0)                                                  \
    X(36, 256, 256, false, 1, 128, 2, 2, 4, 0, 16, 0)                                                  \
    X(37, 256, 256, false, 1, 64, 4, 2, 4, 0, 16, 0)                                                   \
    X(38, 256, 256, false, 1, 64, 4, 2, 2, 0, 16, 0)                                                   \
    X(39, 256, 256, false, 1, 64, 4, 2, 2, 1, 16, 0)                                                   \
    X(40, 256, 256, false, 1, 64, 5, 2, 2, 0, 16, 0)                                                   \
    X(41, 256, 256, false, 1, 128, 2, 2, 2, 2, 32, 0)                                                  \
    X(42, 256, 256, false, 1, 128, 2, 2, 4, 2, 32, 0)                                                  \
    X(43, 128, 128, false, 2, 128, 2, 2, 2, 2, 32, 0)                                                  \
    X(44, 256, 128, false, 1, 128, 3, 2, 2, 3, 32, 0)                                                  \
    X(45, 256, 128, false, 1, 128, 3, 2, 2, 3, 16, 0)                                                  \
    X(46, 256, 128, true, 1, 128, 3, 2, 2, 3, 32, 0)                                                   \
    X(47, 256, 128, false, 1, 128, 3, 2, 2, 0, 32, 0)                                                  \
    X(48, 256, 256, 2, 1, 128, 2, 2, 2, 0, 32, 0)                                                      \
    X(49, 128, 128, 2, 2, 128, 2, 2, 2, 0, 32, 0)                                                      \
    X(50, 128, 128, 2, 1, 128, 4, 2, 2, 0, 32, 0)                                                      \
    X(51, 256, 256, 3, 1, 128, 2, 2, 2, 0, 32, 0)                                                      \
    X(52, 128, 128, 3, 2, 128, 2, 2, 2, 0, 32, 0)                                                      \
    X(53, 128, 128, 3, 1, 128, 4, 2, 2, 0, 32, 0)                                                   \
    X(54, 256, 256, false, 1, 128, 2, 2, 2, 0, 32, 1)                                               \
    X(55, 128, 128, false, 2, 128, 2, 2, 2, 0, 32, 1)                                               \
    X(56, 64, 64, false, 4, 128, 2, 2, 2, 0, 32, 1)                                                 \
    X(57, 256, 256, false, 1, 128, 2, 2, 4, 0, 16, 1)                                               \
    X(58, 128, 128, false, 1, 128, 4, 2, 2, 0, 32, 1)                                               \
    X(59, 256, 256, 4, 1, 128, 2, 2, 2, 0, 32, 0)                                                   \
    X(60, 128, 128, 4, 2, 128, 2, 2, 2, 0, 32, 0)                                                   \
    X(61, 128, 128, 4, 1, 128, 4, 2, 2, 0, 32, 0)                                                   \
    X(62, 256, 256, false, 1, 128, 2, 2, 2, 4, 16, 0)                                               \
    X(63, 256, 256, false, 1, 128, 2, 2, 4, 5, 16, 0)                                               \
    X(64, 256, 256, 1, 1, 128, 2, 2, 2, 5, 32, 0)                                                   \
    X(65, 256, 256, false, 1, 128, 2, 2, 4, 6, 16, 0)                                               \
    X(66, 256, 256, 1, 1, 128, 2, 2, 4, 6, 32, 0)

/* every instantiation agrees with its tile-table entry */
#define X(id, tm, tn, f8, mb, rb, st, wm, wn, sp, mi, opn)                                                      \
    static_assert(kTiles[id].dtype_class == (int)(f8) && kTiles[id].TM == tm &&                  \
                      kTiles[id].TN == tn && kTiles[id].min_blocks == mb &&                      \
                      kTiles[id].row_bytes == rb && kTiles[id].stages == st &&                   \
                      kTiles[id].waves_m == wm && kTiles[id].waves_n == wn &&                    \
                      kTiles[id].TK == ((f8) == 3 ? 2 * rb : (f8) ? rb : rb / 2) &&             \
                      kTiles[id].spread == sp &&                                                 \
                      kTiles[id].mfma == mi && kTiles[id].op == opn,                              \
                  "tile table entry " #id);
GEMM355_TILES(X)
#undef X
#define X(id, tm, tn, f8, mb, rb, st, wm, wn, sp, mi, opn) +1
static_assert(0 GEMM355_TILES(X) == kNumTiles, "one instantiation per tile-table entry");
#undef X

hipError_t launch_gemm(int32_t tile, int32_t fmt, const GemmParams &p, hipStream_t stream)
{
    switch (tile) {
#define X(id, tm, tn, f8, mb, rb, st, wm, wn, sp, mi, opn) \
    case id: return launch_tile<tm, tn, f8, mb, rb, st, wm, wn, sp, opn, mi>(fmt, p, stream);
        GEMM355_TILES(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

const void *gemm_kernel_symbol(int32_t tile)
{
    switch (tile) {
#define X(id, tm, tn, f8, mb, rb, st, wm, wn, sp, mi, opn) \
    case id: return (const void *)gemm_tile_kernel<tm, tn, f8, mb, rb, st, wm, wn, sp, opn, mi, 0>;
        GEMM355_TILES(X)
#undef X
    default: return nullptr;
    }
}

hipError_t launch_reduce(const ReduceParams &r0, int32_t tiles, hipStream_t stream)
{
    ReduceParams r = r0;
    const int32_t nsl = r.tail ? r.s.tail_split : r.s.split;
    /* slice groups: about four slices per thread, at most 64 groups */
    int32_t lg = 0;
    while (lg < 6 && (2 << lg) * 4 <= nsl) ++lg;
    r.sg_log2 = lg;
    const int64_t tile_f4 = (int64_t)r.TM * r.TN / 4;
    const int32_t P = 256 >> lg;
    r.chunks = (int32_t)((tile_f4 + P - 1) / P);
    hipLaunchKernelGGL(reduce_kernel, dim3((uint32_t)((int64_t)tiles * r.chunks)), dim3(256), 0, stream, r);
    return hipGetLastError();
}

static int64_t pack_blocks(const PackParams &pk)
{
    if (pk.kmajor) return (int64_t)pk.batch * (((int64_t)pk.rows * (pk.ldd_bytes / 16) + 255) / 256);
    const int64_t kblocks = (pk.ldd_bytes / pk.esize + 63) / 64;
    const int64_t rblocks = (pk.rows + 63) / 64;
    return (int64_t)pk.batch * rblocks * kblocks;
}

hipError_t launch_pack(const PackParams *pk, int n, hipStream_t stream)
{
    const int64_t nb0 = pack_blocks(pk[0]);
    const int64_t nb = nb0 + (n > 1 ? pack_blocks(pk[1]) : 0);
    if (nb >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)nb), dim3(256), 0, stream, pk[0], n > 1 ? pk[1] : pk[0],
                       (uint32_t)nb0);
    return hipGetLastError();
}

hipError_t launch_pack_scales(const ScalePackParams &sp, hipStream_t stream)
{
    const int64_t blocks = (int64_t)sp.batch * ((sp.rows + 63) / 64) * ((sp.nK + 31) / 32);
    hipLaunchKernelGGL(pack_scales_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, sp);
    return hipGetLastError();
}

hipError_t launch_zero(void *C, int32_t M, int32_t N, int64_t ldc, int64_t stride_c,
                       int32_t batch, int32_t esize, hipStream_t stream)
{
    const int64_t total = (int64_t)batch * M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, C, M, N, ldc,
                       stride_c, batch, esize);
    return hipGetLastError();
}

} /* namespace g355 */
