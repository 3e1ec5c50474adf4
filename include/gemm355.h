/*
 * gemm355.h -- C ABI of libgemm355, a tiled dense matrix product for AMD
 * Instinct MI355X (gfx950).
 *
 * Operation (page "10. Tensor Cores, shapes, and tile alignment", section
 * "Shape the operation", the problem statement and the FLOPs equation):
 *
 *     C[M x N] = alpha * A[M x K] * B[K x N]        (useful work 2MNK)
 *
 * with low-precision inputs and an fp32 accumulator (page "The Tensor Core",
 * the input/accumulate table: BF16 in the Ampere row, FP8 E4M3 in the Hopper
 * row, both accumulating in FP32).  C is overwritten (no beta term).  alpha
 * is 1 unless per-tensor scales are passed (scale_a[g] * scale_b[g] for
 * batch entry g), which is how E4M3 operands are dequantised.
 *
 * Conventions for every entry point:
 *   - Dimensions, leading dimensions and strides are counted in ELEMENTS of
 *     the operand's type.  C is row-major: C(i,j) is at C[i*ldc + j].
 *   - A, B, C, the scales and any workspace are device memory owned by the
 *     caller.  The library never frees them and keeps no reference after the
 *     call returns.  A and B are only read; C is only written.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL means the null
 *     stream).  Argument errors are reported before anything is launched;
 *     faults inside kernels surface at the caller's next synchronisation.
 *   - No entry point aborts, prints or throws; each returns a status code.
 *   - One HIP runtime per process: the library calls the libamdhip64 the
 *     process has loaded.  PyTorch's ROCm wheels carry their own copy,
 *     which they load under a name the loader does not match to one loaded
 *     first from the system ROCm; in a process that uses such a PyTorch,
 *     load PyTorch before this library (the Python binding does), or the
 *     process holds two runtimes and PyTorch's device memory is foreign to
 *     the library's launches (they fail with EHIP).
 *   - All entry points are thread-safe.  Scratch the library owns is kept
 *     per device and stream; a call holds that buffer from its lookup until
 *     its last kernel is enqueued, so concurrent calls on one stream enqueue
 *     their kernels call by call and never share partial sums.  A
 *     caller-provided workspace belongs to the caller: calls that may run
 *     at the same time (on different streams) need different workspaces.
 */
#ifndef GEMM355_H
#define GEMM355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM355_API __attribute__((visibility("default")))

typedef enum gemm355_status {
    GEMM355_OK = 0,
    GEMM355_EINVAL = 1,        /* bad size, leading dimension, pointer, enum,
                                  split factor, or C overlapping A/B */
    GEMM355_EALIGN = 2,        /* pointer not aligned to its element size */
    GEMM355_EUNSUPPORTED = 3,  /* extents beyond the 32-bit offsets the
                                  kernels use, an unknown tile id, an MX
                                  dtype with K not a multiple of 128, or an
                                  MX FP4 / FP6 call outside its limits */
    GEMM355_ENOMEM = 4,        /* caller workspace smaller than the plan's
                                  workspace_bytes, library scratch over the
                                  cap of gemm355_set_scratch_limit, or
                                  allocation failed */
    GEMM355_EHIP = 5,          /* a HIP runtime call failed (no device,
                                  launch failure) */
    GEMM355_ETOOBIG = 6        /* gemm355_gemm_noalloc: the plan needs more
                                  scratch than its fixed per-device buffer */
} gemm355_status;

/* Element types, input -> output.  The two 8-bit formats are the FP8 pair
 * of the Hopper row of the input/accumulate table (page "The Tensor Core"):
 * OCP E4M3FN (bias 7, max 448, no infinities, NaN 0x7F/0xFF) and OCP E5M2
 * (bias 15, max 57344, infinities 0x7C/0xFC, NaN above them).  Operands
 * must be finite. */
typedef enum gemm355_dtype {
    GEMM355_BF16_F32 = 0,   /* bf16 A, B; fp32 C                              */
    GEMM355_BF16_BF16 = 1,  /* bf16 A, B; bf16 C (fp32 result rounded to
                               nearest even)                                  */
    GEMM355_E4M3_F32 = 2,   /* E4M3 A, B; fp32 C                              */
    GEMM355_E4M3_BF16 = 3,  /* E4M3 A, B; bf16 C                              */
    GEMM355_E5M2_F32 = 4,   /* E5M2 A, B; fp32 C                              */
    GEMM355_E5M2_BF16 = 5,  /* E5M2 A, B; bf16 C                              */
    GEMM355_E4M3_E5M2_F32 = 6,  /* E4M3 A, E5M2 B; fp32 C                     */
    GEMM355_E4M3_E5M2_BF16 = 7, /* E4M3 A, E5M2 B; bf16 C                     */
    /* Block-scaled ("microscaled", the precision-table row after the FP8
     * pair on page "The Tensor Core"; format as in the OCP Microscaling
     * specification v1.0): every 32 consecutive K-values of a row of A and
     * of a column of B share one E8M0 scale 2^(e - 127), given in
     * block_scale_a / block_scale_b.  K must be a multiple of 128. */
    GEMM355_MXE4M3_F32 = 8,     /* MX E4M3 A, B; fp32 C                       */
    GEMM355_MXE4M3_BF16 = 9,    /* MX E4M3 A, B; bf16 C                       */
    GEMM355_MXE5M2_F32 = 10,    /* MX E5M2 A, B; fp32 C                       */
    GEMM355_MXE5M2_BF16 = 11,   /* MX E5M2 A, B; bf16 C                       */
    GEMM355_MXE4M3_E5M2_F32 = 12,  /* MX E4M3 A, MX E5M2 B; fp32 C            */
    GEMM355_MXE4M3_E5M2_BF16 = 13, /* MX E4M3 A, MX E5M2 B; bf16 C            */
    /* MX FP4: OCP E2M1 elements (1 sign, 2 exponent bits with bias 1, 1
     * mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte, element
     * 2i in the low nibble of byte i.  Native layout only (A row-major,
     * B column-major), lda, ldb and strides even, rows 16-byte aligned,
     * K a multiple of 256 (EUNSUPPORTED otherwise). */
    GEMM355_MXFP4_F32 = 14,        /* MX FP4 A, B; fp32 C                     */
    GEMM355_MXFP4_BF16 = 15,       /* MX FP4 A, B; bf16 C                     */
    /* MX FP6: OCP E2M3 (1 sign, 2 exponent bits with bias 1, 3 mantissa
     * bits; largest 7.5) or E3M2 (3 exponent bits with bias 3, 2 mantissa
     * bits; largest 28) elements, no infinities or NaN, packed four per
     * three bytes as a little-endian bit stream (element i in bits
     * 6i .. 6i+5 of its row).  Native layout only, lda, ldb and strides
     * multiples of 64, rows 16-byte aligned, K a multiple of 128
     * (EUNSUPPORTED otherwise). */
    GEMM355_MXFP6_E2M3_F32 = 16,   /* MX E2M3 A, B; fp32 C                    */
    GEMM355_MXFP6_E2M3_BF16 = 17,  /* MX E2M3 A, B; bf16 C                    */
    GEMM355_MXFP6_E3M2_F32 = 18,   /* MX E3M2 A, B; fp32 C                    */
    GEMM355_MXFP6_E3M2_BF16 = 19   /* MX E3M2 A, B; bf16 C                    */
} gemm355_dtype;

/* 8-bit formats of the quantiser. */
typedef enum gemm355_fp8 {
    GEMM355_FP8_E4M3 = 0,   /* OCP E4M3FN, largest finite 448                 */
    GEMM355_FP8_E5M2 = 1    /* OCP E5M2, largest finite 57344                 */
} gemm355_fp8;

/* Source element types of the quantiser. */
typedef enum gemm355_src {
    GEMM355_SRC_F32 = 0,
    GEMM355_SRC_BF16 = 1
} gemm355_src;

/* Operand storage (the row/column vocabulary of the sweep command in
 * section "Practical shape sweep"):
 *   A row-major:    a(i,k) = A[i*lda + k], lda >= K
 *   A column-major: a(i,k) = A[k*lda + i], lda >= M
 *   B column-major: b(k,j) = B[j*ldb + k], ldb >= K
 *   B row-major:    b(k,j) = B[k*ldb + j], ldb >= N
 * A row-major with B column-major (both K-contiguous) is the native layout;
 * the other three are first repacked into it on the device (counted in the
 * call's time). */
typedef enum gemm355_layout {
    GEMM355_A_ROW_B_COL = 0,
    GEMM355_A_ROW_B_ROW = 1,
    GEMM355_A_COL_B_COL = 2,
    GEMM355_A_COL_B_ROW = 3
} gemm355_layout;

/* Full argument set (strided batch, scales, workspace, tuning knobs). */
typedef struct gemm355_args {
    int64_t M, N, K;
    const void *A;  int64_t lda; int64_t stride_a;  /* stride_*: elements  */
    const void *B;  int64_t ldb; int64_t stride_b;  /* between consecutive */
    void *C;        int64_t ldc; int64_t stride_c;  /* batch entries       */
    int64_t batch;                 /* >= 1 independent products           */
    const float *scale_a;          /* device fp32 [batch] or NULL (= 1.0)  */
    const float *scale_b;          /* device fp32 [batch] or NULL (= 1.0)  */
    gemm355_dtype dtype;
    gemm355_layout layout;
    int32_t split_k;     /* 0: automatic; 1: off; s >= 2: cut K into s slices
                            (clamped to the number of K-tiles)             */
    int32_t persistent;  /* -1: automatic; 0: one workgroup per work unit;
                            1: grid of resident capacity looping over units,
                            with the last partial round split along K      */
    int32_t tile;        /* -1: automatic; else an index of the tile table */
    int32_t cus;         /* compute units S used for planning; 0: query the
                            current device (256 when no device is present) */
    void *workspace;          /* device scratch for split-K partial sums and
                                 repacked operands, 256-byte aligned
                                 (EALIGN otherwise); NULL: library-owned  */
    size_t workspace_bytes;   /* size of `workspace`                      */
    uint64_t *unit_stamps;    /* device uint64 [6 * plan.units] or NULL.
                                 When set, work unit u records the device
                                 real-time clock (100 MHz) when its
                                 workgroup starts it at [6u] and after its
                                 stores have completed at [6u + 1], and the
                                 shader clock counter (cycles) at the same
                                 two points at [6u + 2] and [6u + 3], when
                                 its first wavefront leaves the main loop
                                 at [6u + 4] and when that wavefront has
                                 issued its output stores at [6u + 5], for
                                 measuring how evenly the units fill the
                                 device and where a unit's cycles go.
                                 8-byte aligned (EALIGN).                  */
    /* Block scales of the MX dtypes (NULL otherwise, else EINVAL): E8M0
     * bytes, dense, block_scale_a[g][i][k / 32] for row i of A and
     * block_scale_b[g][j][k / 32] for column j of B (rows of K / 32 bytes,
     * batch entries M * K / 32 and N * K / 32 bytes apart), whatever the
     * element layout.  Device memory, 4-byte aligned (EALIGN); NULL with
     * M, N, K > 0 is EINVAL; overlapping C is EINVAL.  Scale 255 (NaN)
     * makes the affected outputs NaN.  The per-tensor scale_a / scale_b
     * still multiply the result when given. */
    const uint8_t *block_scale_a;
    const uint8_t *block_scale_b;
} gemm355_args;

/* Everything the planner decided for one call.  Efficiencies are exact
 * rationals num/den in lowest terms. */
typedef struct gemm355_plan_t {
    int32_t tile;                 /* tile-table index                      */
    int32_t T_M, T_N, T_K;        /* output tile and K-step of the loop    */
    int32_t stages, waves;        /* LDS ring depth; wavefronts per group  */
    int32_t lds_bytes;            /* LDS per workgroup                     */
    int32_t vgpr_budget;          /* VGPR+AGPR per lane the kernel may use */
    int32_t S;                    /* compute units                         */
    int32_t b;                    /* resident workgroups per CU            */
    int64_t G;                    /* output tiles, all batch entries       */
    int64_t nK;                   /* K-tiles: ceil(K / T_K)                */
    int64_t M_pad, N_pad, K_pad;  /* ceil(X / T_X) * T_X                   */
    int32_t split;                /* uniform K-split (1 = none)            */
    int32_t persistent;           /* 1 if the grid loops over units        */
    int64_t tail_tiles;           /* tiles of the last partial round that
                                     are split along K (0 = none)          */
    int32_t tail_split;           /* slices per tail tile                  */
    int32_t repack;               /* bit 0: A repacked, bit 1: B repacked  */
    int64_t units;                /* work units (tile, K-range)            */
    int64_t grid;                 /* workgroups launched by the main kernel */
    int64_t eta_wave_num, eta_wave_den;    /* G / (ceil(G/(S b)) S b)      */
    int64_t eta_pad_num, eta_pad_den;      /* MNK / (M'N'K')               */
    int64_t eta_sched_num, eta_sched_den;  /* sum of unit work over S*b
                                              times the busiest workgroup's */
    size_t workspace_bytes;       /* scratch this call needs               */
    double model_seconds;         /* the planner's time estimate (planning
                                     model only, not a measurement)        */
    /* The estimate's inputs for this schedule, so that a calibration can
     * refit the tile priors from timed plans:
     *   model_seconds = model_fixed_seconds
     *     + (t_mfma^4 + t_mem^4 + t_copy^4)^(1/4)
     *     + model_units_in_turn * (the per-unit fill and epilogue time),
     *   t_mfma = model_mfma_peak_seconds / model_mfma_eff,
     *   t_mem  = model_bytes / (5e12 * model_stream_eff * model_spread),
     *   t_copy = model_copy_seconds. */
    double model_mfma_peak_seconds; /* busiest CU's MFMA work at the dense
                                       peak of the input class           */
    double model_mfma_eff;        /* tile prior for the resident groups    */
    double model_bytes;           /* algorithmic bytes + partial-sum writes */
    double model_spread;          /* all work / (S x busiest CU's work)    */
    double model_stream_eff;      /* tile prior                            */
    double model_copy_seconds;    /* busiest CU's L2 -> LDS copies         */
    double model_fixed_seconds;   /* launches and the combine read-back    */
    int64_t model_units_in_turn;  /* units one workgroup slot runs in turn */
} gemm355_plan_t;

/*
 * gemm355_gemm -- C = A*B for one product, fp32 accumulate.
 *   M, N, K >= 0.  M == 0 or N == 0: nothing is done.  K == 0: C = 0.
 *   split_k: 0 automatic, 1 off, s >= 2 forced (clamped to ceil(K/T_K)).
 *   persistent: -1 automatic, 0 off, 1 on.
 * Split-K (page "10. Tensor Cores, ...", section "When shape alone can't fix
 * wave efficiency") writes fp32 partial sums into scratch and combines them
 * in a second kernel, summing slices in ascending order.  The persistent
 * mode (same section) launches S*b workgroups that loop over the work units.
 * Scratch is library-owned here (allocated on first use per device, grown
 * when needed, freed at unload).  The MX dtypes need block scales, which
 * only gemm355_gemm_ex takes: here they fail with EINVAL (unless M, N or K
 * is 0).
 * Errors: EINVAL, EALIGN, EUNSUPPORTED, ENOMEM, EHIP as listed above.
 */
GEMM355_API gemm355_status gemm355_gemm(int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda,
                            const void *B, int64_t ldb,
                            void *C, int64_t ldc,
                            gemm355_dtype dtype, gemm355_layout layout,
                            int32_t split_k, int32_t persistent, void *stream);

/*
 * gemm355_gemm_ex -- the same operation with the full argument set: a strided
 * batch of independent products in one launch, per-entry fp32 scales
 * (alpha_g = scale_a[g] * scale_b[g]), a forced tile, and caller-provided
 * scratch (needs at least plan.workspace_bytes; ENOMEM otherwise).
 * The batch strides must keep entries from overlapping C with A or B.
 * MX dtypes: the block scales are first regrouped on the device into the
 * scratch (one dword per row and K-tile of 128 values, K-tile-major), then
 * the main loop stages them through LDS beside the operand tiles and feeds
 * them to the scaled matrix instruction.
 */
GEMM355_API gemm355_status gemm355_gemm_ex(const gemm355_args *args, void *stream);

/*
 * gemm355_gemm_noalloc -- gemm355_gemm_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): it calls no hipMalloc, hipFree or other
 * allocating routine.  Same arguments, plan, kernels and results as
 * gemm355_gemm_ex, except that the scratch (split-K partial sums, repacked
 * operands, regrouped block scales; plan.workspace_bytes) comes from a
 * fixed array of 64 MiB (67,108,864 bytes) in each device's memory,
 * reserved when the library is loaded and held until the process ends;
 * its device address is looked up on the first call on each device.
 *   args->workspace must be NULL and workspace_bytes 0 (EINVAL otherwise).
 *   ETOOBIG if plan.workspace_bytes exceeds the fixed size (nothing is
 *   launched; a smaller split_k or another tile brings the plan under it).
 * Every call on one device uses that device's one array, and a call leaves
 * its contents behind (nothing in it needs to start at zero: every kernel
 * writes the scratch it later reads).  Calls that overlap in time on one
 * device race on the array and may corrupt each other's results: calls on
 * different streams must be ordered by the caller.  Calls on one stream,
 * from any number of threads, enqueue call by call and are safe.
 * Errors otherwise as gemm355_gemm_ex.
 */
GEMM355_API gemm355_status gemm355_gemm_noalloc(const gemm355_args *args, void *stream);

/*
 * gemm355_plan -- what gemm355_gemm_ex would do with `args` (pointers are
 * only inspected for alignment, never dereferenced).  Pure host arithmetic;
 * needs no device when args->cus > 0.  The fields are the quantities of
 * page "10. Tensor Cores, shapes, and tile alignment": the tile grid G and
 * wave efficiency (section "Shape the operation", the tile-count and
 * wave-efficiency equations), the padded sizes and padding efficiency
 * (section "Padding efficiency"), the split-K factor and the persistent grid
 * (section "When shape alone can't fix wave efficiency"), and the resident
 * workgroups per compute unit b (page "Grid 24 is not headroom", section
 * "The question I never asked": residency is the minimum over shared memory
 * and registers).
 * Errors: EINVAL / EALIGN / EUNSUPPORTED as gemm355_gemm_ex would return
 * them; EHIP only when args->cus == 0 and the device query fails.
 */
GEMM355_API gemm355_status gemm355_plan(const gemm355_args *args, gemm355_plan_t *out);

/*
 * gemm355_set_scratch_limit -- cap on the scratch the library allocates for
 * itself (page "10. Tensor Cores, ...", section "When shape alone can't fix
 * wave efficiency": split-K's partial sums go to a buffer of their own,
 * combined by a second pass; repacked rows and regrouped block scales use
 * the same buffer).  A call of gemm355_gemm, gemm355_gemm_ex without a
 * workspace, gemm355_conv2d or gemm355_quantize whose plan needs more than
 * `bytes` returns ENOMEM before anything is launched, and a buffer is
 * never grown past the cap; buffers already larger are kept until unload.
 * Calls with a caller workspace and gemm355_gemm_noalloc are not affected.
 * UINT64_MAX (the default) means no cap; 0 refuses every call that needs
 * scratch.  The previous cap goes to *previous (may be NULL).  Process-wide,
 * for every device; thread-safe.  Never fails.
 */
GEMM355_API gemm355_status gemm355_set_scratch_limit(uint64_t bytes, uint64_t *previous);

/*
 * Wave efficiency G / (ceil(G/(S*b)) * S * b) for G tiles on S compute units
 * holding b workgroups each (page "10. Tensor Cores, ...", section "Shape the
 * operation", wave-efficiency equation).  Returns the binary64 value nearest
 * the exact rational, or NaN if G < 1, S < 1 or b < 1.
 */
GEMM355_API double gemm355_eta_wave(int64_t G, int32_t S, int32_t b);

/*
 * Padding efficiency MNK / (M'N'K') with X' = ceil(X/T_X)*T_X (section
 * "Padding efficiency" of the same page).  Returns the binary64 value nearest
 * the exact rational, or NaN if any argument is < 1.
 */
GEMM355_API double gemm355_eta_pad(int64_t M, int64_t N, int64_t K,
                       int64_t T_M, int64_t T_N, int64_t T_K);

/*
 * K-tile range [*begin, *end) of split-K slice i when nK K-tiles are cut into
 * s slices: begin = floor(i*nK/s), end = floor((i+1)*nK/s).  Split-K cuts
 * the K loop of every tile into slices whose partial sums go to a separate
 * buffer and are combined afterwards (page "10. Tensor Cores, shapes, and
 * tile alignment", section "When shape alone can't fix wave efficiency");
 * the page does not say where the cuts fall, and this even partition (slice
 * sizes differ by at most one K-tile) is the library's reading.
 * begin and end are host pointers, written on success.
 * EINVAL unless nK >= 0, s >= 1, 0 <= i < s and both pointers are non-NULL.
 */
GEMM355_API gemm355_status gemm355_kslice(int64_t nK, int32_t s, int32_t i,
                              int64_t *begin, int64_t *end);

/*
 * Work unit u of a plan, decoded by the same function the kernels use:
 * batch entry, tile row and column, and K-tile range (host pointers, written
 * on success).  The persistent grid of page "10. Tensor Cores, shapes, and
 * tile alignment" (section "When shape alone can't fix wave efficiency")
 * loops its workgroups over such a queue: workgroup w takes units w, w + P,
 * w + 2P, ... of a grid of P.  Errors: those of gemm355_plan, and EINVAL if
 * u is out of range or an output pointer is NULL.  (Host-side view of the
 * tile queue, for inspection and tests.)
 */
GEMM355_API gemm355_status gemm355_unit(const gemm355_args *args, int64_t u,
                            int64_t *batch, int64_t *tile_m, int64_t *tile_n,
                            int64_t *kt_begin, int64_t *kt_end);

/* Number of entries in the tile table, and one entry's parameters: the
 * tile shape T_M x T_N x T_K of the tile-count and padding equations (page
 * "10. Tensor Cores, shapes, and tile alignment", sections "Shape the
 * operation" and "Padding efficiency") and the on-chip resources that fix
 * how many workgroups a compute unit holds (page "Grid 24 is not headroom",
 * section "The question I never asked").
 * dtype_class: 0 = bf16 inputs, 1 = 8-bit inputs (E4M3 and/or E5M2), 2 =
 * block-scaled 8-bit inputs (the MX 8-bit dtypes), 3 = block-scaled FP4
 * inputs, 4 = block-scaled FP6 inputs; T_K counts elements; stages: LDS
 * ring depth; waves: wavefronts per workgroup; lds_bytes: LDS per
 * workgroup; b_max: resident workgroups per compute unit from the LDS,
 * register and wavefront-slot limits; op: 0 matrix product, 1 convolution
 * (gemm355_conv2d); schedule: the copy schedule of the main loop (0: a
 * K-tile's copies in the last K-step of the tile `stages` before; 1: spread
 * over the K-steps, 3 or more stages; 2: fragments two K-steps ahead, copies
 * over the last two K-steps; 3: producer wavefronts issue every copy; 4: as
 * 0 with A's fragments single-buffered; 5: as 0 with B's ring one stage
 * deeper than A's, B's copies in the first K-step, so lds_bytes holds
 * stages A tiles and stages + 1 B tiles; 6: schedule 5 in a ping-pong loop,
 * the two block rows of wavefronts alternating phases of MFMAs only and of
 * fragment reads and copies, one phase apart).  Outputs are host pointers; NULL
 * ones are skipped.  EINVAL if tile is not in [0, gemm355_num_tiles()). */
GEMM355_API int32_t gemm355_num_tiles(void);
GEMM355_API gemm355_status gemm355_tile_info(int32_t tile, int32_t *dtype_class,
                                 int32_t *T_M, int32_t *T_N, int32_t *T_K,
                                 int32_t *stages, int32_t *waves,
                                 int32_t *lds_bytes, int32_t *b_max, int32_t *op,
                                 int32_t *schedule);

/* Workgroups of a tile's main-loop kernel that fit on one compute unit of
 * the current device, as the HIP runtime reports it
 * (hipOccupancyMaxActiveBlocksPerMultiprocessor at the tile's workgroup
 * size: 64 threads per wavefront): the runtime's side of the residency
 * arithmetic of page "Grid 24 is not headroom", section "The question I
 * never asked", against which b_max of gemm355_tile_info is checked.
 * *blocks_per_cu is a host pointer.  EINVAL for an unknown tile or a NULL
 * pointer; needs a device, EHIP otherwise. */
GEMM355_API gemm355_status gemm355_tile_occupancy(int32_t tile, int32_t *blocks_per_cu);

/*
 * gemm355_quantize -- per-tensor scaling of `batch` tensors of n elements each
 * to an 8-bit format, on the device (page "10. Tensor Cores, ...", section
 * "Practical shape sweep": the quantisation is part of an 8-bit product's
 * measured cost).  For tensor g (elements x[g*n .. g*n + n - 1]):
 *     amax  = max_i |x_i|                       (exact)
 *     s     = amax / F  in fp32, rounded to nearest (s = 1 if amax == 0),
 *             F = 448 (E4M3) or 57344 (E5M2)
 *     q_i   = the format's code nearest to min(max(x_i / s, -F), F), the
 *             quotient x_i / s rounded to nearest in fp32 first; ties go to
 *             the code with an even mantissa
 * so that x_i ~ s * dec(q_i): s is the dequantisation factor to pass as
 * scale_a or scale_b of gemm355_gemm_ex.
 *   x:     device, batch*n elements of `src` (fp32 or bf16), finite.
 *   q:     device, batch*n bytes (codes of `fmt`), written.
 *   scale: device fp32 [batch], written (s of each tensor).
 *   n >= 0, batch >= 1; n == 0 writes scale[g] = 1 and nothing else.
 * Two kernels on `stream`: per-block maxima into library-owned scratch, then
 * each block reduces its tensor's maxima (max is exact in any order), forms
 * s and quantises its share.  x may not overlap q or scale (EINVAL).
 * Errors: EINVAL (sizes, enums, null pointers, overlap), EALIGN (x not
 * aligned to its element size, scale not 4-byte aligned), EUNSUPPORTED
 * (n * batch >= 2^40), ENOMEM, EHIP.
 */
GEMM355_API gemm355_status gemm355_quantize(const void *x, int64_t n, int64_t batch, gemm355_src src,
                                gemm355_fp8 fmt, void *q, float *scale, void *stream);

/*
 * Two-dimensional convolution as an implicit matrix product (page "The
 * Tensor Core": convolutions reduce to GEMM; page "Grid 24 is not headroom"
 * profiles a convolution kernel beside the GEMM).  Cross-correlation, as in
 * deep-learning frameworks (the filter is not flipped):
 *
 *   y[n][p][q][k] = sum_{r, s, c} x[n][p*stride_h - pad_h + r*dil_h]
 *                                   [q*stride_w - pad_w + s*dil_w][c] * w[k][r][s][c]
 *
 * with x read as zero outside its H x W extent.  Layouts (dense): x NHWC,
 * w KRSC, y NPQK with P = (H + 2 pad_h - dil_h (R - 1) - 1) / stride_h + 1
 * and Q likewise.  It is the product C = A B with M = N P Q output pixels,
 * N = K output channels and K = R S C: row (n, p, q) of A gathers the R x S
 * input pixels of the window, a column of B is one filter, C is y.  The
 * main loop forms A's addresses from the window instead of reading an
 * im2col copy.
 *   dtype: GEMM355_BF16_F32 or GEMM355_BF16_BF16 (EUNSUPPORTED otherwise).
 *   C must be a multiple of 64 (one K-tile is 64 channels of one filter
 *   tap), x and w 16-byte aligned, and x below 2 GiB (EUNSUPPORTED
 *   otherwise).
 *   split_k, persistent, tile, cus, workspace: as in gemm355_args (tile
 *   must name a convolution tile).
 * y must not overlap x or w (EINVAL).  Sizes must be positive, strides and
 * dilations >= 1, pads >= 0 and P, Q >= 1 (EINVAL).
 */
typedef struct gemm355_conv_args {
    int64_t N, H, W, C;          /* input images, NHWC                       */
    int64_t K, R, S;             /* filters, KRSC                            */
    int64_t pad_h, pad_w;
    int64_t stride_h, stride_w;
    int64_t dil_h, dil_w;
    const void *x;               /* device, N*H*W*C elements                  */
    const void *w;               /* device, K*R*S*C elements                  */
    void *y;                     /* device, N*P*Q*K elements of the output
                                    type, written                            */
    gemm355_dtype dtype;
    int32_t split_k, persistent, tile, cus;
    void *workspace;
    size_t workspace_bytes;
} gemm355_conv_args;

GEMM355_API gemm355_status gemm355_conv2d(const gemm355_conv_args *args, void *stream);

/* The plan of that convolution's implicit product (M = N P Q, N = K,
 * K = R S C; P and Q follow from the arguments): the same fields as
 * gemm355_plan (tile grid, wave and padding efficiency, split and
 * persistence, as defined on page "10. Tensor Cores, ...", sections "Shape
 * the operation", "Padding efficiency" and "When shape alone can't fix wave
 * efficiency").  Host arithmetic only; x, w and y are only inspected for
 * alignment.  out is a host pointer, written on success.  Errors: the
 * argument errors of gemm355_conv2d, EINVAL for a NULL out. */
GEMM355_API gemm355_status gemm355_conv2d_plan(const gemm355_conv_args *args, gemm355_plan_t *out);

/* Output extent of that convolution (the window positions of the
 * cross-correlation that page "The Tensor Core" lowers to a matrix product):
 * *P = (H + 2 pad_h - dil_h (R - 1) - 1)
 * / stride_h + 1 and *Q likewise along W (the window positions that fit in
 * the padded image), as gemm355_conv2d uses them to size y.  Host
 * arithmetic only; x, w and y are not inspected.  P and Q are host
 * pointers, written on success.  Errors: EINVAL / EUNSUPPORTED for the
 * shape arguments exactly as gemm355_conv2d reports them, EINVAL for NULL
 * pointers. */
GEMM355_API gemm355_status gemm355_conv2d_out_size(const gemm355_conv_args *args, int64_t *P, int64_t *Q);

/* Static description of a status code (this library's own codes; no
 * passage of the pages defines them).  Never NULL: unknown codes get a
 * generic description. */
GEMM355_API const char *gemm355_status_string(gemm355_status status);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_H */
