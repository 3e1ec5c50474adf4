/*
 * tiles.h -- the tile-shape table.
 *
 * Each entry is one instantiation of the MFMA main loop: output tile
 * T_M x T_N, K-step T_K, LDS ring depth, wavefront grid, and the resources
 * that fix how many workgroups a compute unit holds (page "Grid 24 is not
 * headroom", section "The question I never asked": resident workgroups are
 * the minimum over shared memory and the register file).
 *
 * An entry stages RB bytes of K per tile row per stage (RB = 128: 64 bf16 or
 * 128 E4M3 values; RB = 64: half that), so the LDS layout and the copy
 * pattern are the same for both input types; `stages` K-tiles are in the
 * ring.
 */
#ifndef GEMM355_TILES_H
#define GEMM355_TILES_H

#include <stdint.h>

namespace g355 {

struct TileCfg {
    int32_t dtype_class;   /* 0 bf16 inputs, 1 8-bit inputs, 2 8-bit inputs
                              with E8M0 block scales (MX), 3 FP4 inputs
                              with E8M0 block scales, 4 FP6 inputs with
                              E8M0 block scales                             */
    int32_t TM, TN, TK;    /* TK in elements                                 */
    int32_t row_bytes;     /* RB: LDS bytes per tile row per stage (FP6 uses
                              96 of 128)                                    */
    int32_t stages;
    int32_t waves_m, waves_n;
    int32_t spread;        /* copy schedule: 0 copies of a K-tile in the last
                              K-step of the tile STAGES before; 1 spread
                              over the K-steps of the tile before (ring of
                              >= 3 stages); 2 fragments read two K-steps
                              ahead and copies over the last two K-steps of
                              the tile two before (2 stages, 4 K-steps);
                              3 warp specialisation: four more wavefronts
                              (one per SIMD) issue every copy, STAGES-1
                              K-tiles ahead, and the waves_m x waves_n MFMA
                              wavefronts only read LDS (3 stages or more);
                              4 as 0 with A's fragments read in place, one
                              row at a time (bf16); 5 as 0 with B's ring
                              one stage deeper, B's copies of a K-tile in
                              the first K-step two tiles before and A's in
                              the last (2 stages of 2 K-steps); 6 as 5 in
                              a ping-pong loop: the two block rows of
                              wavefronts alternate phases of MFMAs only and
                              of fragment reads and copies, one phase apart
                              (2 x 4 wavefronts)                            */
    int32_t mfma;          /* MFMA block edge: 32 (32x32) or 16 (16x16)      */
    int32_t lds_bytes;     /* stages * (TM + TN) * RB, plus 4 (8 for FP4)
                              bytes of block scales per row and stage for
                              MX; one more B stage with copy schedules 5
                              and 6                                         */
    int32_t min_blocks;    /* workgroups per CU the kernel is compiled for   */
    int32_t vgpr_budget;   /* 512 / (min_blocks * tile_waves / 4): registers
                              per lane one wave may hold                    */
    /* planning prior: fraction of a compute unit's dense MFMA peak (at the
     * 2.4 GHz peak clock) the tile sustains with 1, 2, 3, 4 of its
     * workgroups resident on the unit, board power limit included */
    float mfma_eff[4];
    /* planning prior: the tile's rate of algorithmic bytes, as a multiple
     * of the 5 TB/s planning rate, when the product is bound by memory */
    float stream_eff;
    int32_t op;            /* 0 matrix product; 1 convolution (A gathered
                              from NHWC images, K-tiles of 64 channels of
                              one filter tap); omitted entries are 0       */
};

/* gfx950 compute-unit resources used by the occupancy arithmetic. */
constexpr int32_t kLdsPerCu = 160 * 1024;
constexpr int32_t kRegsPerLanePerSimd = 512;
constexpr int32_t kRegGranule = 8;
constexpr int32_t kSimdsPerCu = 4;
constexpr int32_t kWaveSize = 64;
constexpr int32_t kMaxWavesPerSimd = 8;

constexpr TileCfg kTiles[] = {
    /* bf16, 128-byte K-tiles, 2 stages */
    {0, 256, 256, 64, 128, 2, 2, 2, 0, 32, 2 * (256 + 256) * 128, 1, 512, {0.55f, 0.55f, 0.55f, 0.55f}, 1.16f},
    {0, 128, 128, 64, 128, 2, 2, 2, 0, 32, 2 * (128 + 128) * 128, 2, 256, {0.27f, 0.45f, 0.45f, 0.45f}, 1.16f},
    {0, 64, 64, 64, 128, 2, 2, 2, 0, 32, 2 * (64 + 64) * 128, 4, 128, {0.11f, 0.18f, 0.21f, 0.22f}, 1.16f},
    /* E4M3, 128-byte K-tiles, 2 stages */
    {1, 256, 256, 128, 128, 2, 2, 2, 0, 32, 2 * (256 + 256) * 128, 1, 512, {0.68f, 0.68f, 0.68f, 0.68f}, 1.04f},
    {1, 128, 128, 128, 128, 2, 2, 2, 0, 32, 2 * (128 + 128) * 128, 2, 256, {0.37f, 0.50f, 0.50f, 0.50f}, 0.94f},
    {1, 64, 64, 128, 128, 2, 2, 2, 0, 32, 2 * (64 + 64) * 128, 4, 128, {0.13f, 0.21f, 0.23f, 0.24f}, 1.02f},
    /* 256 x 256 with 64-byte K-tiles and a deeper ring */
    {0, 256, 256, 32, 64, 4, 2, 2, 0, 32, 4 * (256 + 256) * 64, 1, 512, {0.52f, 0.52f, 0.52f, 0.52f}, 1.06f},
    {0, 256, 256, 32, 64, 5, 2, 2, 0, 32, 5 * (256 + 256) * 64, 1, 512, {0.55f, 0.55f, 0.55f, 0.55f}, 1.02f},
    {1, 256, 256, 64, 64, 4, 2, 2, 0, 32, 4 * (256 + 256) * 64, 1, 512, {0.58f, 0.58f, 0.58f, 0.58f}, 1.02f},
    {1, 256, 256, 64, 64, 5, 2, 2, 0, 32, 5 * (256 + 256) * 64, 1, 512, {0.61f, 0.61f, 0.61f, 0.61f}, 1.02f},
    /* 256 x 256 with 8 wavefronts (2 x 4, two per SIMD) */
    {0, 256, 256, 64, 128, 2, 2, 4, 0, 32, 2 * (256 + 256) * 128, 1, 256, {0.58f, 0.58f, 0.58f, 0.58f}, 1.16f},
    {0, 256, 256, 32, 64, 4, 2, 4, 0, 32, 4 * (256 + 256) * 64, 1, 256, {0.53f, 0.53f, 0.53f, 0.53f}, 1.16f},
    {1, 256, 256, 128, 128, 2, 2, 4, 0, 32, 2 * (256 + 256) * 128, 1, 256, {0.63f, 0.63f, 0.63f, 0.63f}, 1.06f},
    {1, 256, 256, 64, 64, 4, 2, 4, 0, 32, 4 * (256 + 256) * 64, 1, 256, {0.66f, 0.66f, 0.66f, 0.66f}, 1.02f},
    /* small tiles with deep rings for streaming (small M, N, long K) */
    {0, 64, 64, 64, 128, 8, 2, 2, 0, 32, 8 * (64 + 64) * 128, 1, 512, {0.11f, 0.11f, 0.11f, 0.11f}, 1.54f},
    {0, 64, 64, 64, 128, 4, 2, 2, 0, 32, 4 * (64 + 64) * 128, 2, 256, {0.11f, 0.18f, 0.18f, 0.18f}, 2.02f},
    {0, 128, 128, 64, 128, 4, 2, 2, 0, 32, 4 * (128 + 128) * 128, 1, 512, {0.34f, 0.34f, 0.34f, 0.34f}, 1.40f},
    {1, 64, 64, 128, 128, 8, 2, 2, 0, 32, 8 * (64 + 64) * 128, 1, 512, {0.13f, 0.13f, 0.13f, 0.13f}, 1.38f},
    {1, 64, 64, 128, 128, 4, 2, 2, 0, 32, 4 * (64 + 64) * 128, 2, 256, {0.13f, 0.21f, 0.21f, 0.21f}, 1.46f},
    {1, 128, 128, 128, 128, 4, 2, 2, 0, 32, 4 * (128 + 128) * 128, 1, 512, {0.37f, 0.37f, 0.37f, 0.37f}, 1.10f},
    /* 64 x 64 with one wavefront (four MFMA blocks per K-step) */
    {0, 64, 64, 64, 128, 2, 1, 1, 0, 32, 2 * (64 + 64) * 128, 4, 512, {0.07f, 0.15f, 0.21f, 0.25f}, 1.00f},
    {0, 64, 64, 64, 128, 4, 1, 1, 0, 32, 4 * (64 + 64) * 128, 2, 512, {0.07f, 0.15f, 0.15f, 0.15f}, 2.50f},
    {1, 64, 64, 128, 128, 2, 1, 1, 0, 32, 2 * (64 + 64) * 128, 4, 512, {0.08f, 0.17f, 0.23f, 0.29f}, 0.88f},
    {1, 64, 64, 128, 128, 4, 1, 1, 0, 32, 4 * (64 + 64) * 128, 2, 512, {0.08f, 0.17f, 0.17f, 0.17f}, 1.50f},
    /* 256 x 256, 64-byte K-tiles, copies spread over the K-steps */
    {0, 256, 256, 32, 64, 4, 2, 2, 1, 32, 4 * (256 + 256) * 64, 1, 512, {0.52f, 0.52f, 0.52f, 0.52f}, 1.12f},
    {0, 256, 256, 32, 64, 5, 2, 2, 1, 32, 5 * (256 + 256) * 64, 1, 512, {0.52f, 0.52f, 0.52f, 0.52f}, 1.10f},
    {0, 256, 256, 32, 64, 4, 2, 4, 1, 32, 4 * (256 + 256) * 64, 1, 256, {0.52f, 0.52f, 0.52f, 0.52f}, 1.16f},
    {0, 256, 256, 32, 64, 5, 2, 4, 1, 32, 5 * (256 + 256) * 64, 1, 256, {0.52f, 0.52f, 0.52f, 0.52f}, 1.16f},
    {1, 256, 256, 64, 64, 4, 2, 2, 1, 32, 4 * (256 + 256) * 64, 1, 512, {0.58f, 0.58f, 0.58f, 0.58f}, 1.12f},
    {1, 256, 256, 64, 64, 5, 2, 2, 1, 32, 5 * (256 + 256) * 64, 1, 512, {0.58f, 0.58f, 0.58f, 0.58f}, 1.04f},
    {1, 256, 256, 64, 64, 4, 2, 4, 1, 32, 4 * (256 + 256) * 64, 1, 256, {0.58f, 0.58f, 0.58f, 0.58f}, 1.18f},
    {1, 256, 256, 64, 64, 5, 2, 4, 1, 32, 5 * (256 + 256) * 64, 1, 256, {0.58f, 0.58f, 0.58f, 0.58f}, 1.16f},
    /* 256 x 256 with 16 wavefronts (4 x 4, four per SIMD, 64 x 64 each) */
    {0, 256, 256, 64, 128, 2, 4, 4, 0, 32, 2 * (256 + 256) * 128, 1, 128, {0.52f, 0.52f, 0.52f, 0.52f}, 1.20f},
    {0, 256, 256, 32, 64, 4, 4, 4, 0, 32, 4 * (256 + 256) * 64, 1, 128, {0.52f, 0.52f, 0.52f, 0.52f}, 1.14f},
    {0, 256, 256, 32, 64, 4, 4, 4, 1, 32, 4 * (256 + 256) * 64, 1, 128, {0.52f, 0.52f, 0.52f, 0.52f}, 1.12f},
    /* 256 x 256 with 16 x 16 MFMA blocks */
    {0, 256, 256, 64, 128, 2, 2, 2, 0, 16, 2 * (256 + 256) * 128, 1, 512, {0.64f, 0.64f, 0.64f, 0.64f}, 1.08f},
    {0, 256, 256, 64, 128, 2, 2, 4, 0, 16, 2 * (256 + 256) * 128, 1, 256, {0.68f, 0.68f, 0.68f, 0.68f}, 1.12f},
    {0, 256, 256, 32, 64, 4, 2, 4, 0, 16, 4 * (256 + 256) * 64, 1, 256, {0.52f, 0.52f, 0.52f, 0.52f}, 1.24f},
    {0, 256, 256, 32, 64, 4, 2, 2, 0, 16, 4 * (256 + 256) * 64, 1, 512, {0.58f, 0.58f, 0.58f, 0.58f}, 1.04f},
    {0, 256, 256, 32, 64, 4, 2, 2, 1, 16, 4 * (256 + 256) * 64, 1, 512, {0.58f, 0.58f, 0.58f, 0.58f}, 1.10f},
    {0, 256, 256, 32, 64, 5, 2, 2, 0, 16, 5 * (256 + 256) * 64, 1, 512, {0.58f, 0.58f, 0.58f, 0.58f}, 1.04f},
    /* 32 x 32 MFMA blocks, fragments read two K-steps ahead, copies over the
     * last two K-steps of each K-tile */
    {0, 256, 256, 64, 128, 2, 2, 2, 2, 32, 2 * (256 + 256) * 128, 1, 512, {0.67f, 0.67f, 0.67f, 0.67f}, 1.04f},
    {0, 256, 256, 64, 128, 2, 2, 4, 2, 32, 2 * (256 + 256) * 128, 1, 256, {0.63f, 0.63f, 0.63f, 0.63f}, 1.12f},
    {0, 128, 128, 64, 128, 2, 2, 2, 2, 32, 2 * (128 + 128) * 128, 2, 256, {0.33f, 0.48f, 0.48f, 0.48f}, 1.12f},
    /* 256 x 128, 3 stages: producer wavefronts (warp specialisation) with
     * 32 x 32 and 16 x 16 blocks and for E4M3, and the same tile with
     * uniform wavefronts for comparison */
    {0, 256, 128, 64, 128, 3, 2, 2, 3, 32, 3 * (256 + 128) * 128, 1, 256, {0.52f, 0.52f, 0.52f, 0.52f}, 1.08f},
    {0, 256, 128, 64, 128, 3, 2, 2, 3, 16, 3 * (256 + 128) * 128, 1, 256, {0.52f, 0.52f, 0.52f, 0.52f}, 1.26f},
    {1, 256, 128, 128, 128, 3, 2, 2, 3, 32, 3 * (256 + 128) * 128, 1, 256, {0.58f, 0.58f, 0.58f, 0.58f}, 1.06f},
    {0, 256, 128, 64, 128, 3, 2, 2, 0, 32, 3 * (256 + 128) * 128, 1, 512, {0.52f, 0.52f, 0.52f, 0.52f}, 1.10f},
    /* block-scaled 8-bit (MX): the 8-bit tiles with the scale dwords of
     * each K-tile in the stage */
    {2, 256, 256, 128, 128, 2, 2, 2, 0, 32, 2 * (256 + 256) * 132, 1, 512, {0.62f, 0.62f, 0.62f, 0.62f}, 1.12f},
    {2, 128, 128, 128, 128, 2, 2, 2, 0, 32, 2 * (128 + 128) * 132, 2, 256, {0.35f, 0.47f, 0.47f, 0.47f}, 1.04f},
    {2, 128, 128, 128, 128, 4, 2, 2, 0, 32, 4 * (128 + 128) * 132, 1, 512, {0.35f, 0.35f, 0.35f, 0.35f}, 1.34f},
    /* block-scaled FP4: 128-byte K-tiles of 256 values, two scale dwords per
     * row and stage */
    {3, 256, 256, 256, 128, 2, 2, 2, 0, 32, 2 * (256 + 256) * 136, 1, 512, {0.62f, 0.62f, 0.62f, 0.62f}, 1.12f},
    {3, 128, 128, 256, 128, 2, 2, 2, 0, 32, 2 * (128 + 128) * 136, 2, 256, {0.35f, 0.47f, 0.47f, 0.47f}, 1.04f},
    {3, 128, 128, 256, 128, 4, 2, 2, 0, 32, 4 * (128 + 128) * 136, 1, 512, {0.35f, 0.35f, 0.35f, 0.35f}, 1.34f},
    /* convolution (bf16): the matrix tiles 0, 1, 2, 36 and 16 with A
     * gathered from the images */
    {0, 256, 256, 64, 128, 2, 2, 2, 0, 32, 2 * (256 + 256) * 128, 1, 512, {0.76f, 0.76f, 0.76f, 0.76f}, 1.16f, 1},
    {0, 128, 128, 64, 128, 2, 2, 2, 0, 32, 2 * (128 + 128) * 128, 2, 256, {0.41f, 0.66f, 0.66f, 0.66f}, 1.82f, 1},
    {0, 64, 64, 64, 128, 2, 2, 2, 0, 32, 2 * (64 + 64) * 128, 4, 128, {0.16f, 0.27f, 0.31f, 0.33f}, 2.36f, 1},
    {0, 256, 256, 64, 128, 2, 2, 4, 0, 16, 2 * (256 + 256) * 128, 1, 256, {0.88f, 0.88f, 0.88f, 0.88f}, 1.42f, 1},
    {0, 128, 128, 64, 128, 4, 2, 2, 0, 32, 4 * (128 + 128) * 128, 1, 512, {0.49f, 0.49f, 0.49f, 0.49f}, 1.46f, 1},
    /* block-scaled FP6: K-tiles of 128 values (96 bytes) staged in 128-byte
     * rows, one scale dword per row and stage */
    {4, 256, 256, 128, 128, 2, 2, 2, 0, 32, 2 * (256 + 256) * 132, 1, 512, {0.62f, 0.62f, 0.62f, 0.62f}, 1.12f},
    {4, 128, 128, 128, 128, 2, 2, 2, 0, 32, 2 * (128 + 128) * 132, 2, 256, {0.35f, 0.47f, 0.47f, 0.47f}, 1.04f},
    {4, 128, 128, 128, 128, 4, 2, 2, 0, 32, 4 * (128 + 128) * 132, 1, 512, {0.35f, 0.35f, 0.35f, 0.35f}, 1.34f},
    /* 16 x 16 blocks with A's fragments read in place (copy schedule 4) */
    {0, 256, 256, 64, 128, 2, 2, 2, 4, 16, 2 * (256 + 256) * 128, 1, 512, {0.52f, 0.52f, 0.52f, 0.52f}, 1.20f},
    /* the 8-wavefront 16 x 16 tile with B's ring a stage deeper (copy
     * schedule 5): the whole 160 KiB of LDS */
    {0, 256, 256, 64, 128, 2, 2, 4, 5, 16, 2 * 256 * 128 + 3 * 256 * 128, 1, 256, {0.70f, 0.70f, 0.70f, 0.70f}, 1.18f},
    /* the 8-bit 256 x 256 tile (4 wavefronts, 32 x 32 blocks) with copy
     * schedule 5 */
    {1, 256, 256, 128, 128, 2, 2, 2, 5, 32, 2 * 256 * 128 + 3 * 256 * 128, 1, 512, {0.70f, 0.70f, 0.70f, 0.70f}, 1.24f},
    /* copy schedule 5 in a ping-pong loop (schedule 6): the bf16 tile 63 and
     * an 8-bit tile of 8 wavefronts with 32 x 32 blocks */
    {0, 256, 256, 64, 128, 2, 2, 4, 6, 16, 2 * 256 * 128 + 3 * 256 * 128, 1, 256, {0.71f, 0.71f, 0.71f, 0.71f}, 1.24f},
    {1, 256, 256, 128, 128, 2, 2, 4, 6, 32, 2 * 256 * 128 + 3 * 256 * 128, 1, 256, {0.66f, 0.66f, 0.66f, 0.66f}, 1.18f},
};
constexpr int32_t kNumTiles = (int32_t)(sizeof(kTiles) / sizeof(kTiles[0]));

/* wavefronts of one workgroup: the MFMA grid plus, with copy schedule 3,
 * one producer per SIMD */
constexpr int32_t tile_waves(const TileCfg &c)
{
    return c.waves_m * c.waves_n + (c.spread == 3 ? kSimdsPerCu : 0);
}

} /* namespace g355 */

#endif
