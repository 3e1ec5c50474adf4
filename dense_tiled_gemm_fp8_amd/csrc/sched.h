/*
 * sched.h -- work units of the tiled product and their decoding, shared by
 * the host planner and the kernels (one definition, so the host's view of the
 * tile queue is exactly the device's).
 *
 * A work unit is one output tile over one range of K-tiles.  Three shapes of
 * queue (page "10. Tensor Cores, shapes, and tile alignment", sections "Shape
 * the operation" and "When shape alone can't fix wave efficiency"):
 *   - whole tiles: unit u is tile u;
 *   - uniform split-K: every tile is cut into `split` K-slices, slice-major
 *     (unit u -> slice u / G_tot, tile u % G_tot), partial sums go to scratch;
 *   - persistent with a split tail: the first `units_main` units are whole
 *     tiles; the remaining `tail_tiles` tiles (those that would form a partial
 *     last round) are cut into `tail_split` K-slices each, slice-major.
 * K-slice i of s over nK K-tiles is [floor(i nK / s), floor((i+1) nK / s)).
 *
 * Tile order inside one batch entry is a grouped raster: bands of `group_m`
 * tile rows, column-major inside a band, so that consecutive units share
 * A row panels and B column panels.  Batch entries follow one another.
 */
#ifndef GEMM355_SCHED_H
#define GEMM355_SCHED_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g355 {

struct Sched {
    int32_t tiles_m, tiles_n;     /* tiles per batch entry along M and N    */
    int32_t tiles_per_batch;      /* tiles_m * tiles_n                      */
    int32_t batch;
    int32_t group_m;              /* raster band height in tiles (>= 1)     */
    int32_t nK;                   /* K-tiles                                */
    int32_t split;                /* uniform split (1 = none)               */
    int32_t units_main;           /* units before the split tail            */
    int32_t tail_first;           /* first tail tile (global tile index)    */
    int32_t tail_tiles;           /* tiles in the split tail (0 = none)     */
    int32_t tail_split;           /* slices per tail tile                   */
    int32_t units;                /* all units                              */
    int32_t grid;                 /* launched workgroups                    */
    int32_t xcd_remap;            /* 1: give each XCD a contiguous block    */
};

struct Unit {
    int32_t tile;                 /* global tile index                      */
    int32_t batch, tile_m, tile_n;
    int32_t kt_begin, kt_end;     /* K-tile range                           */
    int32_t slot;                 /* partial-sum slot, -1 = write C         */
};

/* floor(i * nK / s) in 32-bit unsigned arithmetic; the planner keeps
 * nK < 2^23 and s <= 256, so the product cannot overflow. */
__host__ __device__ inline int32_t kslice_begin(int32_t nK, int32_t s, int32_t i)
{
    return (int32_t)(((uint32_t)i * (uint32_t)nK) / (uint32_t)s);
}

__host__ __device__ inline void tile_coords(const Sched &s, int32_t t, Unit &o)
{
    o.tile = t;
    o.batch = t / s.tiles_per_batch;
    const int32_t r = t - o.batch * s.tiles_per_batch;
    const int32_t per_band = s.group_m * s.tiles_n;
    const int32_t band = r / per_band;
    const int32_t first_m = band * s.group_m;
    const int32_t rows = (s.tiles_m - first_m) < s.group_m ? (s.tiles_m - first_m) : s.group_m;
    const int32_t in = r - band * per_band;
    o.tile_m = first_m + in % rows;
    o.tile_n = in / rows;
}

__host__ __device__ inline Unit decode_unit(const Sched &s, int32_t u)
{
    Unit o;
    int32_t t, slice, nsl;
    if (u < s.units_main) {
        if (s.split > 1) {
            const int32_t gt = s.tiles_per_batch * s.batch;
            slice = u / gt;
            t = u - slice * gt;
            nsl = s.split;
            o.slot = t * s.split + slice;
        } else {
            t = u;
            slice = 0;
            nsl = 1;
            o.slot = -1;
        }
    } else {
        const int32_t j = u - s.units_main;
        slice = j / s.tail_tiles;
        const int32_t q = j - slice * s.tail_tiles;
        t = s.tail_first + q;
        nsl = s.tail_split;
        o.slot = q * s.tail_split + slice;
    }
    tile_coords(s, t, o);
    o.kt_begin = kslice_begin(s.nK, nsl, slice);
    o.kt_end = kslice_begin(s.nK, nsl, slice + 1);
    return o;
}

/* Workgroups are handed to the 8 XCDs round-robin (w -> XCD w % 8), each XCD
 * with its own L2.  Renumber so that XCD x owns a contiguous block of
 * logical ids: neighbouring units (which share operand panels) then run
 * under one L2.  A bijection on [0, grid). */
__host__ __device__ inline int32_t xcd_remap(int32_t w, int32_t grid)
{
    const int32_t x = w & 7, j = w >> 3, q = grid >> 3, r = grid & 7;
    return x * q + (x < r ? x : r) + j;
}

} /* namespace g355 */

#endif
