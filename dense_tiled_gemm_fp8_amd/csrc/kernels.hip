/*
 * kernels.hip -- gfx950 kernels of libgemm355.
 *
 *   gemm_tile_kernel  the MFMA main loop over work units (tile x K-range):
 *                     LDS-staged A/B tiles in a two-stage ring fed by
 *                     direct-to-LDS buffer loads, fp32 accumulators,
 *                     epilogue to C or to a split-K partial slot
 *   reduce_kernel     the split-K combine: sums a tile's partial slots in
 *                     ascending slice order, scales, converts, stores C
 *   pack_kernel       repacks an operand into the K-contiguous, 16-byte
 *                     aligned layout the main loop reads (other layouts,
 *                     misaligned rows, K not a multiple of 16 bytes)
 *   zero_kernel       C = 0 for K == 0
 *
 * Source pages: "10. Tensor Cores, shapes, and tile alignment" (tile grid,
 * split-K, persistent loop) and "The Tensor Core" (stage A and B tiles in
 * on-chip memory once and feed many matrix-unit operations from them; low
 * precision inputs with a wide accumulator).
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "sched.h"
#include "tiles.h"

namespace g355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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
constexpr int kRowBytes = 128;           /* K bytes per tile row per stage */

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

/* 32-bit LDS address of a __shared__ object. */
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

/* One direct-to-LDS copy: each lane fetches 16 bytes at voffset from the
 * buffer and the wavefront writes them to LDS at lds .. lds + 1023 (lane l at
 * lds + 16 l).  Issued as inline assembly so that the compiler neither waits
 * for it before unrelated LDS reads nor counts it: completion is awaited
 * explicitly in stage_barrier(). */
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t lds, uint32_t voffset)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
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

__device__ __forceinline__ float unit_alpha(const GemmParams &p, int32_t batch)
{
    float a = 1.0f;
    if (p.scale_a) a *= p.scale_a[batch];
    if (p.scale_b) a *= p.scale_b[batch];
    return a;
}

/*
 * One workgroup of 4 wavefronts (2 x 2) computes a TM x TN tile; wavefront
 * (wm, wn) owns a (TM/2) x (TN/2) block made of 32 x 32 MFMA blocks.
 *
 * LDS layout of one stage of A (B alike): TM rows of 128 bytes (the tile's
 * K-chunk of that row), row r's 16-byte chunk c stored at chunk position
 * c ^ (r % 8), so that the 8 rows read together by a fragment load hit 8
 * different bank groups.  A direct-to-LDS load instruction writes 1024
 * contiguous bytes per wavefront (lane l -> bytes 16 l .. 16 l + 15), i.e.
 * 8 rows; lane l therefore fetches row l / 8, chunk (l % 8) ^ (l / 8).
 */
template <int TM, int TN, bool FP8, int MINB>
__global__ __launch_bounds__(256, MINB) void gemm_tile_kernel(GemmParams p)
{
    constexpr int NW = 4, WN = 2;
    constexpr int WTM = TM / 2, WTN = TN / 2;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_BYTES = TM * kRowBytes, B_BYTES = TN * kRowBytes;
    constexpr int A_LOADS = TM / 8 / NW, B_LOADS = TN / 8 / NW;
    constexpr int KSTEPS = FP8 ? 2 : 4;   /* MFMA K-steps per stage: 64 or 16 deep */
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && FM >= 1 && FN >= 1, "tile too small");

    __shared__ __attribute__((aligned(1024))) uint8_t sA0[A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sA1[A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int prow = lane >> 3;
    const int lchunk = (lane & 7) ^ prow;
    const int frow = lane & 31, hi = lane >> 5, sw = lane & 7;

    int32_t first = blockIdx.x;
    if (p.s.xcd_remap) first = xcd_remap(first, p.s.grid);

    for (int32_t u = first; u < p.s.units; u += p.s.grid) {
        const Unit un = decode_unit(p.s, u);
        const int32_t m0 = un.tile_m * TM, n0 = un.tile_n * TN;
        const i32x4 ra = rsrc_words(p.A + (int64_t)un.batch * p.stride_a + (int64_t)m0 * p.lda);
        const i32x4 rb = rsrc_words(p.B + (int64_t)un.batch * p.stride_b + (int64_t)n0 * p.ldb);

        uint32_t aoff[A_LOADS], boff[B_LOADS];
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int r = (i * NW + wave) * 8 + prow;
            aoff[i] = (m0 + r < p.M) ? (uint32_t)(r * p.lda + lchunk * 16) : kOOB;
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int r = (i * NW + wave) * 8 + prow;
            boff[i] = (n0 + r < p.N) ? (uint32_t)(r * p.ldb + lchunk * 16) : kOOB;
        }

        auto issue = [&](uint8_t *sa, uint8_t *sb, int32_t kt) {
            const uint32_t kb = (uint32_t)kt * kRowBytes;
            const bool kval = (int32_t)(kb + lchunk * 16) < p.Kb;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i)
                dma16(ra, lds_addr(sa) + (i * NW + wave) * 1024, kval ? aoff[i] + kb : kOOB);
#pragma unroll
            for (int i = 0; i < B_LOADS; ++i)
                dma16(rb, lds_addr(sb) + (i * NW + wave) * 1024, kval ? boff[i] + kb : kOOB);
        };

        f32x16 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x16{};

        auto compute = [&](const uint8_t *sa, const uint8_t *sb) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                if constexpr (!FP8) {
                    const int chunk = (2 * ks + hi) ^ sw;
                    bf16x8 a[FM], b[FN];
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        a[i] = *(const bf16x8 *)(sa + (wm * WTM + i * 32 + frow) * kRowBytes + chunk * 16);
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        b[j] = *(const bf16x8 *)(sb + (wn * WTN + j * 32 + frow) * kRowBytes + chunk * 16);
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                } else {
                    const int c0 = (4 * ks + 2 * hi) ^ sw, c1 = (4 * ks + 2 * hi + 1) ^ sw;
                    i32x8 a[FM], b[FN];
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const uint8_t *row = sa + (wm * WTM + i * 32 + frow) * kRowBytes;
                        const i32x4 lo = *(const i32x4 *)(row + c0 * 16);
                        const i32x4 up = *(const i32x4 *)(row + c1 * 16);
                        a[i] = i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
                    }
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const uint8_t *row = sb + (wn * WTN + j * 32 + frow) * kRowBytes;
                        const i32x4 lo = *(const i32x4 *)(row + c0 * 16);
                        const i32x4 up = *(const i32x4 *)(row + c1 * 16);
                        b[j] = i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
                    }
                    /* format fields 0/0: both operands E4M3; zero scales select
                     * the unscaled instruction */
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
                }
            }
        };

        /* Two-stage ring: stage 0 holds even K-tiles of the unit, stage 1
         * odd ones.  The copy of tile k+1 is issued before tile k's MFMAs;
         * one barrier per K-tile both publishes the copy and retires the
         * stage that the next copy overwrites. */
        const int32_t nkt = un.kt_end - un.kt_begin;
        if (nkt > 0) {
            int32_t kt = un.kt_begin;
            issue(sA0, sB0, kt);
            stage_barrier();
            for (int32_t pair = 0; pair < (nkt >> 1); ++pair) {
                issue(sA1, sB1, kt + 1);
                compute(sA0, sB0);
                stage_barrier();
                if (kt + 2 < un.kt_end) issue(sA0, sB0, kt + 2);
                compute(sA1, sB1);
                stage_barrier();
                kt += 2;
            }
            if (nkt & 1) {
                compute(sA0, sB0);
                stage_barrier();
            }
        }

        /* Epilogue.  Accumulator layout of a 32 x 32 MFMA block: lane l holds
         * column l % 32, register 4 g + r holds row 8 g + 4 (l / 32) + r.
         * Stores go through a buffer resource based at the tile's corner: the
         * lane's column and row group in the VGPR offset, the register's row
         * in the scalar offset; elements outside M x N get VGPR offset kOOB
         * and are dropped.  The lane index is re-materialised here so the
         * compiler cannot hoist the epilogue's addresses above the main loop
         * and hold them in registers across it. */
        int lv = threadIdx.x;
        asm volatile("" : "+v"(lv));
        const int el = lv & 63, ecol = el & 31, ehi = el >> 5;
        if (un.slot >= 0) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.ws + (int64_t)un.slot * (TM * TN));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const uint32_t voff =
                        (uint32_t)(((wm * WTM + i * 32 + ehi * 4) * TN + wn * WTN + j * 32 + ecol) * 4);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        /* copy the element out first: a bit_cast applied to
                         * a vector subscript directly was lowered to element
                         * 0 for every e */
                        const float v = acc[i][j][e];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rw, voff,
                                                              ((e >> 2) * 8 + (e & 3)) * TN * 4, 0);
                    }
                }
        } else {
            const float alpha = unit_alpha(p, un.batch);
            const int esz = p.out_bf16 ? 2 : 4;
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(
                (const uint8_t *)p.C + ((int64_t)un.batch * p.stride_c + (int64_t)m0 * p.ldc + n0) * esz);
            const int32_t mrem = p.M - m0, nrem = p.N - n0;
            const int32_t ldcb = (int32_t)p.ldc * esz;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = wn * WTN + j * 32 + ecol;
                    const int row0 = wm * WTM + i * 32 + ehi * 4;
                    const uint32_t voff = (uint32_t)(row0 * ldcb + col * esz);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int dr = (e >> 2) * 8 + (e & 3);
                        const bool ok = (row0 + dr < mrem) && (col < nrem);
                        const float v = alpha * acc[i][j][e];
                        if (p.out_bf16)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                __builtin_bit_cast(uint16_t, (__bf16)v), rc, ok ? voff : kOOB,
                                dr * ldcb, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b32(
                                __builtin_bit_cast(uint32_t, v), rc, ok ? voff : kOOB, dr * ldcb, 0);
                    }
                }
        }
    }
}

/*
 * Split-K combine.  Block x = one split tile (uniform split: tile x; tail:
 * tail tile x), 256 threads x 4 consecutive elements per step over the
 * TM x TN partial tile.  Slices are summed in ascending order in fp32.
 */
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams r)
{
    const int32_t q = blockIdx.x;
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
    float alpha = 1.0f;
    if (r.scale_a) alpha *= r.scale_a[un.batch];
    if (r.scale_b) alpha *= r.scale_b[un.batch];
    const int64_t tile_elems = (int64_t)r.TM * r.TN;
    const float *src = r.ws + (int64_t)q * nsl * tile_elems;
    const int64_t cbase = (int64_t)un.batch * r.stride_c;
    for (int64_t e = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 4; e < tile_elems;
         e += (int64_t)gridDim.y * blockDim.x * 4) {
        f32x4 s = *(const f32x4 *)(src + e);
        for (int32_t i = 1; i < nsl; ++i) s += *(const f32x4 *)(src + i * tile_elems + e);
        const int32_t row = m0 + (int32_t)(e / r.TN);
        const int32_t col0 = n0 + (int32_t)(e % r.TN);
        if (row >= r.M) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int32_t col = col0 + c;
            if (col < r.N) {
                const float v = alpha * s[c];
                const int64_t idx = cbase + (int64_t)row * r.ldc + col;
                if (r.out_bf16)
                    ((__bf16 *)r.C)[idx] = (__bf16)v;
                else
                    ((float *)r.C)[idx] = v;
            }
        }
    }
}

/*
 * Repack one operand to K-contiguous rows of ldd_bytes (a multiple of 16),
 * zero-filled beyond K.  Source element (row, k) of batch entry g is at
 * src[g*stride + (kmajor ? row*ld + k : k*ld + row)] (elements of esize
 * bytes).  One thread per 16-byte output chunk.
 */
__global__ __launch_bounds__(256) void pack_kernel(PackParams pk)
{
    const int64_t chunks_per_row = pk.ldd_bytes / 16;
    const int64_t total = (int64_t)pk.batch * pk.rows * chunks_per_row;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t g = t / ((int64_t)pk.rows * chunks_per_row);
        const int64_t rem = t - g * pk.rows * chunks_per_row;
        const int64_t row = rem / chunks_per_row;
        const int64_t ch = rem - row * chunks_per_row;
        uint8_t out[16];
        const int per = 16 / pk.esize;
        for (int e = 0; e < per; ++e) {
            const int64_t k = ch * per + e;
            uint16_t v = 0;
            if (k < pk.K) {
                const int64_t idx = g * pk.stride + (pk.kmajor ? row * pk.ld + k : k * pk.ld + row);
                v = pk.esize == 2 ? ((const uint16_t *)pk.src)[idx] : ((const uint8_t *)pk.src)[idx];
            }
            if (pk.esize == 2) {
                out[2 * e] = (uint8_t)(v & 0xFF);
                out[2 * e + 1] = (uint8_t)(v >> 8);
            } else {
                out[e] = (uint8_t)v;
            }
        }
        i32x4 w;
        __builtin_memcpy(&w, out, 16);
        *(i32x4 *)(pk.dst + g * pk.dst_stride_bytes + row * pk.ldd_bytes + ch * 16) = w;
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

template <int TM, int TN, bool FP8, int MINB>
static hipError_t launch_tile(const GemmParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_tile_kernel<TM, TN, FP8, MINB>), dim3(p.s.grid), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm(int32_t tile, const GemmParams &p, hipStream_t stream)
{
    switch (tile) {
    case 0: return launch_tile<256, 256, false, 1>(p, stream);
    case 1: return launch_tile<128, 128, false, 2>(p, stream);
    case 2: return launch_tile<64, 64, false, 4>(p, stream);
    case 3: return launch_tile<256, 256, true, 1>(p, stream);
    case 4: return launch_tile<128, 128, true, 2>(p, stream);
    case 5: return launch_tile<64, 64, true, 4>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

const void *gemm_kernel_symbol(int32_t tile)
{
    switch (tile) {
    case 0: return (const void *)gemm_tile_kernel<256, 256, false, 1>;
    case 1: return (const void *)gemm_tile_kernel<128, 128, false, 2>;
    case 2: return (const void *)gemm_tile_kernel<64, 64, false, 4>;
    case 3: return (const void *)gemm_tile_kernel<256, 256, true, 1>;
    case 4: return (const void *)gemm_tile_kernel<128, 128, true, 2>;
    case 5: return (const void *)gemm_tile_kernel<64, 64, true, 4>;
    default: return nullptr;
    }
}

hipError_t launch_reduce(const ReduceParams &r, int32_t tiles, hipStream_t stream)
{
    const int64_t elems = (int64_t)r.TM * r.TN;
    int32_t ychunks = (int32_t)((elems / 4 + 255) / 256);
    /* enough blocks to cover the device even for one tile */
    if ((int64_t)tiles * ychunks > 4096) ychunks = (int32_t)((4096 + tiles - 1) / tiles);
    if (ychunks < 1) ychunks = 1;
    hipLaunchKernelGGL(reduce_kernel, dim3(tiles, ychunks), dim3(256), 0, stream, r);
    return hipGetLastError();
}

hipError_t launch_pack(const PackParams &pk, hipStream_t stream)
{
    const int64_t total = (int64_t)pk.batch * pk.rows * (pk.ldd_bytes / 16);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, pk);
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
