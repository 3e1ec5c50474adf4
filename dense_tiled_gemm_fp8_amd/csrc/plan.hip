/*
 * plan.hip -- host planner of libgemm355: argument validation, the choice of
 * tile / split-K / persistent schedule, and the exact bookkeeping reported to
 * callers (tile grid G, padded dimensions, wave, padding and schedule
 * efficiency).
 *
 * Formulas (page "10. Tensor Cores, shapes, and tile alignment"):
 *   - section "Shape the operation": useful work 2MNK; G = ceil(M/T_M)
 *     ceil(N/T_N); wave efficiency G / (ceil(G/(S b)) S b);
 *   - section "Padding efficiency": MNK / (M'N'K');
 *   - section "When shape alone can't fix wave efficiency": split-K with a
 *     separate combine pass, and the persistent grid sized to the resident
 *     capacity S b.
 * Resident workgroups b (page "Grid 24 is not headroom", section "The
 * question I never asked"): the minimum over LDS, the register file (with
 * its allocation granule) and the wave slots of a compute unit.
 *
 * The page leaves the schedule of a persistent grid open.  Here the tiles of
 * the last partial round are cut along K across the otherwise idle
 * workgroups, since a loop over equal tiles alone still ends in a partial
 * round.  Efficiency of a schedule with unequal units is total work over
 * (S b x the busiest workgroup's work), in K-tile iterations; for equal
 * units it is exactly the wave-efficiency formula.
 */
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "plan.h"
#include "tiles.h"

namespace g355 {

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;
constexpr int64_t kMaxOffset = 0x7FFF0000;   /* largest 32-bit buffer offset used */
constexpr int32_t kMaxSplit = 256;
constexpr int32_t kMaxNK = 1 << 23;
constexpr int32_t kGroupM = 4;                        /* raster band height in tiles */
constexpr double kPeakBf16PerCu = 2516.6e12 / 256.0;   /* dense MFMA, 2.4 GHz */
constexpr double kPeakFp8PerCu = 5033.2e12 / 256.0;
constexpr double kPeakFp4PerCu = 10066.3e12 / 256.0;
constexpr double kHbmBytesPerSec = 5.0e12;            /* sustained, planning only */
constexpr double kExtraPassSec = 4.0e-6;              /* one launch: main, combine or repack */
/* Modelled times within this factor count as equal and the schedule with
 * the larger eta_sched * eta_pad wins.  A 15 % band let that preference
 * override the time model too often: over 40 sampled products whose plans
 * the two bands choose differently, the 5 % band's plans ran 15 % faster
 * (geometric mean; 29 faster by more than 5 %, 3 slower). */
constexpr double kTieBand = 1.05;
/* Rows that are not 16-byte aligned and read in place turn every copy of a
 * row (once per tile column of the product, or row for B) into unaligned
 * accesses over two lines.  From this dense-MFMA time at peak up, one
 * repack pass costs less than those re-reads (bf16 and E4M3 products from
 * 2500 x 2500 x 2501 up ran 15-31 % faster repacked; at 2000 x 2000 x 2001
 * and below, reading in place was as fast or faster). */
constexpr double kRepackMisalignedSec = 10.0e-6;
constexpr double kCopyBytesPerSecPerCu = 100.0e9;     /* L2 -> LDS copies per compute unit */
constexpr double kUnitSec = 3.0e-6;                   /* per unit run in turn on one slot: pipeline
                                                         fill and epilogue */

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

uint64_t gcd64(uint64_t a, uint64_t b)
{
    while (b) {
        const uint64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

struct Frac {
    uint64_t num, den;
};

Frac reduce(unsigned __int128 n, unsigned __int128 d)
{
    /* n, d < 2^127; reduce by the gcd, then they fit in 64 bits for every
     * quantity the planner forms (validated dimensions < 2^31). */
    unsigned __int128 a = n, b = d;
    while (b) {
        const unsigned __int128 t = a % b;
        a = b;
        b = t;
    }
    if (a == 0) a = 1;
    return Frac{(uint64_t)(n / a), (uint64_t)(d / a)};
}

bool frac_less(const Frac &x, const Frac &y)
{
    return (unsigned __int128)x.num * y.den < (unsigned __int128)y.num * x.den;
}

int bitlen(unsigned __int128 v)
{
    int n = 0;
    while (v) {
        ++n;
        v >>= 1;
    }
    return n;
}

struct Cand {
    int32_t tile = -1;
    int32_t b = 1;
    int64_t tiles_m = 0, tiles_n = 0, G = 0, nK = 0;
    int32_t split = 1;
    bool persistent = false;
    int64_t tail_tiles = 0;
    int32_t tail_split = 1;
    int64_t units_main = 0, units = 0, grid = 0;
    Frac eta_sched{0, 1};
    Frac eta_pad{0, 1};
    double t = 0;
    /* inputs of t (reported with the plan) */
    double mfma_peak_s = 0, mfma_eff = 0, bytes = 0, spread = 1, stream_eff = 0, copy_s = 0, fixed_s = 0;
    int64_t in_turn = 0;
};

/* Work (K-tile iterations) of a unit queue: total, the busiest workgroup's
 * (unit u on workgroup u mod P, P = launched grid capped at the slots), and
 * the busiest compute unit's (workgroup w on unit w mod S).  Mirrors
 * decode_unit's order. */
void schedule_loads(const Cand &c, int64_t slots, int32_t S, uint64_t &total, uint64_t &busiest,
                    uint64_t &busiest_cu)
{
    const int64_t P = std::min<int64_t>(std::max<int64_t>(c.grid, 1), slots);
    std::vector<uint64_t> load((size_t)P, 0);
    total = 0;
    for (int64_t u = 0; u < c.units; ++u) {
        int64_t cost;
        if (u < c.units_main) {
            if (c.split > 1) {
                const int64_t slice = u / c.G;
                cost = kslice_begin((int32_t)c.nK, c.split, (int32_t)slice + 1) -
                       kslice_begin((int32_t)c.nK, c.split, (int32_t)slice);
            } else {
                cost = c.nK;
            }
        } else {
            const int64_t slice = (u - c.units_main) / c.tail_tiles;
            cost = kslice_begin((int32_t)c.nK, c.tail_split, (int32_t)slice + 1) -
                   kslice_begin((int32_t)c.nK, c.tail_split, (int32_t)slice);
        }
        load[(size_t)(u % P)] += (uint64_t)cost;
        total += (uint64_t)cost;
    }
    busiest = 0;
    std::vector<uint64_t> cu((size_t)S, 0);
    for (int64_t w = 0; w < P; ++w) {
        busiest = std::max(busiest, load[(size_t)w]);
        cu[(size_t)(w % S)] += load[(size_t)w];
    }
    busiest_cu = 0;
    for (uint64_t l : cu) busiest_cu = std::max(busiest_cu, l);
}

void finish_candidate(Cand &c, const TileCfg &cfg, int32_t S, int64_t M, int64_t N, int64_t K,
                      int64_t batch, int64_t kbytes, int32_t out_esize, int pack_passes)
{
    const int64_t slots = (int64_t)S * c.b;
    uint64_t total = 0, busiest = 0, busiest_cu = 0;
    schedule_loads(c, slots, S, total, busiest, busiest_cu);
    c.eta_sched = busiest ? reduce((unsigned __int128)total, (unsigned __int128)slots * busiest)
                          : Frac{0, 1};
    c.eta_pad = reduce((unsigned __int128)M * N * K,
                       (unsigned __int128)(c.tiles_m * cfg.TM) * (c.tiles_n * cfg.TN) *
                           (c.nK * cfg.TK));
    /* Time model (planning only).  MFMA side: the busiest compute unit's
     * K-tile iterations at the tile's sustained rate for this many resident
     * workgroups.  Memory side: algorithmic bytes plus the split-K partial
     * sums the main pass writes, at a sustained HBM rate scaled by how
     * evenly the work is spread over the compute units.  The three sides
     * overlap only in part: they combine as a 4-norm (between their sum and
     * their maximum).  Each unit a workgroup slot runs in turn adds a fixed
     * pipeline fill and epilogue; the combine pass reads the partial sums
     * back after the main pass. */
    const double cu_peak = cfg.dtype_class >= 3 ? kPeakFp4PerCu : cfg.dtype_class ? kPeakFp8PerCu : kPeakBf16PerCu;
    /* workgroups actually sharing a compute unit */
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(c.b, cdiv(std::max<int64_t>(c.grid, 1), S)));
    const double eff = cfg.mfma_eff[std::min<int64_t>(per_cu, 4) - 1];
    const double t_mfma = (double)busiest_cu * 2.0 * cfg.TM * cfg.TN * cfg.TK / (cu_peak * eff);
    /* partial sums are written and read for the split tiles' positions
     * inside M x N only */
    double partial = 0;
    if (c.split > 1 || c.tail_tiles) {
        Sched sc{};
        sc.tiles_m = (int32_t)c.tiles_m;
        sc.tiles_n = (int32_t)c.tiles_n;
        sc.tiles_per_batch = (int32_t)(c.tiles_m * c.tiles_n);
        sc.batch = (int32_t)batch;
        sc.group_m = kGroupM;
        const int64_t first = c.split > 1 ? 0 : c.units_main;
        const int64_t count = c.split > 1 ? c.G : c.tail_tiles;
        const int32_t nsl = c.split > 1 ? c.split : c.tail_split;
        for (int64_t t = first; t < first + count; ++t) {
            Unit u;
            tile_coords(sc, (int32_t)t, u);
            const int64_t rows = std::min<int64_t>(cfg.TM, M - (int64_t)u.tile_m * cfg.TM);
            const int64_t cols = std::min<int64_t>(cfg.TN, N - (int64_t)u.tile_n * cfg.TN);
            partial += (double)rows * cols * 4.0 * nsl;
        }
    }
    const double bytes = (double)batch * ((double)(M + N) * kbytes + (double)M * N * out_esize) + partial;
    const double spread = busiest_cu ? (double)total / ((double)S * busiest_cu) : 1.0;
    const double t_mem = bytes / (kHbmBytesPerSec * cfg.stream_eff * spread);
    /* the busiest unit's copies from L2 into LDS (operand panels shared by
     * several tiles are fetched once per tile) */
    const double t_copy = (double)busiest_cu * (cfg.TM + cfg.TN) * cfg.row_bytes / kCopyBytesPerSecPerCu;
    const double p4 = std::pow(t_mfma, 4.0) + std::pow(t_mem, 4.0) + std::pow(t_copy, 4.0);
    const int64_t in_turn = cdiv(std::max<int64_t>(c.units, 1), std::min<int64_t>(std::max<int64_t>(c.grid, 1), slots));
    const double fixed = kExtraPassSec + (partial > 0 ? kExtraPassSec + partial / kHbmBytesPerSec : 0.0) +
                         (pack_passes ? kExtraPassSec : 0.0);
    c.t = fixed + std::pow(p4, 0.25) + (double)in_turn * kUnitSec;
    c.mfma_peak_s = (double)busiest_cu * 2.0 * cfg.TM * cfg.TN * cfg.TK / cu_peak;
    c.mfma_eff = eff;
    c.bytes = bytes;
    c.spread = spread;
    c.stream_eff = cfg.stream_eff;
    c.copy_s = t_copy;
    c.fixed_s = fixed;
    c.in_turn = in_turn;
}

/* true if x should be preferred over y.  Modelled times within 15 % of each
 * other count as equal (the model is coarser than that); among those a
 * schedule that fills the device more than 3 % better (eta_sched * eta_pad)
 * wins, and otherwise the modelled time decides. */
bool better(const Cand &x, const Cand &y)
{
    if (y.tile < 0) return true;
    const bool close = x.t <= y.t * kTieBand && y.t <= x.t * kTieBand;
    if (!close) return x.t < y.t;
    const double ex = rational_to_double(x.eta_sched.num, x.eta_sched.den) *
                      rational_to_double(x.eta_pad.num, x.eta_pad.den);
    const double ey = rational_to_double(y.eta_sched.num, y.eta_sched.den) *
                      rational_to_double(y.eta_pad.num, y.eta_pad.den);
    if (ex > ey * 1.03) return true;
    if (ey > ex * 1.03) return false;
    if (x.t != y.t) return x.t < y.t;
    const Frac fx = reduce((unsigned __int128)x.eta_sched.num * x.eta_pad.num,
                           (unsigned __int128)x.eta_sched.den * x.eta_pad.den);
    const Frac fy = reduce((unsigned __int128)y.eta_sched.num * y.eta_pad.num,
                           (unsigned __int128)y.eta_sched.den * y.eta_pad.den);
    if (frac_less(fy, fx)) return true;
    if (frac_less(fx, fy)) return false;
    if (x.units != y.units) return x.units < y.units;
    if (kTiles[x.tile].TM != kTiles[y.tile].TM) return kTiles[x.tile].TM > kTiles[y.tile].TM;
    return kTiles[x.tile].TN > kTiles[y.tile].TN;
}

inline bool misaligned16(const void *p) { return ((uintptr_t)p & 15u) != 0; }

} /* namespace */

double rational_to_double(uint64_t num, uint64_t den)
{
    if (den == 0) return NAN;
    if (num == 0) return 0.0;
    /* q = floor(num 2^s / den) with 2^53 <= q < 2^54, then round half-even */
    int s = 53 - (bitlen(num) - bitlen(den));
    unsigned __int128 q, r;
    for (;;) {
        unsigned __int128 n = num, d = den;
        if (s >= 0)
            n <<= s;
        else
            d <<= -s;
        q = n / d;
        r = n % d;
        if (q >= ((unsigned __int128)1 << 54)) {
            --s;
        } else if (q < ((unsigned __int128)1 << 53)) {
            ++s;
        } else {
            break;
        }
    }
    uint64_t m = (uint64_t)(q >> 1);
    const bool half = (q & 1) != 0;
    const bool sticky = r != 0;
    if (half && (sticky || (m & 1))) ++m;
    return ldexp((double)m, 1 - s);
}

int32_t resident_workgroups(int32_t tile)
{
    const TileCfg &c = kTiles[tile];
    const int32_t waves = tile_waves(c);
    const int32_t threads = waves * kWaveSize;
    const int32_t by_lds = kLdsPerCu / c.lds_bytes;
    const int32_t regs = (c.vgpr_budget + kRegGranule - 1) / kRegGranule * kRegGranule;
    const int32_t regs_per_cu = kRegsPerLanePerSimd * kWaveSize * kSimdsPerCu;
    const int32_t by_regs = regs_per_cu / (regs * threads);
    const int32_t by_waves = kMaxWavesPerSimd * kSimdsPerCu / waves;
    return std::min(by_lds, std::min(by_regs, by_waves));
}

gemm355_status check_pointers(const gemm355_args &a, const ConvShape *conv)
{
    const int32_t ebits = dtype_ebits(a.dtype);
    const int32_t esize = ebits >= 8 ? ebits / 8 : 1;   /* alignment */
    const int32_t out_esize = dtype_out_bf16(a.dtype) ? 2 : 4;
    const bool a_row = a.layout == GEMM355_A_ROW_B_COL || a.layout == GEMM355_A_ROW_B_ROW;
    const bool b_col = a.layout == GEMM355_A_ROW_B_COL || a.layout == GEMM355_A_COL_B_COL;
    const int64_t M = a.M, N = a.N, K = a.K, batch = a.batch;
    if (M <= 0 || N <= 0) return GEMM355_OK;
    if (!a.C) return GEMM355_EINVAL;
    if (K > 0 && (!a.A || !a.B)) return GEMM355_EINVAL;
    if (((uintptr_t)a.C % (uintptr_t)out_esize) != 0) return GEMM355_EALIGN;
    if (K > 0 && (((uintptr_t)a.A % esize) != 0 || ((uintptr_t)a.B % esize) != 0))
        return GEMM355_EALIGN;
    if (((uintptr_t)a.scale_a & 3u) != 0 || ((uintptr_t)a.scale_b & 3u) != 0) return GEMM355_EALIGN;
    if (((uintptr_t)a.unit_stamps & 7u) != 0) return GEMM355_EALIGN;
    if (!dtype_mx(a.dtype) && (a.block_scale_a || a.block_scale_b)) return GEMM355_EINVAL;
    if (K == 0) return GEMM355_OK;
    if (dtype_mx(a.dtype)) {
        if (!a.block_scale_a || !a.block_scale_b) return GEMM355_EINVAL;
        if (((uintptr_t)a.block_scale_a & 3u) != 0 || ((uintptr_t)a.block_scale_b & 3u) != 0)
            return GEMM355_EALIGN;
    }
    /* C must not overlap A or B (byte ranges spanned by all batch entries) */
    const uintptr_t c_lo = (uintptr_t)a.C;
    const uintptr_t c_hi = c_lo + (uintptr_t)(((batch - 1) * a.stride_c + (M - 1) * a.ldc + N) * out_esize);
    const int64_t a_rows = a_row ? M : K, a_cols = a_row ? K : M;
    const int64_t b_rows = b_col ? N : K, b_cols = b_col ? K : N;
    const uintptr_t a_lo = (uintptr_t)a.A;
    /* element counts to bytes, rounded up (4-bit elements pack two a byte);
     * a convolution's A is its input images */
    auto span = [ebits](int64_t elems) { return (uintptr_t)((elems * ebits + 7) / 8); };
    const uintptr_t a_hi = a_lo + (conv ? span(conv->N * conv->H * conv->W * conv->C)
                                        : span((batch - 1) * a.stride_a + (a_rows - 1) * a.lda + a_cols));
    const uintptr_t b_lo = (uintptr_t)a.B;
    const uintptr_t b_hi = b_lo + span((batch - 1) * a.stride_b + (b_rows - 1) * a.ldb + b_cols);
    if ((c_lo < a_hi && a_lo < c_hi) || (c_lo < b_hi && b_lo < c_hi)) return GEMM355_EINVAL;
    if (dtype_mx(a.dtype)) {
        /* block-scale arrays: batch * rows * ceil(K / 32) bytes */
        const uintptr_t sa_lo = (uintptr_t)a.block_scale_a;
        const uintptr_t sa_hi = sa_lo + (uintptr_t)(batch * M * ((K + 31) / 32));
        const uintptr_t sb_lo = (uintptr_t)a.block_scale_b;
        const uintptr_t sb_hi = sb_lo + (uintptr_t)(batch * N * ((K + 31) / 32));
        if ((c_lo < sa_hi && sa_lo < c_hi) || (c_lo < sb_hi && sb_lo < c_hi)) return GEMM355_EINVAL;
    }
    return GEMM355_OK;
}

gemm355_status make_plan(const gemm355_args &a, int32_t S, Plan &P, const ConvShape *conv)
{
    memset(&P, 0, sizeof P);
    if ((int)a.dtype < 0 || (int)a.dtype >= kNumDtypes) return GEMM355_EINVAL;
    if ((int)a.layout < 0 || (int)a.layout > 3) return GEMM355_EINVAL;
    if (a.M < 0 || a.N < 0 || a.K < 0 || a.batch < 1) return GEMM355_EINVAL;
    if (a.split_k < 0 || a.persistent < -1 || a.persistent > 1) return GEMM355_EINVAL;
    if (a.tile < -1 || a.tile >= kNumTiles) return GEMM355_EINVAL;
    if (S < 1) return GEMM355_EINVAL;
    if (a.stride_a < 0 || a.stride_b < 0 || a.stride_c < 0) return GEMM355_EINVAL;

    const bool fp8 = dtype_fp8(a.dtype), fp4 = dtype_fp4(a.dtype), fp6 = dtype_fp6(a.dtype);
    const int32_t dclass = dtype_class_of(a.dtype);
    const int32_t ebits = dtype_ebits(a.dtype);
    const int32_t esize = fp8 || fp4 || fp6 ? 1 : 2;    /* bytes per element of the repack passes */
    const int32_t out_esize = dtype_out_bf16(a.dtype) ? 2 : 4;
    const bool a_row = a.layout == GEMM355_A_ROW_B_COL || a.layout == GEMM355_A_ROW_B_ROW;
    const bool b_col = a.layout == GEMM355_A_ROW_B_COL || a.layout == GEMM355_A_COL_B_COL;
    const int32_t want_op = conv ? 1 : 0;
    if (a.tile >= 0 && (kTiles[a.tile].dtype_class != dclass || kTiles[a.tile].op != want_op)) return GEMM355_EINVAL;

    const int64_t M = a.M, N = a.N, K = a.K, batch = a.batch;
    if (a.lda < std::max<int64_t>(1, a_row ? K : M)) return GEMM355_EINVAL;
    if (a.ldb < std::max<int64_t>(1, b_col ? K : N)) return GEMM355_EINVAL;
    if (a.ldc < std::max<int64_t>(1, N)) return GEMM355_EINVAL;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim) return GEMM355_EUNSUPPORTED;
    /* block scales are read one dword (four 32-value blocks) per row and
     * K-tile of 128 values */
    if (dtype_mx(a.dtype) && K % 128 != 0) return GEMM355_EUNSUPPORTED;
    /* FP4: native layout, whole bytes per row and batch entry, whole
     * K-tiles of 256 values (two scale dwords per row) */
    if (fp4 && (a.layout != GEMM355_A_ROW_B_COL || K % 256 != 0 || a.lda % 2 || a.ldb % 2 ||
                (batch > 1 && (a.stride_a % 2 || a.stride_b % 2))))
        return GEMM355_EUNSUPPORTED;
    /* FP6: native layout, rows and batch entries of whole 16-byte groups
     * (64 values), whole K-tiles of 128 values */
    if (fp6 && (a.layout != GEMM355_A_ROW_B_COL || K % 128 != 0 || a.lda % 64 || a.ldb % 64 ||
                (batch > 1 && (a.stride_a % 64 || a.stride_b % 64))))
        return GEMM355_EUNSUPPORTED;
    /* the regrouped scales of one batch entry are addressed with 32-bit
     * offsets */
    if (dtype_mx(a.dtype) && std::max(M, N) * (K / 32) > kMaxOffset) return GEMM355_EUNSUPPORTED;

    P.esize = esize;
    P.out_esize = out_esize;
    P.pub.S = S;
    P.pub.tile = -1;

    const bool work = M > 0 && N > 0;
    {
        const gemm355_status pst = check_pointers(a, conv);
        if (pst != GEMM355_OK) return pst;
    }

    /* Operand views of the main loop: K-contiguous rows.  bf16 and 8-bit
     * rows are read in place (16-byte buffer loads take any byte address),
     * except rows that are not 16-byte aligned in products large enough
     * for a repack pass to pay (kRepackMisalignedSec); if K ends inside a
     * 16-byte chunk, the copy schedules that clear the chunk's bytes past K
     * in LDS (0, 4 and 5) are the only candidates.  Other operands (the
     * transposed layouts; block-scaled rows that are not 16-byte aligned or
     * do not end on a chunk) are repacked, zero-filled to a whole number of
     * K-tiles. */
    auto bytes_of = [ebits](int64_t elems) { return elems * ebits / 8; };
    const int64_t kbytes = bytes_of(K);
    const int64_t packed_ld = cdiv(std::max<int64_t>(kbytes, 1), 128) * 128;
    const bool in_place = (dclass == 0 || dclass == 1) && !conv;
    const bool ktail = kbytes % 16 != 0;
    const bool tail_tile_ok = a.tile < 0 || kTiles[a.tile].spread == 0 || kTiles[a.tile].spread == 4 ||
                              kTiles[a.tile].spread == 5 || kTiles[a.tile].spread == 6;
    const double peak_cu = fp4 || fp6 ? kPeakFp4PerCu : dclass ? kPeakFp8PerCu : kPeakBf16PerCu;
    const bool repack_misaligned =
        2.0 * (double)M * (double)N * (double)K * (double)batch / (peak_cu * S) >= kRepackMisalignedSec;
    auto needs_pack = [&](bool kcontig, const void *ptr, int64_t ld, int64_t stride) {
        if (!kcontig) return true;
        const bool mis = misaligned16(ptr) || bytes_of(ld) % 16 || (batch > 1 && bytes_of(stride) % 16);
        if (!in_place) return mis || ktail;
        if (mis && repack_misaligned) return true;
        return ktail && !tail_tile_ok;
    };
    P.pack_a = needs_pack(a_row, a.A, a.lda, a.stride_a);
    P.pack_b = needs_pack(b_col, a.B, a.ldb, a.stride_b);
    /* the repack passes move whole bytes per element */
    if ((fp4 || fp6) && (P.pack_a || P.pack_b)) return GEMM355_EUNSUPPORTED;
    if (conv) {
        /* the main loop gathers A from the images itself: 64-channel K-tiles
         * of 16-byte aligned pixels; B (the filters) must be native */
        if (P.pack_b || misaligned16(a.A) || (conv->C * 2) % 128) return GEMM355_EUNSUPPORTED;
        /* pixel offsets are 32-bit from the first image */
        if (conv->N * conv->H * conv->W * conv->C * 2 > kMaxOffset) return GEMM355_EUNSUPPORTED;
        P.pack_a = 0;
    }
    if (P.pack_a) {
        P.lda_b = packed_ld;
        P.stride_a_b = M * packed_ld;
    } else {
        P.lda_b = bytes_of(a.lda);
        P.stride_a_b = bytes_of(a.stride_a);
    }
    if (P.pack_b) {
        P.ldb_b = packed_ld;
        P.stride_b_b = N * packed_ld;
    } else {
        P.ldb_b = bytes_of(a.ldb);
        P.stride_b_b = bytes_of(a.stride_b);
    }
    P.Kb = (int32_t)std::min<int64_t>(cdiv(kbytes, 16) * 16, kMaxDim);
    /* an operand read in place whose K ends inside a chunk: its bytes past
     * K are cleared in LDS, and only tiles with that clearing are planned */
    const bool tail_in_place = ktail && (!P.pack_a || !P.pack_b);
    P.Kv = tail_in_place ? (int32_t)std::min<int64_t>(kbytes, kMaxDim) : 0;
    P.pub.repack = (P.pack_a ? 1 : 0) | (P.pack_b ? 2 : 0);
    if (256 * P.lda_b > kMaxOffset || 256 * P.ldb_b > kMaxOffset) return GEMM355_EUNSUPPORTED;
    if (256 * a.ldc * out_esize > kMaxOffset) return GEMM355_EUNSUPPORTED;

    /* ---- candidate schedules */
    Cand best;
    for (int32_t t = 0; t < kNumTiles; ++t) {
        const TileCfg &cfg = kTiles[t];
        if (cfg.dtype_class != dclass || cfg.op != want_op) continue;
        if (a.tile >= 0 && a.tile != t) continue;
        if (P.Kv && cfg.spread != 0 && cfg.spread != 4 && cfg.spread != 5 && cfg.spread != 6) continue;
        Cand base;
        base.tile = t;
        base.tiles_m = cdiv(std::max<int64_t>(M, 1), cfg.TM);
        base.tiles_n = cdiv(std::max<int64_t>(N, 1), cfg.TN);
        base.G = batch * base.tiles_m * base.tiles_n;
        base.nK = cdiv(K, cfg.TK);
        if (base.G > kMaxDim || base.nK >= kMaxNK) return GEMM355_EUNSUPPORTED;
        const int32_t b_max = resident_workgroups(t);
        const int pack_passes = (P.pack_a ? 1 : 0) + (P.pack_b ? 1 : 0);

        std::vector<int32_t> splits;
        if (K == 0) {
            splits.push_back(1);
        } else if (a.split_k >= 2) {
            splits.push_back((int32_t)std::min<int64_t>(std::min<int64_t>(a.split_k, base.nK), kMaxSplit));
        } else {
            splits.push_back(1);
            if (a.split_k == 0)
                for (int64_t s = 2; s <= std::min<int64_t>(base.nK, kMaxSplit); ++s)
                    if (base.G * s <= 2 * (int64_t)S * b_max) splits.push_back((int32_t)s);
        }
        for (int32_t s : splits) {
            std::vector<bool> pmodes;
            if (a.persistent == 0) pmodes = {false};
            else if (a.persistent == 1) pmodes = {true};
            else pmodes = {false, true};
            for (bool pers : pmodes) {
                /* a one-shot grid gets whatever residency the hardware gives
                 * (b_max); a persistent grid launches S * b_used groups */
                for (int32_t bu = pers ? 1 : b_max; bu <= b_max; ++bu) {
                    Cand c = base;
                    c.b = bu;
                    const int64_t slots = (int64_t)S * bu;
                    c.split = s;
                    c.persistent = pers;
                    if (K == 0) {
                        c.units_main = c.units = c.grid = 0;
                    } else if (s > 1) {
                        c.units_main = c.units = c.G * s;
                        c.grid = pers ? std::min<int64_t>(c.units, slots) : c.units;
                    } else if (pers) {
                        const int64_t R = c.G / slots;
                        const int64_t T = c.G - R * slots;
                        const int64_t st = T ? std::min<int64_t>(slots / T, c.nK) : 1;
                        if (T && st >= 2) {
                            c.units_main = R * slots;
                            c.tail_tiles = T;
                            c.tail_split = (int32_t)std::min<int64_t>(st, kMaxSplit);
                            c.units = c.units_main + T * c.tail_split;
                        } else {
                            c.units_main = c.units = c.G;
                        }
                        c.grid = std::min<int64_t>(c.units, slots);
                    } else {
                        c.units_main = c.units = c.grid = c.G;
                    }
                    if (c.units > kMaxDim) return GEMM355_EUNSUPPORTED;
                    /* a persistent grid that fits in fewer resident groups
                     * per unit is the same launch with worse bookkeeping */
                    if (pers && bu > 1 && c.grid <= (int64_t)S * (bu - 1)) continue;
                    /* automatic persistence only when it changes the schedule */
                    if (a.persistent == -1 && pers && c.units <= slots && c.tail_tiles == 0 &&
                        bu == b_max)
                        continue;
                    if (K > 0)
                        finish_candidate(c, cfg, S, M, N, K, batch, kbytes, out_esize, pack_passes);
                    if (better(c, best)) best = c;
                }
            }
        }
    }
    if (best.tile < 0) return GEMM355_EINVAL;

    const TileCfg &cfg = kTiles[best.tile];
    gemm355_plan_t &o = P.pub;
    o.tile = best.tile;
    o.model_seconds = best.t;
    o.model_mfma_peak_seconds = best.mfma_peak_s;
    o.model_mfma_eff = best.mfma_eff;
    o.model_bytes = best.bytes;
    o.model_spread = best.spread;
    o.model_stream_eff = best.stream_eff;
    o.model_copy_seconds = best.copy_s;
    o.model_fixed_seconds = best.fixed_s;
    o.model_units_in_turn = best.in_turn;
    o.T_M = cfg.TM;
    o.T_N = cfg.TN;
    o.T_K = cfg.TK;
    o.stages = cfg.stages;
    o.waves = tile_waves(cfg);
    o.lds_bytes = cfg.lds_bytes;
    o.vgpr_budget = cfg.vgpr_budget;
    o.b = best.b;
    o.G = best.G;
    o.nK = best.nK;
    o.M_pad = best.tiles_m * cfg.TM;
    o.N_pad = best.tiles_n * cfg.TN;
    o.K_pad = best.nK * cfg.TK;
    o.split = best.split;
    o.persistent = best.persistent ? 1 : 0;
    o.tail_tiles = best.tail_tiles;
    o.tail_split = best.tail_split;
    o.units = best.units;
    o.grid = best.grid;
    const int64_t slots = (int64_t)S * best.b;
    /* wave efficiency of the plain one-tile-per-workgroup grid (G tiles on
     * S * b slots), whatever schedule was chosen */
    const Frac ew = reduce((unsigned __int128)best.G, (unsigned __int128)cdiv(best.G, slots) * slots);
    o.eta_wave_num = (int64_t)ew.num;
    o.eta_wave_den = (int64_t)ew.den;
    if (K > 0 && work) {
        o.eta_pad_num = (int64_t)best.eta_pad.num;
        o.eta_pad_den = (int64_t)best.eta_pad.den;
        o.eta_sched_num = (int64_t)best.eta_sched.num;
        o.eta_sched_den = (int64_t)best.eta_sched.den;
    } else {
        o.eta_pad_num = 0;
        o.eta_pad_den = 1;
        o.eta_sched_num = 0;
        o.eta_sched_den = 1;
    }

    Sched &s = P.s;
    s.tiles_m = (int32_t)best.tiles_m;
    s.tiles_n = (int32_t)best.tiles_n;
    s.tiles_per_batch = (int32_t)(best.tiles_m * best.tiles_n);
    s.batch = (int32_t)batch;
    s.group_m = kGroupM;
    s.nK = (int32_t)best.nK;
    s.split = best.split;
    s.units_main = (int32_t)best.units_main;
    s.tail_first = (int32_t)best.units_main;
    s.tail_tiles = (int32_t)best.tail_tiles;
    s.tail_split = best.tail_split;
    s.units = (int32_t)best.units;
    s.grid = (int32_t)best.grid;
    s.xcd_remap = 1;

    size_t off = 0;
    auto carve = [&off](size_t bytes, size_t &at) {
        at = off;
        off += (bytes + 255) / 256 * 256;
    };
    size_t partial = 0;
    if (best.split > 1) {
        partial = (size_t)best.G * best.split * cfg.TM * cfg.TN * 4;
        P.reduce_tiles = (int32_t)best.G;
        P.reduce_tail = 0;
    } else if (best.tail_tiles) {
        partial = (size_t)best.tail_tiles * best.tail_split * cfg.TM * cfg.TN * 4;
        P.reduce_tiles = (int32_t)best.tail_tiles;
        P.reduce_tail = 1;
    }
    if (!work || K == 0) {
        partial = 0;
        P.reduce_tiles = 0;
        P.pack_a = P.pack_b = 0;
        o.repack = 0;
    }
    P.ws_partial_bytes = partial;
    carve(partial, P.ws_partial_off);
    P.ws_pack_a_bytes = P.pack_a ? (size_t)(batch * M * P.lda_b) : 0;
    carve(P.ws_pack_a_bytes, P.ws_pack_a_off);
    P.ws_pack_b_bytes = P.pack_b ? (size_t)(batch * N * P.ldb_b) : 0;
    carve(P.ws_pack_b_bytes, P.ws_pack_b_off);
    /* block scales: one dword (four 32-value blocks) per row and K-tile */
    const bool mx = dtype_mx(a.dtype) && work && K > 0;
    P.ws_scale_a_bytes = mx ? (size_t)(batch * M * (K / 32)) : 0;
    carve(P.ws_scale_a_bytes, P.ws_scale_a_off);
    P.ws_scale_b_bytes = mx ? (size_t)(batch * N * (K / 32)) : 0;
    carve(P.ws_scale_b_bytes, P.ws_scale_b_off);
    o.workspace_bytes = off;
    if (!work) {
        o.units = 0;
        o.grid = 0;
        s.units = 0;
        s.grid = 0;
    }
    return GEMM355_OK;
}

} /* namespace g355 */
