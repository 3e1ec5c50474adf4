/*
 * api.hip -- the C ABI of libgemm355 (declared in include/gemm355.h).
 *
 * A call validates and plans on the host (plans are cached per argument
 * shape), then enqueues on the caller's stream: optional operand repacks,
 * the main MFMA kernel over the plan's work units, and for split-K (or a
 * split tail of a persistent grid) the combine kernel.  Nothing here blocks
 * the host except the first use of a device (property query), the growth
 * of library-owned scratch, and waiting for another thread that is
 * enqueueing on the same stream with that stream's scratch.
 */
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <memory>
#include <mutex>
#include <thread>
#include <tuple>
#include <unordered_map>

#include "../../include/gemm355.h"
#include "kernels.h"
#include "plan.h"
#include "tiles.h"

using namespace g355;

namespace {

std::mutex g_mu;

int32_t device_cus()
{
    static std::map<int, int32_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    hipDeviceProp_t prop;
    int32_t cus = 256;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
        cus = prop.multiProcessorCount;
    cache[dev] = cus;
    return cus;
}

int32_t planning_cus(const gemm355_args &a)
{
    if (a.cus > 0) return a.cus;
    if (a.cus < 0) return -1;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return device_cus();
}

/* Plan cache: the plan depends on the shape arguments, the knobs and the
 * 16-byte alignment of A and B, never on the data. */
struct PlanKey {
    int64_t v[32];
    bool operator==(const PlanKey &o) const { return memcmp(v, o.v, sizeof v) == 0; }
};
struct PlanKeyHash {
    size_t operator()(const PlanKey &k) const
    {
        uint64_t h = 1469598103934665603ull;
        for (int64_t x : k.v) {
            h ^= (uint64_t)x;
            h *= 1099511628211ull;
        }
        return (size_t)h;
    }
};
std::unordered_map<PlanKey, Plan, PlanKeyHash> g_plans;

PlanKey key_of(const gemm355_args &a, int32_t S, const ConvShape *conv)
{
    PlanKey k;
    memset(&k, 0, sizeof k);
    if (conv) {
        const int64_t *f = &conv->N;
        for (int i = 0; i < 14; ++i) k.v[16 + i] = f[i];
        k.v[30] = 1;
    }
    k.v[0] = a.M;
    k.v[1] = a.N;
    k.v[2] = a.K;
    k.v[3] = a.lda;
    k.v[4] = a.ldb;
    k.v[5] = a.ldc;
    k.v[6] = a.stride_a;
    k.v[7] = a.stride_b;
    k.v[8] = a.stride_c;
    k.v[9] = a.batch;
    k.v[10] = ((int64_t)a.dtype << 8) | (int64_t)a.layout;
    k.v[11] = ((int64_t)a.split_k << 32) | (uint32_t)(a.persistent + 1);
    k.v[12] = ((int64_t)a.tile << 32) | (uint32_t)S;
    k.v[13] = (int64_t)(((uintptr_t)a.A & 15u) | (((uintptr_t)a.B & 15u) << 4) |
                        (((uintptr_t)a.C & 15u) << 8) | (((uintptr_t)a.scale_a & 3u) << 12) |
                        (((uintptr_t)a.scale_b & 3u) << 14));
    /* null-ness matters for validation */
    k.v[14] = (a.A ? 1 : 0) | (a.B ? 2 : 0) | (a.C ? 4 : 0) | (a.block_scale_a ? 8 : 0) |
              (a.block_scale_b ? 16 : 0);
    return k;
}

gemm355_status get_plan(const gemm355_args &a, Plan &out, const ConvShape *conv = nullptr)
{
    const int32_t S = planning_cus(a);
    if (S < 1) return GEMM355_EINVAL;
    const PlanKey k = key_of(a, S, conv);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_plans.find(k);
        if (it != g_plans.end()) {
            out = it->second;
            return check_pointers(a, conv);
        }
    }
    gemm355_status st = make_plan(a, S, out, conv);
    if (st != GEMM355_OK) return st;
    /* pointer overlap is not part of the key: check_pointers runs on hits */
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_plans.size() > 4096) g_plans.clear();
    g_plans.emplace(k, out);
    return GEMM355_OK;
}

/* Library-owned scratch, one buffer per (device, stream), grown on demand.
 *
 * A call that uses the buffer holds its lock from the lookup until its last
 * kernel is enqueued.  Calls on one stream therefore enqueue their kernels
 * as whole groups, never interleaved (one call's main pass cannot overwrite
 * partial sums another call's combine pass has yet to read), and the stream
 * runs the groups in enqueue order.  A buffer is replaced (after the stream
 * has drained the work of earlier calls) only by a call holding the lock,
 * so no call can be handed a buffer that is then freed under it.  The
 * per-thread default stream is one handle for many streams, so its buffers
 * are kept per thread as well. */
struct Scratch {
    std::mutex mu;
    void *ptr = nullptr;
    size_t bytes = 0;
};
struct ScratchKey {
    int dev;
    void *stream;
    std::thread::id thread;
    bool operator<(const ScratchKey &o) const
    {
        return std::tie(dev, stream, thread) < std::tie(o.dev, o.stream, o.thread);
    }
};
std::map<ScratchKey, std::unique_ptr<Scratch>> g_scratch;
/* largest library-owned buffer a call may hold (gemm355_set_scratch_limit) */
std::atomic<uint64_t> g_scratch_limit{UINT64_MAX};

gemm355_status library_scratch(size_t need, void *stream, void **out, std::unique_lock<std::mutex> &hold)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM355_EHIP;
    Scratch *s;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        const ScratchKey key{dev, stream,
                             (hipStream_t)stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
        std::unique_ptr<Scratch> &slot = g_scratch[key];
        if (!slot) slot.reset(new Scratch);
        s = slot.get();
    }
    /* entries are never erased before unload, so s stays valid */
    hold = std::unique_lock<std::mutex>(s->mu);
    const uint64_t limit = g_scratch_limit.load();
    /* over the cap: refused like a failed allocation, before the buffer
     * that earlier calls may still read is touched */
    if (need > limit) return GEMM355_ENOMEM;
    if (s->bytes < need) {
        if (s->ptr) {
            /* earlier calls on this stream may still read the old buffer */
            if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return GEMM355_EHIP;
            (void)hipFree(s->ptr);
            s->ptr = nullptr;
            s->bytes = 0;
        }
        size_t grow = need + need / 4;
        if (grow > limit) grow = (size_t)limit;
        if (hipMalloc(&s->ptr, grow) != hipSuccess) {
            (void)hipGetLastError();
            s->ptr = nullptr;
            return GEMM355_ENOMEM;
        }
        s->bytes = grow;
    }
    *out = s->ptr;
    return GEMM355_OK;
}

struct ScratchReaper {
    ~ScratchReaper()
    {
        for (auto &kv : g_scratch)
            if (kv.second && kv.second->ptr) (void)hipFree(kv.second->ptr);
    }
} g_reaper;

/* Scratch of gemm355_gemm_noalloc: a fixed array in every device's memory,
 * held from the library's load until the process ends.  Host code never
 * passes `scratch` itself to a kernel (on the host the name denotes a
 * stand-in, not a device address): the device address is looked up once
 * per device, with that device current, and kept per device. */
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

struct NoAllocScratch {
    std::mutex mu;          /* held by a call until its last enqueue */
    void *ptr = nullptr;    /* the array's address on this device */
};
std::mutex g_noalloc_mu;
std::map<int, std::unique_ptr<NoAllocScratch>> g_noalloc;

gemm355_status noalloc_scratch(void **out, std::unique_lock<std::mutex> &hold)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM355_EHIP;
    }
    NoAllocScratch *s;
    {
        std::lock_guard<std::mutex> lk(g_noalloc_mu);
        std::unique_ptr<NoAllocScratch> &slot = g_noalloc[dev];
        if (!slot) {
            void *ptr = nullptr;
            if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
                (void)hipGetLastError();
                return GEMM355_EHIP;
            }
            slot.reset(new NoAllocScratch);
            slot->ptr = ptr;
        }
        s = slot.get();
    }
    /* calls from several threads on one stream enqueue call by call */
    hold = std::unique_lock<std::mutex>(s->mu);
    *out = s->ptr;
    return GEMM355_OK;
}

/* no_alloc: take scratch from the fixed per-device array instead of the
 * caller's workspace or library-owned memory (nothing is allocated). */
gemm355_status run(const gemm355_args &a, void *stream, const ConvShape *conv = nullptr, bool no_alloc = false)
{
    Plan P;
    gemm355_status st = get_plan(a, P, conv);
    if (st != GEMM355_OK) return st;
    if (a.M == 0 || a.N == 0) return GEMM355_OK;
    hipStream_t hs = (hipStream_t)stream;

    if (a.K == 0) {
        if (launch_zero(a.C, (int32_t)a.M, (int32_t)a.N, a.ldc, a.stride_c, (int32_t)a.batch,
                        P.out_esize, hs) != hipSuccess)
            return GEMM355_EHIP;
        return GEMM355_OK;
    }

    uint8_t *ws = nullptr;
    /* held until this call's last launch is enqueued (library scratch) */
    std::unique_lock<std::mutex> hold;
    if (P.pub.workspace_bytes) {
        if (no_alloc) {
            /* every kernel writes the scratch it later reads (partial slots,
             * repacked rows, regrouped scales), so nothing needs clearing */
            if (P.pub.workspace_bytes > kNoAllocScratchBytes) return GEMM355_ETOOBIG;
            void *p = nullptr;
            st = noalloc_scratch(&p, hold);
            if (st != GEMM355_OK) return st;
            ws = (uint8_t *)p;
        } else if (a.workspace) {
            if (a.workspace_bytes < P.pub.workspace_bytes) return GEMM355_ENOMEM;
            if (((uintptr_t)a.workspace & 255u) != 0) return GEMM355_EALIGN;
            ws = (uint8_t *)a.workspace;
        } else {
            void *p = nullptr;
            st = library_scratch(P.pub.workspace_bytes, stream, &p, hold);
            if (st != GEMM355_OK) return st;
            ws = (uint8_t *)p;
        }
    }

    const uint8_t *Aop = (const uint8_t *)a.A;
    const uint8_t *Bop = (const uint8_t *)a.B;
    const bool a_row = a.layout == GEMM355_A_ROW_B_COL || a.layout == GEMM355_A_ROW_B_ROW;
    const bool b_col = a.layout == GEMM355_A_ROW_B_COL || a.layout == GEMM355_A_COL_B_COL;
    PackParams pks[2];
    int npk = 0;
    if (P.pack_a) {
        PackParams &pk = pks[npk++];
        pk.src = a.A;
        pk.dst = ws + P.ws_pack_a_off;
        pk.ld = a.lda;
        pk.stride = a.stride_a;
        pk.ldd_bytes = P.lda_b;
        pk.dst_stride_bytes = P.stride_a_b;
        pk.rows = (int32_t)a.M;
        pk.K = (int32_t)a.K;
        pk.batch = (int32_t)a.batch;
        pk.esize = P.esize;
        pk.kmajor = a_row ? 1 : 0;
        Aop = pk.dst;
    }
    if (P.pack_b) {
        PackParams &pk = pks[npk++];
        pk.src = a.B;
        pk.dst = ws + P.ws_pack_b_off;
        pk.ld = a.ldb;
        pk.stride = a.stride_b;
        pk.ldd_bytes = P.ldb_b;
        pk.dst_stride_bytes = P.stride_b_b;
        pk.rows = (int32_t)a.N;
        pk.K = (int32_t)a.K;
        pk.batch = (int32_t)a.batch;
        pk.esize = P.esize;
        pk.kmajor = b_col ? 1 : 0;
        Bop = pk.dst;
    }
    if (npk && launch_pack(pks, npk, hs) != hipSuccess) return GEMM355_EHIP;

    GemmParams gp;
    gp.A = Aop;
    gp.B = Bop;
    gp.C = a.C;
    gp.ws = (float *)(ws ? ws + P.ws_partial_off : nullptr);
    gp.lda = P.lda_b;
    gp.ldb = P.ldb_b;
    gp.stride_a = P.stride_a_b;
    gp.stride_b = P.stride_b_b;
    gp.ldc = a.ldc;
    gp.stride_c = a.stride_c;
    gp.scale_a = a.scale_a;
    gp.scale_b = a.scale_b;
    gp.M = (int32_t)a.M;
    gp.N = (int32_t)a.N;
    gp.Kb = P.Kb;
    gp.Kv = P.Kv;
    gp.out_bf16 = P.out_esize == 2 ? 1 : 0;
    gp.c_vec = ((uintptr_t)a.C % 16 == 0) && (a.ldc * P.out_esize) % 16 == 0 &&
               (a.batch <= 1 || (a.stride_c * P.out_esize) % 16 == 0);
    gp.stamps = a.unit_stamps;
    gp.bsa = gp.bsb = nullptr;
    gp.ktp_a = a.M * 4;
    gp.ktp_b = a.N * 4;
    gp.stride_bsa = a.M * (a.K / 32);
    gp.stride_bsb = a.N * (a.K / 32);
    if (P.ws_scale_a_bytes) {
        /* regroup the block scales K-tile-major so that one direct-to-LDS
         * dword copy of 64 rows reads 256 contiguous bytes */
        ScalePackParams sp;
        sp.src = a.block_scale_a;
        sp.dst = (uint32_t *)(ws + P.ws_scale_a_off);
        sp.rows = (int32_t)a.M;
        sp.nK = (int32_t)(a.K / 128);
        sp.batch = (int32_t)a.batch;
        if (launch_pack_scales(sp, hs) != hipSuccess) return GEMM355_EHIP;
        gp.bsa = (const uint8_t *)sp.dst;
        sp.src = a.block_scale_b;
        sp.dst = (uint32_t *)(ws + P.ws_scale_b_off);
        sp.rows = (int32_t)a.N;
        if (launch_pack_scales(sp, hs) != hipSuccess) return GEMM355_EHIP;
        gp.bsb = (const uint8_t *)sp.dst;
    }
    gp.cv_H = gp.cv_W = gp.cv_C = gp.cv_S = gp.cv_P = gp.cv_Q = 0;
    gp.cv_ph = gp.cv_pw = gp.cv_sh = gp.cv_sw = gp.cv_dh = gp.cv_dw = 0;
    if (conv) {
        gp.cv_H = (int32_t)conv->H;
        gp.cv_W = (int32_t)conv->W;
        gp.cv_C = (int32_t)conv->C;
        gp.cv_S = (int32_t)conv->S;
        gp.cv_P = (int32_t)conv->P;
        gp.cv_Q = (int32_t)conv->Q;
        gp.cv_ph = (int32_t)conv->pad_h;
        gp.cv_pw = (int32_t)conv->pad_w;
        gp.cv_sh = (int32_t)conv->stride_h;
        gp.cv_sw = (int32_t)conv->stride_w;
        gp.cv_dh = (int32_t)conv->dil_h;
        gp.cv_dw = (int32_t)conv->dil_w;
    }
    gp.s = P.s;
    /* operand-format pair of an 8-bit product: 0 E4M3 x E4M3, 1 E5M2 x E5M2,
     * 2 E4M3 x E5M2 */
    const int32_t fmt = !(dtype_fp8(a.dtype) || dtype_fp6(a.dtype)) ? 0
                        : dtype_fmt_a(a.dtype) ? 1 : dtype_fmt_b(a.dtype) ? 2 : 0;
    if (P.s.grid > 0 && launch_gemm(P.pub.tile, fmt, gp, hs) != hipSuccess) return GEMM355_EHIP;

    if (P.reduce_tiles > 0) {
        ReduceParams rp;
        rp.ws = gp.ws;
        rp.C = a.C;
        rp.ldc = a.ldc;
        rp.stride_c = a.stride_c;
        rp.scale_a = a.scale_a;
        rp.scale_b = a.scale_b;
        rp.M = (int32_t)a.M;
        rp.N = (int32_t)a.N;
        rp.TM = P.pub.T_M;
        rp.TN = P.pub.T_N;
        rp.out_bf16 = gp.out_bf16;
        rp.tail = P.reduce_tail;
        rp.s = P.s;
        if (launch_reduce(rp, P.reduce_tiles, hs) != hipSuccess) return GEMM355_EHIP;
    }
    return GEMM355_OK;
}

/* A convolution's implicit product: validation, output size, the product's
 * arguments and the shape the main loop gathers A with. */
gemm355_status conv_setup(const gemm355_conv_args *c, gemm355_args &a, ConvShape &cs)
{
    if (!c) return GEMM355_EINVAL;
    if (c->N < 1 || c->H < 1 || c->W < 1 || c->C < 1 || c->K < 1 || c->R < 1 || c->S < 1) return GEMM355_EINVAL;
    if (c->stride_h < 1 || c->stride_w < 1 || c->dil_h < 1 || c->dil_w < 1 || c->pad_h < 0 || c->pad_w < 0)
        return GEMM355_EINVAL;
    const int64_t lim = (int64_t)1 << 30;
    if (c->N > lim || c->H > lim || c->W > lim || c->C > lim || c->K > lim || c->R > lim || c->S > lim ||
        c->pad_h > lim || c->pad_w > lim || c->stride_h > lim || c->stride_w > lim || c->dil_h > lim ||
        c->dil_w > lim)
        return GEMM355_EUNSUPPORTED;
    const int64_t ph = c->H + 2 * c->pad_h - c->dil_h * (c->R - 1) - 1;
    const int64_t pw = c->W + 2 * c->pad_w - c->dil_w * (c->S - 1) - 1;
    if (ph < 0 || pw < 0) return GEMM355_EINVAL;
    if ((int)c->dtype < 0 || (int)c->dtype >= kNumDtypes) return GEMM355_EINVAL;
    if (c->dtype != GEMM355_BF16_F32 && c->dtype != GEMM355_BF16_BF16) return GEMM355_EUNSUPPORTED;
    cs.N = c->N;
    cs.H = c->H;
    cs.W = c->W;
    cs.C = c->C;
    cs.R = c->R;
    cs.S = c->S;
    cs.P = ph / c->stride_h + 1;
    cs.Q = pw / c->stride_w + 1;
    cs.pad_h = c->pad_h;
    cs.pad_w = c->pad_w;
    cs.stride_h = c->stride_h;
    cs.stride_w = c->stride_w;
    cs.dil_h = c->dil_h;
    cs.dil_w = c->dil_w;
    if (cs.N * cs.P * cs.Q > lim || cs.R * cs.S * cs.C > lim) return GEMM355_EUNSUPPORTED;
    memset(&a, 0, sizeof a);
    a.M = cs.N * cs.P * cs.Q;
    a.N = c->K;
    a.K = cs.R * cs.S * cs.C;
    a.A = c->x;
    a.lda = a.K;
    a.B = c->w;
    a.ldb = a.K;
    a.C = c->y;
    a.ldc = c->K;
    a.batch = 1;
    a.dtype = c->dtype;
    a.layout = GEMM355_A_ROW_B_COL;
    a.split_k = c->split_k;
    a.persistent = c->persistent;
    a.tile = c->tile;
    a.cus = c->cus;
    a.workspace = c->workspace;
    a.workspace_bytes = c->workspace_bytes;
    return GEMM355_OK;
}

} /* namespace */

extern "C" {

gemm355_status gemm355_conv2d(const gemm355_conv_args *args, void *stream)
{
    gemm355_args a;
    ConvShape cs;
    const gemm355_status st = conv_setup(args, a, cs);
    if (st != GEMM355_OK) return st;
    return run(a, stream, &cs);
}

gemm355_status gemm355_conv2d_plan(const gemm355_conv_args *args, gemm355_plan_t *out)
{
    if (!out) return GEMM355_EINVAL;
    gemm355_args a;
    ConvShape cs;
    gemm355_status st = conv_setup(args, a, cs);
    if (st != GEMM355_OK) return st;
    Plan P;
    st = get_plan(a, P, &cs);
    if (st != GEMM355_OK) return st;
    *out = P.pub;
    return GEMM355_OK;
}

gemm355_status gemm355_conv2d_out_size(const gemm355_conv_args *args, int64_t *P, int64_t *Q)
{
    if (!P || !Q) return GEMM355_EINVAL;
    gemm355_args a;
    ConvShape cs;
    const gemm355_status st = conv_setup(args, a, cs);
    if (st != GEMM355_OK) return st;
    *P = cs.P;
    *Q = cs.Q;
    return GEMM355_OK;
}

gemm355_status gemm355_gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                            const void *B, int64_t ldb, void *C, int64_t ldc, gemm355_dtype dtype,
                            gemm355_layout layout, int32_t split_k, int32_t persistent,
                            void *stream)
{
    gemm355_args a;
    memset(&a, 0, sizeof a);
    a.M = M;
    a.N = N;
    a.K = K;
    a.A = A;
    a.lda = lda;
    a.B = B;
    a.ldb = ldb;
    a.C = C;
    a.ldc = ldc;
    a.batch = 1;
    a.dtype = dtype;
    a.layout = layout;
    a.split_k = split_k;
    a.persistent = persistent;
    a.tile = -1;
    return run(a, stream);
}

gemm355_status gemm355_gemm_ex(const gemm355_args *args, void *stream)
{
    if (!args) return GEMM355_EINVAL;
    return run(*args, stream);
}

gemm355_status gemm355_gemm_noalloc(const gemm355_args *args, void *stream)
{
    if (!args) return GEMM355_EINVAL;
    if (args->workspace || args->workspace_bytes) return GEMM355_EINVAL;
    return run(*args, stream, nullptr, true);
}

gemm355_status gemm355_plan(const gemm355_args *args, gemm355_plan_t *out)
{
    if (!args || !out) return GEMM355_EINVAL;
    Plan P;
    gemm355_status st = get_plan(*args, P);
    if (st != GEMM355_OK) return st;
    *out = P.pub;
    return GEMM355_OK;
}

double gemm355_eta_wave(int64_t G, int32_t S, int32_t b)
{
    if (G < 1 || S < 1 || b < 1) return NAN;
    const uint64_t cap = (uint64_t)S * (uint64_t)b;
    const uint64_t waves = ((uint64_t)G + cap - 1) / cap;
    const uint64_t den = waves * cap;
    uint64_t num = (uint64_t)G, d = den, x = num, y = d;
    while (y) {
        const uint64_t t = x % y;
        x = y;
        y = t;
    }
    return rational_to_double(num / x, d / x);
}

double gemm355_eta_pad(int64_t M, int64_t N, int64_t K, int64_t T_M, int64_t T_N, int64_t T_K)
{
    if (M < 1 || N < 1 || K < 1 || T_M < 1 || T_N < 1 || T_K < 1) return NAN;
    if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF) return NAN;
    /* reduce each factor, then cross-reduce, to keep the rational in 64 bits */
    uint64_t num[3] = {(uint64_t)M, (uint64_t)N, (uint64_t)K};
    uint64_t den[3] = {(uint64_t)((M + T_M - 1) / T_M * T_M), (uint64_t)((N + T_N - 1) / T_N * T_N),
                       (uint64_t)((K + T_K - 1) / T_K * T_K)};
    auto gcd = [](uint64_t x, uint64_t y) {
        while (y) {
            const uint64_t t = x % y;
            x = y;
            y = t;
        }
        return x;
    };
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            const uint64_t g = gcd(num[i], den[j]);
            num[i] /= g;
            den[j] /= g;
        }
    unsigned __int128 n = (unsigned __int128)num[0] * num[1] * num[2];
    unsigned __int128 d = (unsigned __int128)den[0] * den[1] * den[2];
    /* exact (nearest binary64) whenever the reduced denominator fits in 64
     * bits, i.e. always when M'N'K' < 2^64; beyond that within one ulp */
    if (d >> 64) return (double)((long double)n / (long double)d);
    return rational_to_double((uint64_t)n, (uint64_t)d);
}

gemm355_status gemm355_kslice(int64_t nK, int32_t s, int32_t i, int64_t *begin, int64_t *end)
{
    if (!begin || !end || nK < 0 || s < 1 || i < 0 || i >= s) return GEMM355_EINVAL;
    *begin = (int64_t)(((unsigned __int128)i * (uint64_t)nK) / (uint64_t)s);
    *end = (int64_t)(((unsigned __int128)(i + 1) * (uint64_t)nK) / (uint64_t)s);
    return GEMM355_OK;
}

gemm355_status gemm355_unit(const gemm355_args *args, int64_t u, int64_t *batch, int64_t *tile_m,
                            int64_t *tile_n, int64_t *kt_begin, int64_t *kt_end)
{
    if (!args || !batch || !tile_m || !tile_n || !kt_begin || !kt_end) return GEMM355_EINVAL;
    Plan P;
    gemm355_status st = get_plan(*args, P);
    if (st != GEMM355_OK) return st;
    if (u < 0 || u >= P.s.units) return GEMM355_EINVAL;
    const Unit un = decode_unit(P.s, (int32_t)u);
    *batch = un.batch;
    *tile_m = un.tile_m;
    *tile_n = un.tile_n;
    *kt_begin = un.kt_begin;
    *kt_end = un.kt_end;
    return GEMM355_OK;
}

int32_t gemm355_num_tiles(void) { return kNumTiles; }

gemm355_status gemm355_tile_info(int32_t tile, int32_t *dtype_class, int32_t *T_M, int32_t *T_N,
                                 int32_t *T_K, int32_t *stages, int32_t *waves, int32_t *lds_bytes,
                                 int32_t *b_max, int32_t *op, int32_t *schedule)
{
    if (tile < 0 || tile >= kNumTiles) return GEMM355_EINVAL;
    const TileCfg &c = kTiles[tile];
    if (dtype_class) *dtype_class = c.dtype_class;
    if (T_M) *T_M = c.TM;
    if (T_N) *T_N = c.TN;
    if (T_K) *T_K = c.TK;
    if (stages) *stages = c.stages;
    if (waves) *waves = tile_waves(c);
    if (lds_bytes) *lds_bytes = c.lds_bytes;
    if (b_max) *b_max = resident_workgroups(tile);
    if (op) *op = c.op;
    if (schedule) *schedule = c.spread;
    return GEMM355_OK;
}

gemm355_status gemm355_set_scratch_limit(uint64_t bytes, uint64_t *previous)
{
    const uint64_t old = g_scratch_limit.exchange(bytes);
    if (previous) *previous = old;
    return GEMM355_OK;
}

gemm355_status gemm355_tile_occupancy(int32_t tile, int32_t *blocks_per_cu)
{
    if (tile < 0 || tile >= kNumTiles || !blocks_per_cu) return GEMM355_EINVAL;
    int n = 0;
    const int threads = tile_waves(kTiles[tile]) * kWaveSize;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_kernel_symbol(tile), threads, 0) !=
        hipSuccess) {
        (void)hipGetLastError();
        return GEMM355_EHIP;
    }
    *blocks_per_cu = n;
    return GEMM355_OK;
}

gemm355_status gemm355_quantize(const void *x, int64_t n, int64_t batch, gemm355_src src, gemm355_fp8 fmt,
                                void *q, float *scale, void *stream)
{
    if (n < 0 || batch < 1) return GEMM355_EINVAL;
    if ((int)src < 0 || (int)src > 1 || (int)fmt < 0 || (int)fmt > 1) return GEMM355_EINVAL;
    if (!scale || (n > 0 && (!x || !q))) return GEMM355_EINVAL;
    const int64_t es = src == GEMM355_SRC_F32 ? 4 : 2;
    if (((uintptr_t)scale & 3u) != 0) return GEMM355_EALIGN;
    if (n > 0 && ((uintptr_t)x % (uintptr_t)es) != 0) return GEMM355_EALIGN;
    if (n > 0 && (n >= ((int64_t)1 << 40) || batch >= ((int64_t)1 << 40) / n)) return GEMM355_EUNSUPPORTED;
    const int64_t total = n * batch;
    /* blocks per tensor: one per 16 Ki elements, at most 4096 */
    const int32_t parts = (int32_t)std::min<int64_t>(4096, std::max<int64_t>(1, (n + 16383) / 16384));
    if (batch * parts > ((int64_t)1 << 30)) return GEMM355_EUNSUPPORTED;
    /* no overlap between the input, the codes and the scales */
    auto overlap = [](uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; };
    const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)(total * es);
    const uintptr_t q0 = (uintptr_t)q, q1 = q0 + (uintptr_t)total;
    const uintptr_t s0 = (uintptr_t)scale, s1 = s0 + (uintptr_t)(batch * 4);
    if (total > 0 && (overlap(x0, x1, q0, q1) || overlap(x0, x1, s0, s1) || overlap(q0, q1, s0, s1)))
        return GEMM355_EINVAL;
    void *scr = nullptr;
    std::unique_lock<std::mutex> hold;
    gemm355_status st = library_scratch((size_t)(batch * parts) * sizeof(float), stream, &scr, hold);
    if (st != GEMM355_OK) return st;
    QuantParams qp;
    qp.x = x;
    qp.q = (uint8_t *)q;
    qp.scale = scale;
    qp.maxima = (float *)scr;
    qp.n = n;
    qp.batch = batch;
    qp.parts = parts;
    qp.src = src == GEMM355_SRC_F32 ? 0 : 1;
    qp.fmt = fmt == GEMM355_FP8_E4M3 ? 0 : 1;
    qp.vec = (x0 % 16 == 0) && (q0 % 8 == 0) && (n % 8 == 0);
    if (launch_quantize(qp, (hipStream_t)stream) != hipSuccess) return GEMM355_EHIP;
    return GEMM355_OK;
}

const char *gemm355_status_string(gemm355_status status)
{
    switch (status) {
    case GEMM355_OK: return "ok";
    case GEMM355_EINVAL: return "invalid argument";
    case GEMM355_EALIGN: return "misaligned pointer";
    case GEMM355_EUNSUPPORTED: return "unsupported size";
    case GEMM355_ENOMEM: return "workspace too small, scratch over its cap, or allocation failed";
    case GEMM355_EHIP: return "HIP runtime error";
    case GEMM355_ETOOBIG: return "needs more scratch than the allocation-free entry point's fixed buffer";
    default: return "unknown status";
    }
}

} /* extern "C" */
