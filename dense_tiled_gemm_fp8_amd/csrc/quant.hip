/*
 * quant.hip -- per-tensor scaling of fp32 or bf16 tensors to the 8-bit
 * formats of the Hopper row of the input/accumulate table (page "The Tensor
 * Core"): OCP E4M3FN and OCP E5M2.  The page "10. Tensor Cores, shapes, and
 * tile alignment" (section "Practical shape sweep") counts this quantisation
 * as part of an 8-bit product's cost when its speed is measured.
 *
 *   amax_kernel      per-block maxima of |x| over contiguous shares of each
 *                    tensor
 *   quantize_kernel  each block reduces its tensor's maxima (max is exact
 *                    in any order, so every block sees the same amax),
 *                    forms s = amax / F (F = largest finite value of the
 *                    format; s = 1 when amax == 0), and writes
 *                    q = code nearest (x / s clamped to [-F, F]), ties to
 *                    the even mantissa; block 0 of the tensor writes s.
 *
 * The code of a value v with |v| <= F is formed on the binary32 bits: in the
 * subnormal range of the format (|v| < 2^(1-bias)) it is the integer
 * |v| / 2^(1-bias-m) rounded to nearest even (exact scaling by a power of
 * two, then rint); above it the binary32 significand is rounded to m bits
 * (add half an ulp of the target minus one, plus the target's lowest kept
 * bit, then truncate) and the exponent re-biased.  The sign of the code is
 * the sign bit of v.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace g355 {

namespace {

template <int FMT>
__device__ __forceinline__ uint32_t encode8(float v)
{
    const uint32_t bits = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t a = bits & 0x7FFFFFFFu;
    const float av = __builtin_bit_cast(float, a);
    uint32_t code;
    if constexpr (FMT == 0) {
        /* E4M3FN: bias 7, 3 mantissa bits, smallest normal 2^-6, step 2^-9 */
        if (a < 0x3C800000u) {
            code = (uint32_t)__builtin_rintf(av * 512.0f);
        } else {
            const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
            code = (r >> 20) - ((127u - 7u) << 3);
        }
    } else {
        /* E5M2: bias 15, 2 mantissa bits, smallest normal 2^-14, step 2^-16 */
        if (a < 0x38800000u) {
            code = (uint32_t)__builtin_rintf(av * 65536.0f);
        } else {
            const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
            code = (r >> 21) - ((127u - 15u) << 2);
        }
    }
    return sign | code;
}

__device__ __forceinline__ float load_elem(const void *x, int64_t i, int32_t src)
{
    if (src == 0) return ((const float *)x)[i];
    const uint16_t h = ((const uint16_t *)x)[i];
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

/* 8 consecutive elements starting at a 16-byte (bf16) or 32-byte (fp32)
 * aligned index.  Loaded as HIP's four-member vector structs: a bit cast
 * applied to a subscript of an extended vector has been lowered to element 0
 * for every subscript. */
__device__ __forceinline__ void load8(const void *x, int64_t i, int32_t src, float (&v)[8])
{
    if (src == 0) {
        const float4 a = *(const float4 *)((const float *)x + i);
        const float4 b = *(const float4 *)((const float *)x + i + 4);
        v[0] = a.x;
        v[1] = a.y;
        v[2] = a.z;
        v[3] = a.w;
        v[4] = b.x;
        v[5] = b.y;
        v[6] = b.z;
        v[7] = b.w;
    } else {
        const uint4 a = *(const uint4 *)((const uint16_t *)x + i);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __builtin_bit_cast(float, w[j] << 16);
            v[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
        }
    }
}

/* Share [lo, hi) of part `part` of P parts of n elements; with vec set the
 * shares are cut at multiples of 8 elements (n is then a multiple of 8). */
__device__ __forceinline__ void share(int64_t n, int32_t P, int32_t part, bool vec, int64_t &lo, int64_t &hi)
{
    if (vec) {
        const int64_t nv = n / 8;
        lo = nv * part / P * 8;
        hi = nv * (part + 1) / P * 8;
    } else {
        lo = n * part / P;
        hi = n * (part + 1) / P;
    }
}

__device__ __forceinline__ float block_max(float m, float *red)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
}

} /* namespace */

__global__ __launch_bounds__(256) void amax_kernel(QuantParams qp)
{
    __shared__ float red[4];
    const int64_t g = blockIdx.x / qp.parts;
    const int32_t part = (int32_t)(blockIdx.x % qp.parts);
    const char *xg = (const char *)qp.x + g * qp.n * (qp.src == 0 ? 4 : 2);
    int64_t lo, hi;
    share(qp.n, qp.parts, part, qp.vec != 0, lo, hi);
    float m = 0.0f;
    if (qp.vec) {
        /* two vectors in flight per thread */
        int64_t i = lo + 8 * (int64_t)threadIdx.x;
        for (; i + 8 * 256 < hi; i += 2 * 8 * 256) {
            float v[8], w[8];
            load8(xg, i, qp.src, v);
            load8(xg, i + 8 * 256, qp.src, w);
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fmaxf(fabsf(v[j]), fabsf(w[j])));
        }
        if (i < hi) {
            float v[8];
            load8(xg, i, qp.src, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
        }
    } else {
        for (int64_t i = lo + threadIdx.x; i < hi; i += 256) m = fmaxf(m, fabsf(load_elem(xg, i, qp.src)));
    }
    m = block_max(m, red);
    if (threadIdx.x == 0) qp.maxima[blockIdx.x] = m;
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(QuantParams qp)
{
    __shared__ float red[4];
    const int64_t g = blockIdx.x / qp.parts;
    const int32_t part = (int32_t)(blockIdx.x % qp.parts);
    float m = 0.0f;
    for (int32_t i = threadIdx.x; i < qp.parts; i += 256) m = fmaxf(m, qp.maxima[g * qp.parts + i]);
    const float amax = block_max(m, red);
    constexpr float F = FMT == 0 ? 448.0f : 57344.0f;
    /* correctly rounded binary32 division */
    const float s = amax > 0.0f ? amax / F : 1.0f;
    if (part == 0 && threadIdx.x == 0) qp.scale[g] = s;
    const char *xg = (const char *)qp.x + g * qp.n * (qp.src == 0 ? 4 : 2);
    uint8_t *qg = qp.q + g * qp.n;
    int64_t lo, hi;
    share(qp.n, qp.parts, part, qp.vec != 0, lo, hi);
    /* x / s rounded to nearest: with r the reciprocal of s rounded to
     * nearest, q0 = x r is within an ulp of the quotient and one residual
     * step q0 + (x - q0 s) r gives the quotient rounded to nearest
     * (Markstein's theorem; the residual is exact by the fused
     * multiply-add).  Quotients that would be subnormal in binary32 lie far
     * below the smallest 8-bit code, where either rounding gives a zero
     * code of the same sign. */
    const float r = 1.0f / s;
    auto code = [&](float v) __attribute__((always_inline)) {
        /* on the magnitude; the quotient's sign is v's (s > 0) */
        const float a = fabsf(v);
        const float q0 = a * r;
        const float e = __builtin_fmaf(-q0, s, a);
        const float t = fminf(__builtin_fmaf(e, r, q0), F);
        return encode8<FMT>(__builtin_copysignf(t, v));
    };
    auto quant8 = [&](int64_t i, const float (&v)[8]) __attribute__((always_inline)) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w0 |= code(v[j]) << (8 * j);
            w1 |= code(v[j + 4]) << (8 * j);
        }
        *(uint2 *)(qg + i) = make_uint2(w0, w1);
    };
    if (qp.vec) {
        /* two vectors in flight per thread */
        int64_t i = lo + 8 * (int64_t)threadIdx.x;
        for (; i + 8 * 256 < hi; i += 2 * 8 * 256) {
            float v[8], w[8];
            load8(xg, i, qp.src, v);
            load8(xg, i + 8 * 256, qp.src, w);
            quant8(i, v);
            quant8(i + 8 * 256, w);
        }
        if (i < hi) {
            float v[8];
            load8(xg, i, qp.src, v);
            quant8(i, v);
        }
    } else {
        for (int64_t i = lo + threadIdx.x; i < hi; i += 256) qg[i] = (uint8_t)code(load_elem(xg, i, qp.src));
    }
}

hipError_t launch_quantize(const QuantParams &qp0, hipStream_t stream)
{
    QuantParams qp = qp0;
    const uint32_t grid = (uint32_t)(qp.batch * qp.parts);
    hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(256), 0, stream, qp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (qp.fmt == 0)
        hipLaunchKernelGGL(quantize_kernel<0>, dim3(grid), dim3(256), 0, stream, qp);
    else
        hipLaunchKernelGGL(quantize_kernel<1>, dim3(grid), dim3(256), 0, stream, qp);
    return hipGetLastError();
}

} /* namespace g355 */
