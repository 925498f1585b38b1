// Per-row int8 activation quantisation, optionally preceded by the weightless
// RMSNorm it absorbs ("Optimizing the Linear Kernel": the quantisation absorbs
// the RMSNorm that precedes it).  One block of 256 threads per row.
//
//   RMSNorm:  ss = sum x^2 (fp64), r = 1/sqrtf((float)(ss/K) + 1e-6f), t = bf16(x*r)
//   quant:    amax = max|t|, s = amax/127, q = clamp(rint(t/s), -127, 127)
// The fp64 sum makes ss independent of summation order for all practical
// inputs, so every rounding decision below is the same one the exact
// definition takes; the quantisation itself is fp32 with IEEE divide.
#include "mbq_internal.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

constexpr int kThreads = 256;

template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, Op op, T *smem) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) smem[w] = v;
    __syncthreads();
    T r = smem[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = op(r, smem[i]);
    return r;
}

__device__ __forceinline__ void load8(const uint16_t *p, float (&v)[8]) {
    const int4 raw = *reinterpret_cast<const int4 *>(p);
    const uint32_t u[4] = {(uint32_t)raw.x, (uint32_t)raw.y, (uint32_t)raw.z, (uint32_t)raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(u[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
    }
}

template <bool NORM>
__global__ __launch_bounds__(kThreads) void prologue_quant_kernel(const uint16_t *__restrict__ x,
                                                                  int64_t x_stride, int64_t K,
                                                                  int8_t *__restrict__ q,
                                                                  float *__restrict__ s) {
    __shared__ double red_d[kThreads / 64];
    __shared__ float red_f[kThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t *xr = x + m * x_stride;
    const int64_t chunks = K / 8;

    float r = 1.0f;
    if (NORM) {
        double ss = 0.0;
        for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
            float v[8];
            load8(xr + 8 * c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)v[i] * (double)v[i];
        }
        ss = block_reduce(ss, [](double a, double b) { return a + b; }, red_d);
        const float ms = (float)(ss / (double)K);
        r = 1.0f / sqrtf(ms + 1e-6f);
    }
    auto t_of = [&](float v) -> float {
        return NORM ? bf16_bits_to_f32(f32_to_bf16_bits(v * r)) : v;
    };

    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
        float v[8];
        load8(xr + 8 * c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t_of(v[i])));
    }
    amax = block_reduce(amax, [](float a, float b) { return fmaxf(a, b); }, red_f);
    const float sc = amax / 127.0f;
    if (threadIdx.x == 0) s[m] = sc;

    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
        float v[8];
        load8(xr + 8 * c, v);
        uint32_t packed[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float qv = 0.0f;
            if (amax != 0.0f) {
                qv = rintf(t_of(v[i]) / sc);
                qv = fminf(fmaxf(qv, -127.0f), 127.0f);
            }
            packed[i >> 2] |= ((uint32_t)(int)qv & 0xFFu) << (8 * (i & 3));
        }
        *reinterpret_cast<uint2 *>(q + m * K + 8 * c) = make_uint2(packed[0], packed[1]);
    }
}

}  // namespace

hipError_t launch_prologue_quant(bool rmsnorm, int64_t M, int64_t K, const void *x, int64_t x_stride,
                                 int8_t *q, float *s, hipStream_t st) {
    if (rmsnorm)
        prologue_quant_kernel<true><<<dim3((unsigned)M), dim3(kThreads), 0, st>>>(
            (const uint16_t *)x, x_stride, K, q, s);
    else
        prologue_quant_kernel<false><<<dim3((unsigned)M), dim3(kThreads), 0, st>>>(
            (const uint16_t *)x, x_stride, K, q, s);
    return hipGetLastError();
}

}  // namespace mbq
