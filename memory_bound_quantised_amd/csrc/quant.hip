// Per-row int8 activation quantisation, optionally preceded by the prologue it
// absorbs ("Optimizing the Linear Kernel": the quantisation absorbs the
// RMSNorm or SwiGLU that precedes it).  One block of 256 threads per row.
//
//   RMSNorm:   ss = sum x^2 (fp64), r = 1/sqrtf((float)(ss/K) + 1e-6f), t = bf16(x*r)
//   weighted:  the same r, t = bf16(x*w*r) (x*w exact in fp32)
//   SwiGLU:    t = bf16(silu(g)*u), silu(g) = g / (1 + exp(-g)) in fp32
//   quant:     amax = max|t|, s = amax/127, q = clamp(rint(t/s), -127, 127)
// The fp64 sum makes ss independent of summation order for all practical
// inputs, so every rounding decision below is the same one the exact
// definition takes; the quantisation itself is fp32 with IEEE divide.
#include "mbq_internal.h"
#include "mbq.h"
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

// Prologue PRO (an MBQ_PRO_* value) of 8 consecutive columns: x (and, for
// SwiGLU, u; for the weighted norm, w) at column 8c.
template <int PRO>
__device__ __forceinline__ void prologue8(const uint16_t *xr, const uint16_t *ur, const uint16_t *w, int64_t c,
                                          float r, float (&t)[8]) {
    load8(xr + 8 * c, t);
    if constexpr (PRO == MBQ_PRO_RMSNORM_QUANT) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = bf16_bits_to_f32(f32_to_bf16_bits(t[i] * r));
    } else if constexpr (PRO == MBQ_PRO_WRMSNORM_QUANT) {
        float wv[8];
        load8(w + 8 * c, wv);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = bf16_bits_to_f32(f32_to_bf16_bits(t[i] * wv[i] * r));
    } else if constexpr (PRO == MBQ_PRO_SWIGLU_QUANT) {
        float uv[8];
        load8(ur + 8 * c, uv);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = swiglu_bf16f(t[i], uv[i]);
    }
}

template <int PRO>
__global__ __launch_bounds__(kThreads) void prologue_quant_kernel(const uint16_t *__restrict__ x, int64_t x_stride,
                                                                  const uint16_t *__restrict__ u, int64_t u_stride,
                                                                  const uint16_t *__restrict__ w,
                                                                  uint16_t *__restrict__ h, int64_t K,
                                                                  int8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ double red_d[kThreads / 64];
    __shared__ float red_f[kThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t *xr = x + m * x_stride;
    const uint16_t *ur = u ? u + m * u_stride : nullptr;
    const int64_t chunks = K / 8;

    float r = 1.0f;
    if constexpr (PRO == MBQ_PRO_RMSNORM_QUANT || PRO == MBQ_PRO_WRMSNORM_QUANT) {
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

    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
        float t[8];
        prologue8<PRO>(xr, ur, w, c, r, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
    amax = block_reduce(amax, [](float a, float b) { return fmaxf(a, b); }, red_f);
    const float sc = amax / 127.0f;
    if (threadIdx.x == 0) s[m] = sc;

    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
        float t[8];
        prologue8<PRO>(xr, ur, w, c, r, t);
        uint32_t packed[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float qv = 0.0f;
            if (amax != 0.0f) {
                qv = rintf(t[i] / sc);
                qv = fminf(fmaxf(qv, -127.0f), 127.0f);
            }
            packed[i >> 2] |= ((uint32_t)(int)qv & 0xFFu) << (8 * (i & 3));
        }
        *reinterpret_cast<uint2 *>(q + m * K + 8 * c) = make_uint2(packed[0], packed[1]);
        if (PRO == MBQ_PRO_SWIGLU_QUANT && h) {
            uint32_t hp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hp[i] = f32_to_bf16_bits(t[2 * i]) | (f32_to_bf16_bits(t[2 * i + 1]) << 16);
            *reinterpret_cast<uint4 *>(h + m * K + 8 * c) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
        }
    }
}

}  // namespace

hipError_t launch_prologue_quant(int pro, int64_t M, int64_t K, const void *x, int64_t x_stride,
                                 const void *u, int64_t u_stride, const void *w, void *h, int8_t *q,
                                 float *s, hipStream_t st) {
    const dim3 grid((unsigned)M), block(kThreads);
    const uint16_t *xs = (const uint16_t *)x, *us = (const uint16_t *)u, *ws = (const uint16_t *)w;
    uint16_t *hs = (uint16_t *)h;
    switch (pro) {
        case MBQ_PRO_RMSNORM_QUANT:
            prologue_quant_kernel<MBQ_PRO_RMSNORM_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
        case MBQ_PRO_WRMSNORM_QUANT:
            prologue_quant_kernel<MBQ_PRO_WRMSNORM_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
        case MBQ_PRO_SWIGLU_QUANT:
            prologue_quant_kernel<MBQ_PRO_SWIGLU_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
        default:
            prologue_quant_kernel<MBQ_PRO_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
    }
    return hipGetLastError();
}

}  // namespace mbq
