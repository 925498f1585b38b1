// One activation row through the quantisation prologue and the per-row int8
// quantisation, for a block of NT threads: the definition behind
// mbq_quantize_act and its prologue forms ("Optimizing the Linear Kernel":
// the quantisation absorbs the RMSNorm or SwiGLU that precedes it).
//
//   RMSNorm:   ss = sum x^2 (fp64), r = 1/sqrtf((float)(ss/K) + 1e-6f), t = bf16(x*r)
//   weighted:  the same r, t = bf16(x*w*r) (x*w exact in fp32)
//   SwiGLU:    t = bf16(silu(g)*u), silu(g) = g / (1 + exp(-g)) in fp32
//   quant:     amax = max|t|, s = amax/127, q = clamp(rint(t/s), -127, 127)
//
// The sum of squares runs in fp64 over products of bf16 values (16
// significant bits each): orders of summation differ by at most a few units
// of 2^-40 of the sum, far below the fp32 step of r, so a block of another
// size (another order) gives the same r, scale and codes unless ss / K lies
// that close to an fp32 rounding boundary.  The absolute maximum does not
// depend on the order.
#pragma once

#include "mbq_internal.h"
#include "../../include/mbq.h"

namespace mbq {

template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce_n(T v, Op op, T *smem) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) smem[w] = v;
    __syncthreads();
    T r = smem[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r = op(r, smem[i]);
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

// Quantise row xr (and ur, w) of K columns: every thread of the block takes
// the 8-column chunks c = tid, tid + NT, ...; put(c, lo, hi) receives chunk
// c's eight codes (little-endian bytes), and put_t(c, t), when PUT_T, its
// eight prologue outputs (the SwiGLU h).  Returns the row's scale, on every
// thread.  red_d, red_f: NT / 64 words of shared scratch each.
template <int PRO, int NT, bool PUT_T, typename Put, typename PutT>
__device__ __forceinline__ float quant_row(const uint16_t *xr, const uint16_t *ur, const uint16_t *w, int64_t K,
                                           double *red_d, float *red_f, Put put, PutT put_t) {
    const int64_t chunks = K / 8;
    float r = 1.0f;
    if constexpr (PRO == MBQ_PRO_RMSNORM_QUANT || PRO == MBQ_PRO_WRMSNORM_QUANT) {
        double ss = 0.0;
        for (int64_t c = threadIdx.x; c < chunks; c += NT) {
            float v[8];
            load8(xr + 8 * c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)v[i] * (double)v[i];
        }
        ss = block_reduce_n<NT>(ss, [](double a, double b) { return a + b; }, red_d);
        const float ms = (float)(ss / (double)K);
        r = 1.0f / sqrtf(ms + 1e-6f);
    }

    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < chunks; c += NT) {
        float t[8];
        prologue8<PRO>(xr, ur, w, c, r, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
    amax = block_reduce_n<NT>(amax, [](float a, float b) { return fmaxf(a, b); }, red_f);
    const float sc = amax / 127.0f;

    for (int64_t c = threadIdx.x; c < chunks; c += NT) {
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
        put(c, packed[0], packed[1]);
        if constexpr (PUT_T) put_t(c, t);
    }
    return sc;
}

}  // namespace mbq
