// The fused decode-step walk: one persistent kernel streams every weight
// matrix of a decode step ("What is the bottleneck?" on the page "Doubling
// LLM token rates in ComfyUI": a step reads all weights once, so the bus must
// stay busy from the first matrix to the last; "Optimizing the Linear
// Kernel": the activation quantisation, with the RMSNorm before it, is fused
// into the linear as a prologue).
//
// Work: ops with the same input form a phase (q/k/v, o, gate/up, down).  A
// phase's 64-row x 128-k tiles are ordered (k chunk of 1024, row block,
// group) and cut into equal contiguous ranges, one per wave.  Ordering by k
// chunk first keeps the k range a workgroup touches -- and so the activations
// it quantises into LDS -- to one or two chunks.
//
// Weight stream decoupled from the dataflow: a fifth wave per workgroup, the
// loader, streams the tiles of the four compute waves into per-wave rings in
// LDS (LDS-DMA loads, a fixed number of tiles in flight), across phase
// boundaries and without waiting for anything but ring space, since weights
// do not depend on activations.  While the compute waves wait for a phase's
// input, the bus keeps delivering the next tiles.
//
// Dataflow instead of grid barriers.  Everything one wave hands to another is
// a 64-bit word whose high half is an epoch tag, so one load fetches and
// validates it:
//   - a wave that finishes part of a row block stores its fp32 partial;
//   - the owner of the row block's last tile gathers the parts in a fixed
//     order (bitwise reproducible results), writes the bf16 outputs, a tagged
//     copy of them for the consumer, and the block's row statistics
//     (max |y|, fp64 sum of y^2);
//   - a workgroup starts a phase by loading the statistics of its input and
//     the input columns it needs, re-polling any word whose tag is stale.
// Every wait is bounded; a wait that gives up sets the plan's error word and
// the kernel still runs to completion.
#pragma once

#include "mbq_internal.h"
#include "mbq.h"
#include "mbq_kernels.h"
#include "mbq_seq.h"

namespace mbq {

namespace {

constexpr int64_t kSpinLimit = 1ll << 23;    // polls before a wait gives up

__device__ __forceinline__ uint32_t make_tag(uint32_t gen, int phase) {
    return gen * 1024u + (uint32_t)(phase + 1);
}
__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t tag) { return (uint64_t)v | ((uint64_t)tag << 32); }
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }

// Plan data is read-only for the whole launch.  Where it is read at
// wave-uniform addresses it goes through the constant address space, so the
// compiler uses scalar loads and the vector-memory counter stays with the
// weight stream (waiting on a tile never waits on a plan read).
#define MBQ_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ T cload(const T *p, int64_t i = 0) {
    static_assert(sizeof(T) % 4 == 0, "plan records are whole dwords");
    T out;
    const uint32_t MBQ_CONST *src = (const uint32_t MBQ_CONST *)(p + i);
    uint32_t *dst = reinterpret_cast<uint32_t *>(&out);
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 4); ++k) dst[k] = src[k];
    return out;
}

// Dynamic LDS: [activations: M rows x q_stride bytes][partial slots: waves x
// slots x M x 64 floats][metadata slot 0][metadata slot 1].  A metadata slot
// holds a phase record followed by the workgroup's block for that phase.
extern __shared__ __align__(16) int8_t g_lds[];

struct Lay {
    int qs;           // LDS bytes per activation row
    int slots;        // LDS partial slots per wave
    int meta_off;     // LDS offset of metadata slot 0
    int meta_bytes;   // bytes per metadata slot
    int seg_cap;      // segment entries per block
    int blk_bytes;    // bytes per block
    int grid;
    int n_phases;
    int part_stride;  // contributions per parity half of the partial area
    int ring_off;     // LDS offset of the weight rings
    int ring_slots;   // tiles per compute wave's ring
    int rec_off;      // LDS offset of the loader's run records (kSeqWaves x kRecBuf)
    int hdr_off;      // LDS offset of the per-slot run headers (kSeqWaves x kMaxRingSlots words)
    // Plan pointers used every phase, read once at kernel start: re-reading
    // them from the plan costs a scalar-cache round trip at every phase entry.
    const SeqPhase *phases;
    const uint8_t *blocks;
    uint64_t *stats;
    int64_t stat_stride, stat_rep;
    uint64_t *partials;
};

// ---------------------------------------------------------------- LDS control words
//
// [0..3] tiles arrived in each compute wave's ring (the loader adds), [4..7]
// tiles each compute wave has consumed (it stores), [8] barrier arrivals,
// [9] barrier generation.
__shared__ uint32_t g_ctl[16];
constexpr int kCtlArrived = 0, kCtlConsumed = 4, kCtlBarCount = 8, kCtlBarGen = 9;

#define MBQ_LDS __attribute__((address_space(3)))
__device__ __forceinline__ MBQ_LDS uint32_t *ctl(int i) { return (MBQ_LDS uint32_t *)&g_ctl[i]; }
__device__ __forceinline__ uint32_t ctl_load(int i) {
    return __hip_atomic_load(ctl(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void ctl_store(int i, uint32_t v) {
    __hip_atomic_store(ctl(i), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The loader's own LDS operations, as inline assembly.  After an LDS-DMA
// load the compiler waits for every vector-memory operation in flight before
// each later LDS access it generates (it cannot tell the DMA's destination
// from other LDS words), which would drain the weight stream at every tile.
// The loader orders its LDS accesses against its DMA loads itself (a tile is
// published only after its own wait on the vector-memory counter), so these
// forms carry no such wait.  A read waits for its own result inside the
// same block; the outputs are always used.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const MBQ_LDS void *)p;
}
__device__ __forceinline__ void lds_add_u32_asm(uint32_t addr, uint32_t v) {
    asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_u32_asm(uint32_t addr, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t lds_read_u32_asm(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ v4i lds_read_b128_asm(uint32_t addr) {
    v4i v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// Wait for this wave's LDS operations (lgkmcnt 0; vector-memory counts untouched).
__device__ __forceinline__ void lds_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float *lds_partials(const Lay &L, int M) { return reinterpret_cast<float *>(g_lds + M * L.qs); }
__device__ __forceinline__ int8_t *lds_meta(const Lay &L, int p) { return g_lds + L.meta_off + (p & 1) * L.meta_bytes; }
__device__ __forceinline__ const SeqPhase *meta_phase(const Lay &L, int p) {
    return reinterpret_cast<const SeqPhase *>(lds_meta(L, p));
}
__device__ __forceinline__ const SeqWgHead *meta_head(const Lay &L, int p) {
    return reinterpret_cast<const SeqWgHead *>(lds_meta(L, p) + sizeof(SeqPhase));
}
__device__ __forceinline__ const SeqWgSeg *meta_seg(const Lay &L, int p) {
    return reinterpret_cast<const SeqWgSeg *>(lds_meta(L, p) + sizeof(SeqPhase) + sizeof(SeqWgHead));
}
__device__ __forceinline__ const SeqFin *meta_fin(const Lay &L, int p) {
    return reinterpret_cast<const SeqFin *>(lds_meta(L, p) + sizeof(SeqPhase) + sizeof(SeqWgHead) +
                                            L.seg_cap * sizeof(SeqWgSeg));
}

// Metadata of phase p for this workgroup: every thread loads up to
// kMetaIters dwords now and stores them into the LDS slot later, so the
// loads overlap whatever the workgroup waits for in between.
constexpr int kMetaIters = kMetaMaxBytes / 4 / kSeqThreads;
__device__ __forceinline__ void fetch_meta(const SeqPlan *P, const Lay &L, int p, int wg,
                                           uint32_t (&v)[kMetaIters]) {
    if (p >= L.n_phases) return;
    constexpr int kPhDw = (int)(sizeof(SeqPhase) / 4);
    const int n_dw = kPhDw + L.blk_bytes / 4;
    const uint32_t *ph = reinterpret_cast<const uint32_t *>(L.phases + p);
    const uint32_t *blk =
        reinterpret_cast<const uint32_t *>(L.blocks + ((int64_t)p * L.grid + wg) * L.blk_bytes);
    // Every thread loads all kMetaIters words, clamped into the record: a
    // conditional load into this array makes the compiler copy (and so wait
    // for) the loaded value at once, which would put a memory round trip at
    // the start of every phase.
#pragma unroll
    for (int it = 0; it < kMetaIters; ++it) {
        const int i = min((int)threadIdx.x + it * kSeqThreads, n_dw - 1);
        const uint32_t *src = i < kPhDw ? ph + i : blk + (i - kPhDw);
        v[it] = *gptr(src);
    }
}
// Every word is written, the clamped ones onto the record's last word (which
// they hold): a loaded word left unwritten on some path would stay pending in
// the compiler's view, and it would then wait for every memory operation in
// flight at the next phase's entry.
__device__ __forceinline__ void store_meta(const Lay &L, int p, const uint32_t (&v)[kMetaIters]) {
    if (p >= L.n_phases) return;
    const int n_dw = (int)(sizeof(SeqPhase) / 4) + L.blk_bytes / 4;
    uint32_t *dst = reinterpret_cast<uint32_t *>(lds_meta(L, p));
#pragma unroll
    for (int it = 0; it < kMetaIters; ++it) dst[min((int)threadIdx.x + it * kSeqThreads, n_dw - 1)] = v[it];
}

__device__ __forceinline__ bool gave_up(const SeqPlan *P, int64_t &spins) {
    if ((++spins & 255) == 0 && load_shared(P->err) != 0u) return true;
    if (spins > kSpinLimit) {
        store_shared(P->err, 1u);
        return true;
    }
    __builtin_amdgcn_s_sleep(2);
    return false;
}

// ---------------------------------------------------------------- vector-memory budget
//
// A wave's outstanding vector-memory instructions (loads and stores alike)
// are tracked by a counter whose waits encode at most 63: with more in flight
// a wait for a given load can return before that load has landed.  Compute
// waves issue no weight loads (the loader does), but their partial,
// output and statistics stores can still be in flight when they poll, so
// every batch of loads first makes room for itself: vm_room<n>() waits until
// at most 63 - n operations are outstanding.  Batch sizes leave room for the
// next phase's metadata loads (kMetaIters) and are at most 4.
constexpr int kVmemLimit = 63;
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0xF << 8); }
template <int N>
__device__ __forceinline__ void vm_room() {
    static_assert(N >= 1 && N <= kVmemLimit, "a batch must fit the counter");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kVmemLimit - N));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
constexpr int batch_within(int free_slots, int per_item) {
    return free_slots / per_item >= 4 ? 4 : free_slots / per_item;
}
// Statistics records per lane per round trip (wave 0): also at most 24
// words in flight, which bounds the registers the batch holds (two per word).
template <int M>
constexpr int stat_batch() { return batch_within(24, 3 * M) >= 1 ? batch_within(24, 3 * M) : 1; }
// Input words (2 columns each) per thread per round trip: at most 16 words
// in flight per thread (the registers a batch holds, two per word).
template <int M, bool X>
constexpr int x_batch() { return batch_within(16, M) >= 1 ? batch_within(16, M) : 1; }

// Barrier of the four compute waves (the loader never joins one: it must
// keep streaming).  LDS executes each wave's operations in order, so every
// LDS write a wave made before arriving is visible to a wave that has seen
// the generation change.  Bounded like every other wait.
__device__ __forceinline__ void cw_sync(const SeqPlan *P) {
    const int lane = threadIdx.x & 63;
    lds_done();
    const uint32_t gen = uniform((int)ctl_load(kCtlBarGen));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctl(kCtlBarCount), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
    if (old == kSeqWaves - 1) {
        if (lane == 0) {
            ctl_store(kCtlBarCount, 0u);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            ctl_store(kCtlBarGen, gen + 1);
        }
    } else {
        int64_t spins = 0;
        while (uniform((int)ctl_load(kCtlBarGen)) == (int)gen) {
            if (++spins > kSpinLimit) {
                store_shared(P->err, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    lds_done();
}

// True if any lane of the wave passes true.
__device__ __forceinline__ bool wave_any(bool b) { return __builtin_amdgcn_ballot_w64(b) != 0; }

// Publish one stats record (word 0 of copy 0 at rec, word c of copy k at
// rec + k * rep + c * stride) from per-lane values: v feeds the sum of
// squares, a the maximum magnitude (lanes past the stats rows pass 0).  Lane
// 63 holds the reductions; every lane then writes one (copy, word) of the
// record, kStatReplicas copies of each word side by side in lane order, so the
// 3M words of all copies take 3M / 8 stores (rounded up), not 3M: every store
// counts against the wave's 63 memory operations in flight until it has
// reached memory.
template <int M>
__device__ __forceinline__ void publish_stats(uint64_t *rec, int64_t stride, int64_t rep, const float (&v)[M],
                                              const float (&a)[M], uint32_t tag, int lane) {
    uint32_t w[3 * M];   // the record's words (wave-uniform)
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const double ss = wave_sum63((double)v[m] * (double)v[m]);
        const float am = wave_max63(fabsf(a[m]));
        const uint64_t bits = (uint64_t)__double_as_longlong(ss);
        w[3 * m + 1] = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, 63);
        w[3 * m + 2] = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), 63);
        w[3 * m] = (uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(am), 63);
    }
    static_assert(64 % kStatReplicas == 0, "whole words per store");
    constexpr int kWordsPerStore = 64 / kStatReplicas;
    const int k = lane % kStatReplicas;
#pragma unroll
    for (int c0 = 0; c0 < 3 * M; c0 += kWordsPerStore) {
        const int c = c0 + lane / kStatReplicas;
        uint32_t val = w[c0];
#pragma unroll
        for (int i = 1; i < kWordsPerStore && c0 + i < 3 * M; ++i) val = c == c0 + i ? w[c0 + i] : val;
        if (c < 3 * M) store_shared(rec + k * rep + c * stride, tagged(val, tag));
    }
}

// ---------------------------------------------------------------- kernel-start stats of external inputs

template <int M>
__device__ void external_stats(const SeqPlan *P, int w, int waves, int lane, uint32_t gen) {
    const int n_ext_rb = cload(&P->n_ext_rb), n_ext = cload(&P->n_ext);
    const SeqExt *ext = cload(&P->ext);
    uint64_t *stats = cload(&P->stats);
    const int64_t stride = cload(&P->stat_stride), rep = cload(&P->stat_rep);
    for (int b = w; b < n_ext_rb; b += waves) {
        vm_room<2 * M + 1>();
        int e = 0;
        while (e + 1 < n_ext && b >= cload(ext, e + 1).rb_first) ++e;
        const SeqExt x = cload(ext, e);
        const int rb = b - x.rb_first;
        const int col = rb * 64 + lane;
        const uint32_t tag = make_tag(gen, -1);
        const float wv = x.norm_w && col < x.K ? bf16_bits_to_f32(*gptr(x.norm_w + col)) : 1.0f;
        float v[M], a[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            v[m] = 0.0f;
            if (col < x.K) {
                const uint32_t word = *gptr(x.in + (int64_t)m * x.in_stride2 + (col >> 1));
                v[m] = bf16_bits_to_f32((word >> (16 * (col & 1))) & 0xFFFFu);
                if (x.in2) {
                    const uint32_t uw = *gptr(x.in2 + (int64_t)m * x.in2_stride2 + (col >> 1));
                    v[m] = swiglu_bf16f(v[m], bf16_bits_to_f32((uw >> (16 * (col & 1))) & 0xFFFFu));
                }
            }
            if (x.in2) {   // hand the gated values over in pairs, like a finaliser
                const uint32_t hb = f32_to_bf16_bits(v[m]);
                const uint32_t ho = dpp_u32<kDppQuadSwap1>(hb);   // the odd neighbour's value
                if (!(lane & 1) && col < x.K)
                    store_shared(x.xt + (int64_t)m * (x.K >> 1) + (col >> 1), tagged(hb | (ho << 16), tag));
            }
            a[m] = v[m] * wv;   // exact: both factors are bf16
        }
        publish_stats<M>(stats + x.rec + rb, stride, rep, v, a, tag, lane);
    }
}

// ---------------------------------------------------------------- phase prologue (workgroup-wide)

// int8 code of t at scale s (rinv = 1 / s): rint(t / s) clamped to +-127.
// The product t * rinv is within two ulps of the correctly rounded quotient,
// so it rounds to the same integer unless it lies next to a half-integer;
// only there (and when 1 / s overflows) is the quotient computed exactly.
// thr is 2^-14, or infinity where 1 / s overflows (always the exact quotient:
// t * rinv may then be 0 * inf); a zero scale comes with rinv = 0, which
// gives code 0 without the quotient.  A NaN distance (t * rinv not finite)
// takes the quotient too, which yields the same code as the product.
// The quotient sits under a wave-wide branch: it is rarely needed, and
// computed for every code it costs more than the rest of the code together.
__device__ __forceinline__ float quant_code(float t, float s, float rinv, float thr) {
    float x = t * rinv;
    const float fx = fabsf(x);
    const bool exact = !(fabsf(fx - floorf(fx) - 0.5f) >= thr);
    if (__builtin_amdgcn_ballot_w64(exact) != 0) x = exact ? t / s : x;
    return fminf(fmaxf(rintf(x), -127.0f), 127.0f);
}

// Input words of the workgroup's column range: a batch is XB words (two
// bf16 columns each) per thread, for each of the M rows, tagged 64-bit words
// from the producer's copy (or plain words of an input written before the
// walk).  Loading, settling (re-polling stale tags) and quantising are split
// so that the first batch can be loaded while wave 0 waits for the
// statistics.
template <int M, int XB>
struct Words {
    uint64_t v[XB][M];
};

template <int M, int XB>
__device__ __forceinline__ void issue_words(Words<M, XB> &w, const SeqPhase &ph, const SeqWgHead &h, int j0,
                                            int words) {
    vm_room<XB * M>();
    const bool tagged_in = ph.in_xt != nullptr;
    const uint64_t *xsrc = ph.in_xt + (h.k_lo >> 1);
    // unconditional loads of an index clamped into the range (words >= 1): a
    // conditional load would be waited for at once (see fetch_meta); the
    // words past the range are never used
#pragma unroll
    for (int u = 0; u < XB; ++u) {
        const int j = min(j0 + (int)threadIdx.x + u * kSeqThreads, words - 1);
#pragma unroll
        for (int m = 0; m < M; ++m)
            w.v[u][m] = tagged_in ? load_shared(xsrc + (int64_t)m * ph.in_stride2 + j)
                                  : (uint64_t)*gptr(ph.in + (int64_t)m * ph.in_stride2 + (h.k_lo >> 1) + j);
    }
}

template <int M, int XB>
__device__ __forceinline__ void settle_words(const SeqPlan *P, Words<M, XB> &w, const SeqPhase &ph,
                                             const SeqWgHead &h, int j0, int words, uint32_t want) {
    if (ph.in_xt == nullptr) return;
    const uint64_t *xsrc = ph.in_xt + (h.k_lo >> 1);
    int64_t spins = 0;
    for (;;) {
        bool stale = false;
#pragma unroll
        for (int u = 0; u < XB; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m)
                stale |= j0 + (int)threadIdx.x + u * kSeqThreads < words && tag_of(w.v[u][m]) != want;
        if (!wave_any(stale) || gave_up(P, spins)) break;
        vm_room<XB * M>();
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int j = j0 + threadIdx.x + u * kSeqThreads;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (j < words && tag_of(w.v[u][m]) != want) w.v[u][m] = load_shared(xsrc + (int64_t)m * ph.in_stride2 + j);
        }
    }
}

// Quantise the workgroup's input words [0, words) (bf16 pairs from column
// k_lo on) into LDS.  WEIGHTED multiplies by the norm weights before the
// RMSNorm scaling (x * w exactly, then * r).  With use_first, the first
// batch is `first`, already issued (and possibly settled).
template <int M, int XB, bool WEIGHTED, bool PRE>
__device__ __forceinline__ void quant_cols(const SeqPlan *P, const Lay &L, const SeqPhase &ph, const SeqWgHead &h,
                                           uint32_t want, int words, bool norm, const float (&s)[M],
                                           const float (&r)[M], const float (&rinv)[M], const bool (&rinv_ok)[M],
                                           const Words<M, XB> &first, bool use_first) {
    // the row's uniform cases as constants, so that no code branches on them
    float rq[M], thr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        rq[m] = s[m] != 0.0f ? rinv[m] : 0.0f;
        thr[m] = s[m] != 0.0f && !rinv_ok[m] ? INFINITY : 0x1p-14f;
    }
    for (int j0 = 0; j0 < words; j0 += XB * kSeqThreads) {
        Words<M, XB> xw;
        if (PRE && j0 == 0 && use_first) xw = first;
        else issue_words<M, XB>(xw, ph, h, j0, words);
        uint32_t ww[WEIGHTED ? XB : 1];
        if (WEIGHTED) {
            vm_room<XB>();
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                const int j = min(j0 + (int)threadIdx.x + u * kSeqThreads, words - 1);
                ww[WEIGHTED ? u : 0] = *gptr(ph.norm_w + (h.k_lo >> 1) + j);
            }
        }
        settle_words<M, XB>(P, xw, ph, h, j0, words, want);
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int j = j0 + threadIdx.x + u * kSeqThreads;
            if (j >= words) continue;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint32_t pair = (uint32_t)xw.v[u][m];
                uint32_t packed = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float t = bf16_bits_to_f32((pair >> (16 * e)) & 0xFFFFu);
                    if (WEIGHTED) t *= bf16_bits_to_f32((ww[WEIGHTED ? u : 0] >> (16 * e)) & 0xFFFFu);
                    const float tn = bf16_bits_to_f32(f32_to_bf16_bits(t * r[m]));
                    t = norm ? tn : t;
                    const float qv = quant_code(t, s[m], rq[m], thr[m]);
                    packed |= ((uint32_t)(int)qv & 0xFFu) << (8 * e);
                }
                *reinterpret_cast<uint16_t *>(g_lds + m * L.qs + 2 * j) = (uint16_t)packed;
            }
        }
    }
}

// Wave 0's poll of the statistics records [0, nrec) of the phase input: lane
// l takes records l, l + 64, ... and accumulates each row's maximum (am) and,
// with NORM, its sum of squares (ss).  A batch holds kStatBatch x 3M words:
// with NORM, kStatBatch whole records (maximum, sum-of-squares low and high
// words per row); without, only the maxima are read, M words per record, so a
// batch covers three times the records.
template <int M, bool NORM>
__device__ __forceinline__ void poll_stats(const SeqPlan *P, const uint64_t *stats, int64_t stride, int nrec,
                                           uint32_t want, int lane, double (&ss)[M], float (&am)[M]) {
    constexpr int kStatBatch = stat_batch<M>();
    constexpr int kRecs = NORM ? kStatBatch : 3 * kStatBatch;   // records per lane per batch
    // record (within the batch) and word (within the record) of slot (u, c)
    constexpr auto slot_rec = [](int u, int c) { return NORM ? u : 3 * u + c / M; };
    constexpr auto slot_word = [](int u, int c) { return NORM ? c : 3 * (c % M); };
    for (int base = 0; base < nrec; base += 64 * kRecs) {
        vm_room<kStatBatch * 3 * M>();
        uint64_t v[kStatBatch][3 * M];
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u)
#pragma unroll
            for (int c = 0; c < 3 * M; ++c) {
                const int i = base + lane + 64 * slot_rec(u, c);
                v[u][c] = i < nrec ? load_shared(stats + slot_word(u, c) * stride + i) : 0;
            }
        int64_t spins = 0;
        for (;;) {
            bool stale = false;
#pragma unroll
            for (int u = 0; u < kStatBatch; ++u)
#pragma unroll
                for (int c = 0; c < 3 * M; ++c)
                    stale |= base + lane + 64 * slot_rec(u, c) < nrec && tag_of(v[u][c]) != want;
            if (!wave_any(stale) || gave_up(P, spins)) break;
#pragma unroll
            for (int u = 0; u < kStatBatch; ++u)
#pragma unroll
                for (int c = 0; c < 3 * M; ++c) {
                    const int i = base + lane + 64 * slot_rec(u, c);
                    if (i < nrec && tag_of(v[u][c]) != want) v[u][c] = load_shared(stats + slot_word(u, c) * stride + i);
                }
        }
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) {
            if constexpr (NORM) {
                if (base + lane + 64 * u < nrec) {
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const uint64_t lo = v[u][3 * m + 1], hi = v[u][3 * m + 2];
                        am[m] = fmaxf(am[m], __uint_as_float((uint32_t)v[u][3 * m]));
                        ss[m] += __longlong_as_double((long long)(((hi & 0xFFFFFFFFull) << 32) | (lo & 0xFFFFFFFFull)));
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < 3 * M; ++c)
                    if (base + lane + 64 * slot_rec(u, c) < nrec)
                        am[c % M] = fmaxf(am[c % M], __uint_as_float((uint32_t)v[u][c]));
            }
        }
    }
}

// Quantise columns [k_lo, k_hi) of the phase input into LDS (int8, row stride
// q_stride), after the phase's RMSNorm with or without weights (a SwiGLU
// input arrives gated, in the tagged copy).  Row statistics come from
// the producer's stats records, reduced in a fixed order so that every
// workgroup derives bit-identical scales.  Wave 0 alone waits, first for the
// partial area of this phase's parity to be free, then for the statistics
// (the scales also serve the row blocks the workgroup finalises); the other
// waves sleep in the barrier.  Only then does every wave read its share of
// the input words: the producer wrote them before the statistics, so they are
// all but always current by then.  Keeping the waiting to one wave with
// contiguous reads keeps the polling traffic small: every workgroup polls at
// once, and a flood of polls slows every other memory request.  The next
// phase's metadata is fetched meanwhile.
template <int BITS, int M, bool X>
__device__ __forceinline__ void enter_phase(const SeqPlan *P, const Lay &L, int p, uint32_t gen, int wg,
                                            float (*s_sh)[kMaxM], float (*r_sh)[kMaxM]) {
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    uint32_t pre[kMetaIters];
    vm_room<kMetaIters>();
    fetch_meta(P, L, p + 1, wg, pre);
    const SeqPhase ph = *meta_phase(L, p);
    const SeqWgHead h = *meta_head(L, p);
    const bool norm = ph.prologue == MBQ_PRO_RMSNORM_QUANT || ph.prologue == MBQ_PRO_WRMSNORM_QUANT;
    const bool weighted = ph.norm_w != nullptr;
    const uint32_t want = make_tag(gen, ph.in_phase);
    const int words = (h.k_hi - h.k_lo) >> 1;          // bf16 pairs per activation row
    const bool has = h.k_hi > h.k_lo;
    const bool need_scale = has || h.n_fin > 0;   // finalising rescales by the input scale
    // The first batch of input words goes out before the statistics poll
    // (the producer wrote them before its statistics): waves 1..3 settle
    // theirs while wave 0 polls, wave 0 after.  Up to four rows only: more
    // would hold too many registers across the wait.
    constexpr int XB = x_batch<M, X>();
    constexpr bool kPre = M <= 4;
    Words<M, XB> xpre;
    if (kPre && has) issue_words<M, XB>(xpre, ph, h, 0, words);

    if (kPre && has && wave != 0) settle_words<M, XB>(P, xpre, ph, h, 0, words, want);
    if (wave == 0) {
        // the partial area of this phase's parity is free once the phase two back is finalised
        if (ph.wait_n > 0) {
            int64_t spins = 0;
            while (load_shared(ph.wait_count) < (uint32_t)ph.wait_n && !gave_up(P, spins)) {
            }
        }
        if (need_scale) {
            double ss[M];
            float am[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                ss[m] = 0.0;
                am[m] = 0.0f;
            }
            const int64_t stride = L.stat_stride;
            const uint64_t *stats = L.stats + (wg % kStatReplicas) * L.stat_rep + ph.in_rec;
            if (uniform(norm ? 1 : 0))
                poll_stats<M, true>(P, stats, stride, ph.in_nrec, want, lane, ss, am);
            else
                poll_stats<M, false>(P, stats, stride, ph.in_nrec, want, lane, ss, am);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const double tot = wave_sum63(ss[m]);
                const float amax = wave_max63(am[m]);
                float r = 1.0f, amax_t = amax;
                if (norm) {
                    const float ms = (float)(tot / (double)ph.K);
                    r = 1.0f / sqrtf(ms + 1e-6f);
                    // max |bf16(x * r)| = bf16(max|x| * r): rounding is monotonic (and with
                    // weights, x * w is exact in fp32, so the same holds for max|x w|)
                    amax_t = bf16_bits_to_f32(f32_to_bf16_bits(amax * r));
                }
                if (lane == 63) {
                    s_sh[p & 1][m] = amax_t / 127.0f;
                    r_sh[p & 1][m] = r;
                }
            }
        }
    }
    cw_sync(P);   // the scales from wave 0
    float s[M], r[M], rinv[M];
    bool rinv_ok[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        s[m] = s_sh[p & 1][m];
        r[m] = r_sh[p & 1][m];
        rinv[m] = 1.0f / s[m];
        rinv_ok[m] = fabsf(rinv[m]) < INFINITY;
    }
    // weighted RMSNorm: a copy of the loop of its own, so that the others
    // carry none of its registers
    if (X && uniform(weighted ? 1 : 0))
        quant_cols<M, XB, X, kPre>(P, L, ph, h, want, words, norm, s, r, rinv, rinv_ok, xpre, kPre && has);
    else
        quant_cols<M, XB, false, kPre>(P, L, ph, h, want, words, norm, s, r, rinv, rinv_ok, xpre, kPre && has);
    store_meta(L, p + 1, pre);
    cw_sync(P);
}

// ---------------------------------------------------------------- hand-over of a phase

// Sum contributions [c_begin, c_end) of the partial area (lane l's M tagged
// words of contribution c at area + (c * M + m) * 64 + l) in their fixed order
// into tot, re-polling stale words.  PAIR: contributions from index split on
// (a gate block's up partner) go to a fresh sum: the sums before it end up in
// tot2.
template <int M, bool PAIR>
__device__ __forceinline__ void gather_sum(const SeqPlan *P, const uint64_t *area, uint32_t tag, int c_begin,
                                           int c_end, int split, float (&tot)[M], float (&tot2)[M], int lane) {
#pragma unroll
    for (int m = 0; m < M; ++m) tot[m] = tot2[m] = 0.0f;
    constexpr int B = 32 / M;   // contributions per round trip (within the vector-memory counter)
    for (int c0 = c_begin; c0 < c_end; c0 += B) {
        vm_room<B * M>();
        uint64_t v[B][M];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const uint64_t *src = area + (int64_t)(c0 + u) * M * 64 + lane;
#pragma unroll
            for (int m = 0; m < M; ++m) v[u][m] = c0 + u < c_end ? load_shared(src + m * 64) : 0;
        }
        // re-poll every stale word together: one round trip per round
        int64_t spins = 0;
        for (;;) {
            bool stale = false;
#pragma unroll
            for (int u = 0; u < B; ++u)
#pragma unroll
                for (int m = 0; m < M; ++m) stale |= c0 + u < c_end && tag_of(v[u][m]) != tag;
            if (!wave_any(stale) || gave_up(P, spins)) break;
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const uint64_t *src = area + (int64_t)(c0 + u) * M * 64 + lane;
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (c0 + u < c_end && tag_of(v[u][m]) != tag) v[u][m] = load_shared(src + m * 64);
            }
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            if constexpr (PAIR) {
                // only a split inside the range starts the up sums here; a
                // range ending at the split is all gate sums (handled below)
                if (uniform(c0 + u == split && c0 + u < c_end)) {   // wave-uniform: plain blocks pay nothing
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        tot2[m] = tot[m];
                        tot[m] = 0.0f;
                    }
                }
            }
            if (c0 + u < c_end) {
#pragma unroll
                for (int m = 0; m < M; ++m) tot[m] += __uint_as_float((uint32_t)v[u][m]);
            }
        }
    }
    // a range wholly before the split holds gate sums only
    if constexpr (PAIR) {
        if (uniform(split >= c_end ? 1 : 0)) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                tot2[m] = tot[m];
                tot[m] = 0.0f;
            }
        }
    }
}

// A row block's outputs from its contribution sums: the bf16 outputs, their
// tagged copy and its stats record (the caller counts it as done).
template <int BITS, int M>
__device__ __forceinline__ void emit_rb(const SeqFin &f, uint32_t tag, const float (&tot)[M], const float *s_act,
                                        int64_t stat_stride, int64_t stat_rep, int lane) {
    using Lt = Layout<BITS>;
    const float unscale = 1.0f / (float)(1 << Lt::kAccShift);
    float yv[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t yb = f32_to_bf16_bits(s_act[m] * (tot[m] * unscale));
        const uint32_t hi = dpp_u32<kDppQuadSwap1>(yb);   // the odd neighbour's value
        const uint32_t pair = yb | (hi << 16);
        if (!(lane & 1) && lane < f.rows) {
            const int64_t idx = (int64_t)m * f.row_words + (lane >> 1);
            *gptr(f.out + idx) = pair;
            if (f.xt) store_shared(f.xt + idx, tagged(pair, tag));
        }
        yv[m] = lane < f.stat_rows ? bf16_bits_to_f32(yb) : 0.0f;
    }
    if (f.stats) publish_stats<M>(f.stats, stat_stride, stat_rep, yv, yv, tag, lane);
}

// The same for walks with weighted RMSNorms or SwiGLU pairs: a gate block
// paired with its up block (tot2: gate sums, tot: up sums) writes both outputs
// and hands over silu(gate) * up; a consumer's norm weights scale the maxima.
template <int BITS, int M>
__device__ __forceinline__ void emit_rb_full(const SeqFin &f, uint32_t tag, const float (&tot)[M],
                                             const float (&tot2)[M], const float *s_act, int64_t stat_stride,
                                             int64_t stat_rep, int lane) {
    using Lt = Layout<BITS>;
    const float unscale = 1.0f / (float)(1 << Lt::kAccShift);
    float yv[M], ya[M];
    if (uniform(f.out2 != nullptr ? 1 : 0)) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int64_t idx = (int64_t)m * f.row_words + (lane >> 1);
            const uint32_t gb = f32_to_bf16_bits(s_act[m] * (tot2[m] * unscale));
            const uint32_t ub = f32_to_bf16_bits(s_act[m] * (tot[m] * unscale));
            const uint32_t hb = f32_to_bf16_bits(swiglu_bf16f(bf16_bits_to_f32(gb), bf16_bits_to_f32(ub)));
            // the odd neighbours' values
            const uint32_t go = dpp_u32<kDppQuadSwap1>(gb), uo = dpp_u32<kDppQuadSwap1>(ub);
            const uint32_t ho = dpp_u32<kDppQuadSwap1>(hb);
            if (!(lane & 1) && lane < f.rows) {
                *gptr(f.out + idx) = gb | (go << 16);
                *gptr(f.out2 + idx) = ub | (uo << 16);
                if (f.xt) store_shared(f.xt + idx, tagged(hb | (ho << 16), tag));
            }
            yv[m] = ya[m] = lane < f.stat_rows ? bf16_bits_to_f32(hb) : 0.0f;
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint32_t yb = f32_to_bf16_bits(s_act[m] * (tot[m] * unscale));
            const uint32_t hi = dpp_u32<kDppQuadSwap1>(yb);   // the odd neighbour's value
            const uint32_t pair = yb | (hi << 16);
            if (!(lane & 1) && lane < f.rows) {
                const int64_t idx = (int64_t)m * f.row_words + (lane >> 1);
                *gptr(f.out + idx) = pair;
                if (f.xt) store_shared(f.xt + idx, tagged(pair, tag));
            }
            yv[m] = ya[m] = lane < f.stat_rows ? bf16_bits_to_f32(yb) : 0.0f;
        }
    }
    if (uniform(f.norm_w != nullptr ? 1 : 0)) {   // the consumer's weights scale the maxima
        vm_room<1>();
        const float wv = lane < f.stat_rows ? bf16_bits_to_f32(*gptr(f.norm_w + lane)) : 0.0f;
#pragma unroll
        for (int m = 0; m < M; ++m) ya[m] = yv[m] * wv;   // exact: both factors are bf16
    }
    if (f.stats) publish_stats<M>(f.stats, stat_stride, stat_rep, yv, ya, tag, lane);
}

// Workgroup-wide exit from phase p (every wave has parked its parts in LDS):
// merge the waves' parts of every segment the workgroup touched (in wave
// order) and publish one tagged partial per (segment, workgroup).
template <int M>
__device__ __forceinline__ void leave_phase(const SeqPlan *P, const Lay &L, int p, uint32_t gen) {
    cw_sync(P);
    const SeqWgHead h = *meta_head(L, p);
    const int lane = threadIdx.x & 63;
    const int j = uniform(threadIdx.x >> 6);
    const uint32_t tag = make_tag(gen, p);
    const float *lp = lds_partials(L, M) + lane;
    uint64_t *area = L.partials + (int64_t)(p & 1) * L.part_stride * 64 * M;
    for (int e = j; e < h.n_seg; e += kSeqWaves) {
        const SeqWgSeg sg = meta_seg(L, p)[e];
        float v[M];
#pragma unroll
        for (int m = 0; m < M; ++m) v[m] = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kSeqWaves; ++ww) {
            if (sg.slot[ww] != 0xFF) {
                const float *src = lp + ((ww * L.slots + sg.slot[ww]) * M) * 64;
#pragma unroll
                for (int m = 0; m < M; ++m) v[m] += src[m * 64];
            }
        }
        // row m's 64 words side by side: each store is one contiguous 512-byte
        // run (a lane's M words side by side would scatter every store over
        // M times as many lines, each written through in part)
        uint64_t *dst = area + (int64_t)sg.cidx * M * 64 + lane;
#pragma unroll
        for (int m = 0; m < M; ++m) store_shared(dst + m * 64, tagged(__float_as_uint(v[m]), tag));
    }
}

// Contributions above which the waves of a finaliser with one or two row
// blocks share each block's gather (the fixed-order sum of the parts).
constexpr int kShareContribs = 8;

// A finalising workgroup's row blocks of phase p, spread over its waves.
// With one or two blocks and more than kShareContribs contributions, 4 / n_fin
// waves share each block: each sums a contiguous quarter (or half) of its
// contributions, and the block's first wave adds those sums in wave order (a
// fixed order, so results stay reproducible) and emits the block.
// c_sh: kSeqWaves x (X ? 2 : 1) x M x 64 floats of LDS.
// Inline: a call would wait for every outstanding store on entry and exit.
template <int BITS, int M, bool X>
__device__ __forceinline__ void finalize_phase(const SeqPlan *P, const Lay &L, int p, uint32_t gen,
                                            const float *s_act, float *c_sh) {
    const SeqWgHead h = *meta_head(L, p);
    const int lane = threadIdx.x & 63;
    const int j = uniform(threadIdx.x >> 6);
    const uint32_t tag = make_tag(gen, p);
    const uint64_t *area = L.partials + (int64_t)(p & 1) * L.part_stride * 64 * M;
    uint32_t *fin_count = meta_phase(L, p)->fin_count;
    const int64_t stat_stride = L.stat_stride, stat_rep = L.stat_rep;
    // The choice depends on the plan alone, never on M, so that a row's sums
    // are added in the same order whatever the number of rows (a walk of M
    // rows gives each row the bits of that row's own walk).
    bool share = false;
    if (h.n_fin >= 1 && h.n_fin <= 2)
        for (int i = 0; i < h.n_fin; ++i) {
            const SeqFin &f = meta_fin(L, p)[i];
            share |= f.nc + f.nc_2 > kShareContribs;
        }
    share = uniform(share ? 1 : 0) != 0;
    // shared: wave j takes part j % g of block j / g (one pass); else wave j
    // takes blocks j, j + 4, ... whole
    const int g = share ? kSeqWaves / h.n_fin : 1;
    const int part = share ? j % g : 0;
    uint32_t done = 0;
    for (int i = share ? j / g : j; i < h.n_fin; i += kSeqWaves) {
        const SeqFin f = meta_fin(L, p)[i];
        const int n_all = f.nc + f.nc_2;
        const int a = f.c0 + n_all * part / g, b = f.c0 + n_all * (part + 1) / g;
        float tot[M], tot2[M];
        if constexpr (X)
            gather_sum<M, true>(P, area, tag, a, b, f.nc_2 > 0 ? f.c0 + f.nc : -1, tot, tot2, lane);
        else
            gather_sum<M, false>(P, area, tag, a, b, -1, tot, tot2, lane);
        if (share) {
            constexpr int NS = X ? 2 : 1;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                c_sh[((j * NS + 0) * M + m) * 64 + lane] = tot[m];
                if constexpr (X) c_sh[((j * NS + 1) * M + m) * 64 + lane] = tot2[m];
            }
            cw_sync(P);   // every wave passes here exactly once
            if (part != 0) break;
#pragma unroll
            for (int m = 0; m < M; ++m) tot[m] = tot2[m] = 0.0f;
            for (int w = j; w < j + g; ++w) {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    tot[m] += c_sh[((w * NS + 0) * M + m) * 64 + lane];
                    if constexpr (X) tot2[m] += c_sh[((w * NS + 1) * M + m) * 64 + lane];
                }
            }
        }
        if constexpr (X) {
            emit_rb_full<BITS, M>(f, tag, tot, tot2, s_act, stat_stride, stat_rep, lane);
            done += f.out2 ? 2u : 1u;
        } else {
            emit_rb<BITS, M>(f, tag, tot, s_act, stat_stride, stat_rep, lane);
            ++done;
        }
    }
    // one count per wave: the row blocks whose contributions it has read
    if (done > 0 && lane == 0) counter_add(fin_count, done);
}

// ---------------------------------------------------------------- the weight stream

template <int BITS>
struct Slot {
    v4i w[Layout<BITS>::kSlabs];
    v2u sc;
    uint32_t hdr;   // the run header if this tile opens a run, else 0
};

// Tiles each loader keeps in flight: enough bytes per CU for the bus to stay
// busy, few enough that a poll from the same CU is not queued behind a long
// line of weight loads.  Measured on 27B- and 9B-shaped walks: W4 3 tiles up
// to four rows (4 cost 0.5-1 %, 2 cost 5 %), 4 from five rows on (3 cost
// 1.7 % at M = 8); W6 2 tiles (3 cost 1 % at M = 1 and 3).
// The window also fixes the vector-memory wait after each tile, so it must
// stay within the 63-op counter: (tiles - 1) x loads per tile <= 63.
constexpr int loader_window_of(int bits, int m) { return bits == 4 ? (m <= 4 ? 3 : 4) : 2; }
template <int BITS, int M>
constexpr int loader_window() { return loader_window_of(BITS, M); }
template <int BITS>
constexpr int loads_per_tile() { return Layout<BITS>::kSlabs + 1; }
// The loader's wait takes one of two immediates: every window is the one of
// M = 1 or the one of M = kMaxM, and the latter is the largest.
constexpr bool two_windows(int bits) {
    const int lo = loader_window_of(bits, 1), hi = loader_window_of(bits, kMaxM);
    for (int m = 1; m <= kMaxM; ++m)
        if (loader_window_of(bits, m) != lo && loader_window_of(bits, m) != hi) return false;
    return lo <= hi;
}
static_assert(two_windows(4) && two_windows(6), "loader windows");
static_assert((loader_window<4, kMaxM>() - 1) * loads_per_tile<4>() <= kVmemLimit &&
                  (loader_window<6, kMaxM>() - 1) * loads_per_tile<6>() <= kVmemLimit,
              "loader window within vmcnt");
constexpr int kLdsDmaNt = 2;
// Offset of a tile's LDS/global base from its start: the slabs and scales lie
// within +-kDmaMid of it, inside the instruction offset's range (+-4 KiB).
template <int BITS>
constexpr int kDmaMid = BITS == 4 ? 2048 : 3072;
static_assert(Layout<4>::kWeightBytes - kDmaMid<4> < 4096 && Layout<6>::kWeightBytes - kDmaMid<6> < 4096,
              "DMA offsets within range");
// The tile's scales (128 bytes at kWeightBytes) on lanes 0..7, same base.
template <int BITS>
__device__ __forceinline__ void dma_scales(const uint8_t *g16, int8_t *dst) {
    constexpr int kOff = Layout<BITS>::kWeightBytes - kDmaMid<BITS>;
    __builtin_amdgcn_global_load_lds((const MBQ_GLOBAL void *)g16, (MBQ_LDS void *)dst, 16, kOff, kLdsDmaNt);
}
// Slab J.. of a tile from g16 (the lane's address at the tile's base) into
// LDS at dst (the slot's base); the instruction offset must be a constant.
template <int BITS, int J>
__device__ __forceinline__ void dma_slabs(const uint8_t *g16, int8_t *dst) {
    if constexpr (J < Layout<BITS>::kSlabs) {
        __builtin_amdgcn_global_load_lds((const MBQ_GLOBAL void *)g16, (MBQ_LDS void *)dst, 16,
                                         J * kSlab - kDmaMid<BITS>, kLdsDmaNt);
        dma_slabs<BITS, J + 1>(g16, dst);
    }
}   // cache policy of the LDS-DMA loads: non-temporal

// Position in a compute wave's LDS ring.
struct RingPos {
    int gt;         // tiles of this wave consumed so far (all phases)
    int slot;       // ring slot of tile gt
    int arrived;    // last arrival count read
};

// Read the wave's next tile and its run header from its ring (waiting for
// the loader if needed), then hand the slot back.
template <int BITS>
__device__ __forceinline__ void take_tile(const SeqPlan *P, const Lay &L, int wi, int lane, RingPos &rp,
                                          Slot<BITS> &s) {
    using Lt = Layout<BITS>;
    if (rp.arrived <= rp.gt) {
        int64_t spins = 0;
        for (;;) {
            rp.arrived = uniform((int)ctl_load(kCtlArrived + wi));
            if (rp.arrived > rp.gt) break;
            if (++spins > kSpinLimit) {   // the loader gave up: carry on with what is there
                store_shared(P->err, 1u);
                rp.arrived = rp.gt + 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    const int8_t *t = g_lds + L.ring_off + (wi * L.ring_slots + rp.slot) * Lt::kTileBytes;
#pragma unroll
    for (int j = 0; j < Lt::kSlabs; ++j) s.w[j] = *((const MBQ_LDS v4i *)(t + j * kSlab) + lane);
    s.sc = *((const MBQ_LDS v2u *)(t + Lt::kWeightBytes) + (lane & 15));
    s.hdr = (uint32_t)uniform((int)*(const MBQ_LDS uint32_t *)(g_lds + L.hdr_off + (wi * kMaxRingSlots + rp.slot) * 4));
    lds_done();   // the slot's bytes are in registers: the loader may refill it
    ++rp.gt;
    rp.slot = rp.slot + 1 == L.ring_slots ? 0 : rp.slot + 1;
    if (lane == 0) ctl_store(kCtlConsumed + wi, (uint32_t)rp.gt);
}

// The loader wave: walks the four compute waves' run lists in turn, putting
// each next tile into its wave's ring as soon as the ring has a free slot,
// with at most loader_window tiles in flight; a tile is published (arrival
// count of its wave) once the loads after it leave only the window's newest
// in flight.  It waits for nothing but ring space and its own loads.
//
// The run records come through LDS too: each wave's list is read 32 records
// ahead with LDS-DMA loads into a 64-record buffer, so opening a run costs an
// LDS read, not a scalar-cache miss (one such miss, serialised over four
// waves' lists, stalls the whole stream for a memory round trip).  The
// loader writes each tile's run header (or 0) next to its ring slot for the
// compute wave.  A record block is used at least 32 runs after its loads
// were issued, and every tile after it waits until at most loader_window
// tiles are in flight, so by then it has landed.
template <int BITS>
__device__ void loader(const SeqPlan *P, const Lay &L, int wg, int lane, int w0, int wt) {
    using Lt = Layout<BITS>;
    constexpr int T = Lt::kTileBytes;
    constexpr int NL = loads_per_tile<BITS>();
    // the window: loader_window<BITS, M>, a constant where the kernel calls this
    constexpr int WT_MAX = loader_window<BITS, kMaxM>();
    static_assert(kRecHalf >= WT_MAX, "a record block lands before it is used");
    const int S = L.ring_slots;
    const SeqWave *wtab = cload(&P->wtab);
    const SeqRun *runs0 = cload(&P->runs);
    const SeqRun *runs[kSeqFed];
    const uint8_t *src[kSeqFed];
    uint32_t hdr_next[kSeqFed];
    int next[kSeqFed], left[kSeqFed], issued[kSeqFed], total[kSeqFed], cons[kSeqFed], slot[kSeqFed];
    const auto rec_lds = [&](int w, int i) {
        return (const MBQ_LDS SeqRun *)(g_lds + L.rec_off + ((w0 + w) * kRecBuf + (i & (kRecBuf - 1))) * (int)sizeof(SeqRun));
    };
    const auto fetch_records = [&](int w, int first, int n) {   // records [first, first + n) into the buffer
        if (lane < n)
            __builtin_amdgcn_global_load_lds((const MBQ_GLOBAL void *)(runs[w] + first + lane),
                                             (MBQ_LDS void *)(g_lds + L.rec_off +
                                                              ((w0 + w) * kRecBuf + (first & (kRecBuf - 1))) *
                                                                  (int)sizeof(SeqRun)),
                                             16, 0, 0);
    };
#pragma unroll
    for (int w = 0; w < kSeqFed; ++w) {
        const SeqWave sw = cload(wtab, wg * kSeqWaves + w0 + w);
        runs[w] = runs0 + sw.run_begin;
        total[w] = sw.tiles;
        src[w] = nullptr;
        hdr_next[w] = 0;
        next[w] = left[w] = issued[w] = cons[w] = slot[w] = 0;
        fetch_records(w, 0, kRecBuf);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // Compute wave of each tile in flight, oldest in the low bits: 2 bits per
    // tile, at most 32 tiles.
    static_assert(WT_MAX <= 32 && kSeqFed <= 4, "in-flight order fits 64 bits");
    uint64_t order = 0;
    int seq = 0, pub = 0;
    int64_t spins = 0;
    auto publish_oldest = [&]() {
        const int wd = (int)(order & 3u);
        order >>= 2;
        ++pub;
        if (lane == 0) lds_add_u32_asm(lds_addr(&g_ctl[kCtlArrived + w0 + wd]), 1u);
    };
    for (;;) {
        bool any = false, pending = false;
#pragma unroll
        for (int w = 0; w < kSeqFed; ++w) {
            if (issued[w] >= total[w]) continue;
            pending = true;
            if (issued[w] - cons[w] >= S) {
                cons[w] = uniform((int)lds_read_u32_asm(lds_addr(&g_ctl[kCtlConsumed + w0 + w])));
                if (issued[w] - cons[w] >= S) continue;
            }
            uint32_t hdr = 0;
            if (left[w] == 0) {
                // the record's four dwords (src low, src high, hdr, n), one LDS read
                const v4i rec = lds_read_b128_asm(lds_addr((const void *)rec_lds(w, next[w])));
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane(rec.x);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane(rec.y);
                src[w] = (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
                hdr = (uint32_t)__builtin_amdgcn_readfirstlane(rec.z);
                left[w] = __builtin_amdgcn_readfirstlane(rec.w);
                ++next[w];
                if ((next[w] & (kRecHalf - 1)) == 0) fetch_records(w, next[w] + kRecHalf, kRecHalf);
            }
            // one LDS base and one address per tile, centred so that every
            // slab and the scales are within the instruction's offset range;
            // the offset moves the global and the LDS address alike
            int8_t *dst = g_lds + L.ring_off + ((w0 + w) * S + slot[w]) * T + kDmaMid<BITS>;
            const uint8_t *g16 = src[w] + kDmaMid<BITS> + lane * 16;
            dma_slabs<BITS, 0>(g16, dst);
            // the 64 rows' fp16 scales: 128 bytes, 16 per lane on 8 lanes (a
            // narrower load would not do: LDS-DMA places every lane's data at
            // least a dword apart)
            if (lane < 8) dma_scales<BITS>(g16, dst);
            if (lane == 0) lds_write_u32_asm(lds_addr(g_lds + L.hdr_off + ((w0 + w) * kMaxRingSlots + slot[w]) * 4), hdr);
            src[w] += T;
            --left[w];
            ++issued[w];
            slot[w] = slot[w] + 1 == S ? 0 : slot[w] + 1;
            order |= (uint64_t)w << (2 * (seq - pub));
            ++seq;
            if (seq - pub >= wt) {   // the oldest tile has landed
                if (wt == WT_MAX) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (WT_MAX - 1)));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (loader_window<BITS, 1>() - 1)));
                publish_oldest();
            }
            any = true;
        }
        if (any) {
            spins = 0;
            continue;
        }
        if (pub < seq) {   // every ring full (or every list done): land and publish the rest
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            while (pub < seq) publish_oldest();
            continue;
        }
        if (!pending) break;
        if (++spins > kSpinLimit) {   // no compute wave hands a slot back: give up
            store_shared(P->err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Park the open run's partial (segment sums of 4 rows x M per lane, reduced
// over the wave's k slices) in its LDS slot, row r at index r.  lp_w is the
// wave's slot area.
template <int M>
__device__ __forceinline__ void close_segment(int slot, float (&facc)[4][M], float *lp_w, int lane) {
    if (slot < 0) return;
    float *dst = lp_w + slot * M * 64 + slice_row(lane);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = facc[i][m];
        dst[m * 64] = slice_reduce(f);
    }
}

// Matrix-core products at every M: each lane accumulates exact int32 group
// sums of whole rows, so a row's fp32 sum is the same sequence of operations
// whatever M is (the v_dot4 form sums k slices separately and reduces them at
// the end, which rounds differently).  A tile's products take a small part of
// the time its bytes take to arrive, so M = 1 pays nothing measurable for the
// 16-row instruction.
#ifndef MBQ_MFMA_MIN_M
#define MBQ_MFMA_MIN_M 1
#endif
template <int M>
constexpr bool use_mfma() { return M >= MBQ_MFMA_MIN_M; }
// Accumulator columns per lane: the dot path keeps all M rows in every lane;
// the matrix-core path keeps rows 4 * (lane >> 4) + j, j < 4.
template <int M>
constexpr int acc_rows() { return use_mfma<M>() && M > 4 ? 4 : M; }

// The matrix-core form of close_segment: lane l holds complete sums of
// weight rows 4 * (l & 15) + i for activation rows 4 * (l >> 4) + j.
template <int M>
__device__ __forceinline__ void close_segment_mfma(int slot, float (&facc)[4][acc_rows<M>()], float *lp_w,
                                                   int lane) {
    if (slot < 0) return;
    float *dst = lp_w + slot * M * 64 + 4 * (lane & 15);
#pragma unroll
    for (int j = 0; j < acc_rows<M>(); ++j) {
        const int m = 4 * (lane >> 4) + j;
        if (m < M) {
            float4 v = {facc[0][j], facc[1][j], facc[2][j], facc[3][j]};
            *reinterpret_cast<float4 *>(dst + m * 64) = v;
        }
    }
}

struct Compute {
    int slot;     // LDS slot of the open run's segment; -1: none
    int q;        // LDS byte offset of the next tile's activation group
};

template <int BITS, int M>
__device__ __forceinline__ void compute(const Lay &L, int lane, Compute &c, float (&facc)[4][acc_rows<M>()],
                                        const Slot<BITS> &s, float *lp_w) {
    if (s.hdr != 0) {   // the tile opens a run: close the previous segment
        if constexpr (use_mfma<M>())
            close_segment_mfma<M>(c.slot, facc, lp_w, lane);
        else
            close_segment<M>(c.slot, facc, lp_w, lane);
        c.slot = (int)((s.hdr >> kRunPhaseBits) & ((1u << kRunSlotBits) - 1));
        c.q = (int)((s.hdr >> (kRunPhaseBits + kRunSlotBits)) & ((1u << kRunGroupBits) - 1)) * kGroup;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < acc_rows<M>(); ++m) facc[i][m] = 0.0f;
    }
    if constexpr (use_mfma<M>()) {
        // activation row lane & 15; rows past M read row 0 and feed unused outputs
        const int am = (lane & 15) < M ? (lane & 15) : 0;
        v4i acc[4];
        mfma_tile<BITS>(s.w, g_lds + am * L.qs + c.q + (lane >> 4) * 32, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float S = row_scale(s.sc, i);
#pragma unroll
            for (int j = 0; j < acc_rows<M>(); ++j) facc[i][j] = fmaf((float)acc[i][j], S, facc[i][j]);
        }
    } else {
        int acc[4][M];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[i][m] = 0;
        const int8_t *qg = g_lds + c.q + (lane >> 4) * 32;
        const int qs = L.qs;
        dot_tile<BITS, M>(s.w, [&](int m, int d) { return reinterpret_cast<const int *>(qg + m * qs)[d]; }, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float S = row_scale(s.sc, i);
#pragma unroll
            for (int m = 0; m < M; ++m) facc[i][m] = fmaf((float)acc[i][m], S, facc[i][m]);
        }
    }
    c.q += kGroup;
}

// One phase of a compute wave: its n tiles from the ring, in run order.
template <int BITS, int M>
__device__ __forceinline__ void stream_phase(const SeqPlan *P, const Lay &L, int wi, int lane, RingPos &rp, int n,
                                             float (&facc)[4][acc_rows<M>()], float *lp_w) {
    Compute c;
    c.slot = -1;
    c.q = 0;
    for (int t = 0; t < n; ++t) {
        Slot<BITS> s;
        take_tile<BITS>(P, L, wi, lane, rp, s);
        compute<BITS, M>(L, lane, c, facc, s, lp_w);
    }
    if constexpr (use_mfma<M>())
        close_segment_mfma<M>(c.slot, facc, lp_w, lane);
    else
        close_segment<M>(c.slot, facc, lp_w, lane);
}

template <int BITS, int M, bool X>
__global__ __launch_bounds__(kSeqBlock) void seq_kernel(const SeqPlan *__restrict__ P, uint32_t *err) {
    __shared__ float s_sh[2][kMaxM];
    __shared__ float r_sh[2][kMaxM];
    __shared__ float c_sh[kSeqWaves * (X ? 2 : 1) * M * 64];   // shared gathers of a finaliser
    // the workspace must hold a prepared plan, made for this form of the kernel
    if (cload(&P->magic) != kPlanMagic || cload(&P->full) != (X ? 1 : 0)) {
        if (threadIdx.x == 0 && blockIdx.x == 0) store_shared(err, 2u);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int wi = uniform(threadIdx.x >> 6);
    const int wg = blockIdx.x;
    // this launch's tags: those of the workspace's next epoch (22 bits, never 0)
    uint32_t *epoch_p = cload(&P->epoch);
    const uint32_t epoch = (uint32_t)uniform((int)load_shared(epoch_p));
    const uint32_t gen = epoch % ((1u << 22) - 1) + 1;
    Lay L;
    L.qs = cload(&P->q_stride);
    L.slots = cload(&P->slots);
    L.seg_cap = cload(&P->seg_cap);
    L.blk_bytes = cload(&P->blk_bytes);
    L.grid = cload(&P->grid);
    L.n_phases = cload(&P->n_phases);
    L.part_stride = cload(&P->part_stride);
    L.meta_off = M * L.qs + kSeqWaves * L.slots * M * 64 * 4;
    L.meta_bytes = ((int)sizeof(SeqPhase) + L.blk_bytes + 15) & ~15;
    L.rec_off = L.meta_off + 2 * L.meta_bytes;
    L.hdr_off = L.rec_off + kSeqWaves * kRecBuf * (int)sizeof(SeqRun);
    L.ring_off = L.hdr_off + kSeqWaves * kMaxRingSlots * 4;
    L.ring_slots = cload(&P->ring_slots);
    L.phases = cload(&P->phases);
    L.blocks = cload(&P->blocks);
    L.stats = cload(&P->stats);
    L.stat_stride = cload(&P->stat_stride);
    L.stat_rep = cload(&P->stat_rep);
    L.partials = cload(&P->partials);

    if (threadIdx.x < 16) g_ctl[threadIdx.x] = 0u;
    if (wi < kSeqWaves) {   // metadata of the first phase
        uint32_t pre[kMetaIters];
        fetch_meta(P, L, 0, wg, pre);
        store_meta(L, 0, pre);
    }
    __syncthreads();   // the only barrier the loader joins
    if (wi >= kSeqWaves) {
        loader<BITS>(P, L, wg, lane, (wi - kSeqWaves) * kSeqFed, loader_window<BITS, M>());
        return;
    }

    const bool finaliser = is_final_wg(wg, L.grid, M, X);
    external_stats<M>(P, wg * kSeqWaves + wi, L.grid * kSeqWaves, lane, gen);
    cw_sync(P);

    RingPos rp;
    rp.gt = 0;
    rp.slot = 0;
    rp.arrived = 0;
    float *lp_w = lds_partials(L, M) + (wi * L.slots * M) * 64;
    float facc[4][acc_rows<M>()];

    // One code path per step, each step once per phase: the whole loop has
    // to stay resident in the instruction cache, which two CUs share.
    for (int p = 0;; ++p) {
        enter_phase<BITS, M, X>(P, L, p, gen, wg, s_sh, r_sh);
        stream_phase<BITS, M>(P, L, wi, lane, rp, uniform(meta_head(L, p)->tiles[wi]), facc, lp_w);
        leave_phase<M>(P, L, p, gen);
        // Finalisers hand the phase over; the others go straight on to the
        // next phase's entry (the loader has been streaming its tiles).
        if (finaliser) finalize_phase<BITS, M, X>(P, L, p, gen, s_sh[p & 1], c_sh);
        if (p + 1 == L.n_phases) break;
    }

    // The last workgroup to exit clears the counters for the next launch
    // (every wave's counter increments have completed before it counts out)
    // and advances the epoch (every workgroup read it before counting out).
    wait_memory();
    cw_sync(P);
    if (threadIdx.x == 0) {
        uint32_t *cnt = cload(&P->counters);
        if (counter_add(cnt + (int64_t)L.n_phases * kCounterStride, 1u) == (uint32_t)(L.grid - 1)) {
            for (int i = 0; i <= L.n_phases; ++i) store_shared(cnt + (int64_t)i * kCounterStride, 0u);
            store_shared(epoch_p, epoch + 1u);
        }
    }
}

}  // namespace

}  // namespace mbq
