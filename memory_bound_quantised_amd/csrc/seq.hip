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
// Dataflow instead of grid barriers: every wave keeps a register ring of
// tiles in flight across phase boundaries (weights do not depend on
// activations).  Everything one wave hands to another is a 64-bit word whose
// high half is an epoch tag, so one load fetches and validates it:
//   - a wave that finishes part of a row block stores its fp32 partial;
//   - the owner of the row block's last tile gathers the parts in a fixed
//     order (bitwise reproducible results), writes the bf16 outputs, a tagged
//     copy of them for the consumer, and the block's row statistics
//     (max |y|, fp64 sum of y^2);
//   - a workgroup starts a phase by loading the statistics of its input and
//     the input columns it needs, re-polling any word whose tag is stale.
// Every wait is bounded; a wait that gives up sets the plan's error word and
// the kernel still runs to completion.
#include "mbq_internal.h"
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

// Plan data is read-only for the whole launch and always read at
// wave-uniform addresses: reading it through the constant address space lets
// the compiler use scalar loads, which keeps the vector-memory counter for the
// weight stream alone (so waits on a tile never wait for plan reads).
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

// Waves split a phase's T tiles into ranges [T*w/W, T*(w+1)/W); the range
// starts, first segments, segment owners and workgroup k ranges come from
// host-computed tables.

__device__ __forceinline__ int chunk_len(const SeqPhase &ph, int kc) {
    return kc < ph.nkc - 1 ? kChunkGroups : ph.G - kChunkGroups * (ph.nkc - 1);
}

struct Pos {
    int kc, rb, gi;   // k chunk, phase row block, group index inside the chunk
};

__device__ __forceinline__ Pos decode(const SeqPhase &ph, int t) {
    const int chunk_tiles = ph.R * kChunkGroups;
    Pos p;
    p.kc = t / chunk_tiles;
    const int rem = t - p.kc * chunk_tiles;
    const int len = chunk_len(ph, p.kc);
    p.rb = rem / len;
    p.gi = rem - p.rb * len;
    return p;
}

__device__ __forceinline__ int segment(const SeqPhase &ph, int kc, int rb) { return kc * ph.R + rb; }

__device__ __forceinline__ int first_segment(const SeqPhase &ph, int w) { return cload(ph.wave_seg0, w); }
__device__ __forceinline__ int seg_first_owner(const SeqPhase &ph, int seg) { return cload(ph.seg_owner, 2 * seg); }
__device__ __forceinline__ int seg_last_owner(const SeqPhase &ph, int seg) { return cload(ph.seg_owner, 2 * seg + 1); }

__device__ __forceinline__ int op_of_rb(const SeqPlan *P, const SeqPhase &ph, int rb) {
    int j = ph.op_first;
    while (j + 1 < ph.op_first + ph.op_count && rb >= cload(P->ops, j + 1).rb_base) ++j;
    return j;
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

// True if any lane of the wave passes true.
__device__ __forceinline__ bool wave_any(bool b) { return __builtin_amdgcn_ballot_w64(b) != 0; }

// Load a tagged word, re-polling until its tag is `want` (or the wait gives up).
__device__ __forceinline__ uint64_t await_word(const SeqPlan *P, const uint64_t *p, uint64_t first, uint32_t want) {
    uint64_t v = first;
    int64_t spins = 0;
    while (tag_of(v) != want) {
        if (gave_up(P, spins)) break;
        v = load_shared(p);
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ uint64_t *stat_rec(const SeqPlan *P, int64_t r) {
    return reinterpret_cast<uint64_t *>(P->stats + r * kStatRecBytes);
}

// Publish one stats record from per-lane values (lanes past the stats rows pass 0).
template <int M>
__device__ __forceinline__ void publish_stats(const SeqPlan *P, int64_t r, const float (&v)[M], uint32_t tag,
                                              int lane) {
    uint64_t *rec = stat_rec(P, r);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const double ss = wave_sum((double)v[m] * (double)v[m]);
        const float am = wave_max(fabsf(v[m]));
        if (lane == 0) {
            const uint64_t bits = (uint64_t)__double_as_longlong(ss);
            store_shared(rec + 3 * m, tagged(__float_as_uint(am), tag));
            store_shared(rec + 3 * m + 1, tagged((uint32_t)bits, tag));
            store_shared(rec + 3 * m + 2, tagged((uint32_t)(bits >> 32), tag));
        }
    }
}

// ---------------------------------------------------------------- kernel-start stats of external inputs

template <int M>
__device__ void external_stats(const SeqPlan *P, int w, int lane, uint32_t gen) {
    for (int b = w; b < P->n_ext_rb; b += P->waves) {
        int e = 0;
        while (e + 1 < P->n_ext && b >= cload(P->ext, e + 1).rb_first) ++e;
        const SeqExt x = cload(P->ext, e);
        const int rb = b - x.rb_first;
        const int col = rb * 64 + lane;
        float v[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            v[m] = 0.0f;
            if (col < x.K) {
                const uint32_t word = x.in[(int64_t)m * x.in_stride2 + (col >> 1)];
                v[m] = bf16_bits_to_f32((word >> (16 * (col & 1))) & 0xFFFFu);
            }
        }
        publish_stats<M>(P, x.rec + rb, v, make_tag(gen, -1), lane);
    }
}

// ---------------------------------------------------------------- phase prologue (workgroup-wide)

struct WgRange {
    int k_lo, k_hi;   // columns this workgroup quantises; empty if k_hi == k_lo
};

__device__ __forceinline__ WgRange wg_range(const SeqPhase &ph, int wg) {
    return WgRange{cload(ph.wg_k, 2 * wg), cload(ph.wg_k, 2 * wg + 1)};
}

constexpr int kStatBatch = 4;   // stats records per lane per round trip
constexpr int kXBatch = 4;      // input words (2 columns each) per thread per round trip

// Quantise columns [k_lo, k_hi) of the phase input into LDS (int8, row stride
// q_stride), after the optional weightless RMSNorm.  Row statistics come from
// the producer's stats records, reduced in a fixed order so that every
// workgroup derives bit-identical scales.  Returns k_lo.
template <int M>
__device__ __noinline__ void enter_phase(const SeqPlan *P, int p, uint32_t gen, int wg, int8_t *q_lds,
                                        float (*s_sh)[4], float (*r_sh)[4]) {
    const SeqPhase ph = cload(P->phases, p);
    const WgRange kr = wg_range(ph, wg);
    const int lane = threadIdx.x & 63;
    const bool norm = ph.prologue == 1;
    const uint32_t want = make_tag(gen, ph.in_phase);
    const int words = (kr.k_hi - kr.k_lo) >> 1;        // bf16 pairs per activation row
    const bool tagged_in = ph.in_xt != nullptr;
    const bool has = kr.k_hi > kr.k_lo;

    // Issue the first batch of input loads now; they fly while wave 0 reduces the stats.
    uint64_t xw[kXBatch][M];
#pragma unroll
    for (int u = 0; u < kXBatch; ++u)
#pragma unroll
        for (int m = 0; m < M; ++m) xw[u][m] = 0;
    if (has && tagged_in) {
#pragma unroll
        for (int u = 0; u < kXBatch; ++u) {
            const int j = threadIdx.x + u * kSeqThreads;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (j < words) xw[u][m] = load_shared(ph.in_xt + (int64_t)m * ph.in_stride2 + (kr.k_lo >> 1) + j);
        }
    }

    if (has && threadIdx.x < 64) {
        double ss[M];
        float am[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            ss[m] = 0.0;
            am[m] = 0.0f;
        }
        for (int base = 0; base < ph.in_nrec; base += 64 * kStatBatch) {
            uint64_t v[kStatBatch][3 * M];
            const uint64_t *rp[kStatBatch];
#pragma unroll
            for (int u = 0; u < kStatBatch; ++u) {
                const int i = base + lane + 64 * u;
                rp[u] = stat_rec(P, ph.in_rec + (i < ph.in_nrec ? i : 0));
#pragma unroll
                for (int c = 0; c < 3 * M; ++c) v[u][c] = load_shared(rp[u] + c);
            }
            int64_t spins = 0;
            for (;;) {
                bool stale = false;
#pragma unroll
                for (int u = 0; u < kStatBatch; ++u)
#pragma unroll
                    for (int c = 0; c < 3 * M; ++c)
                        stale |= base + lane + 64 * u < ph.in_nrec && tag_of(v[u][c]) != want;
                if (!wave_any(stale) || gave_up(P, spins)) break;
#pragma unroll
                for (int u = 0; u < kStatBatch; ++u)
#pragma unroll
                    for (int c = 0; c < 3 * M; ++c)
                        if (base + lane + 64 * u < ph.in_nrec && tag_of(v[u][c]) != want)
                            v[u][c] = load_shared(rp[u] + c);
            }
#pragma unroll
            for (int u = 0; u < kStatBatch; ++u) {
                if (base + lane + 64 * u < ph.in_nrec) {
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const uint64_t lo = v[u][3 * m + 1], hi = v[u][3 * m + 2];
                        am[m] = fmaxf(am[m], __uint_as_float((uint32_t)v[u][3 * m]));
                        ss[m] += __longlong_as_double((long long)(((hi & 0xFFFFFFFFull) << 32) | (lo & 0xFFFFFFFFull)));
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const double tot = wave_sum(ss[m]);
            const float amax = wave_max(am[m]);
            float r = 1.0f, amax_t = amax;
            if (norm) {
                const float ms = (float)(tot / (double)ph.K);
                r = 1.0f / sqrtf(ms + 1e-6f);
                // max |bf16(x * r)| = bf16(max|x| * r): rounding is monotonic
                amax_t = bf16_bits_to_f32(f32_to_bf16_bits(amax * r));
            }
            if (lane == 0) {
                s_sh[p & 1][m] = amax_t / 127.0f;
                r_sh[p & 1][m] = r;
            }
        }
    }
    __syncthreads();
    if (has) {
        float s[M], r[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            s[m] = s_sh[p & 1][m];
            r[m] = r_sh[p & 1][m];
        }
        for (int j0 = 0; j0 < words; j0 += kXBatch * kSeqThreads) {
            if (j0 > 0 && tagged_in) {
#pragma unroll
                for (int u = 0; u < kXBatch; ++u) {
                    const int j = j0 + threadIdx.x + u * kSeqThreads;
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        if (j < words)
                            xw[u][m] = load_shared(ph.in_xt + (int64_t)m * ph.in_stride2 + (kr.k_lo >> 1) + j);
                }
            }
            if (tagged_in) {
                int64_t spins = 0;
                for (;;) {
                    bool stale = false;
#pragma unroll
                    for (int u = 0; u < kXBatch; ++u)
#pragma unroll
                        for (int m = 0; m < M; ++m)
                            stale |= j0 + threadIdx.x + u * kSeqThreads < words && tag_of(xw[u][m]) != want;
                    if (!wave_any(stale) || gave_up(P, spins)) break;
#pragma unroll
                    for (int u = 0; u < kXBatch; ++u) {
                        const int j = j0 + threadIdx.x + u * kSeqThreads;
#pragma unroll
                        for (int m = 0; m < M; ++m)
                            if (j < words && tag_of(xw[u][m]) != want)
                                xw[u][m] = load_shared(ph.in_xt + (int64_t)m * ph.in_stride2 + (kr.k_lo >> 1) + j);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kXBatch; ++u) {
                const int j = j0 + threadIdx.x + u * kSeqThreads;
                if (j >= words) continue;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint32_t pair = tagged_in ? (uint32_t)xw[u][m]
                                                    : ph.in[(int64_t)m * ph.in_stride2 + (kr.k_lo >> 1) + j];
                    uint32_t packed = 0;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        float t = bf16_bits_to_f32((pair >> (16 * e)) & 0xFFFFu);
                        if (norm) t = bf16_bits_to_f32(f32_to_bf16_bits(t * r[m]));
                        float qv = 0.0f;
                        if (s[m] != 0.0f) qv = fminf(fmaxf(rintf(t / s[m]), -127.0f), 127.0f);
                        packed |= ((uint32_t)(int)qv & 0xFFu) << (8 * e);
                    }
                    *reinterpret_cast<uint16_t *>(q_lds + m * P->q_stride + 2 * j) = (uint16_t)packed;
                }
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- row-block finalisation (cold path)

// The wave owning a row block's last tile gathers every part in (k chunk,
// wave) order and writes the bf16 outputs, their tagged copy and the block's
// stats record.  Out of line: it runs once per row block and phase.
template <int BITS, int M>
__device__ __noinline__ void finalize_rb(const SeqPlan *P, uint32_t gen, int phase, int rb, const float *s_act) {
    using L = Layout<BITS>;
    const SeqPhase ph = cload(P->phases, phase);
    const int lane = threadIdx.x & 63;
    const uint32_t tag = make_tag(gen, phase);
    const int kcl = ph.nkc - 1;
    float tot[M];
#pragma unroll
    for (int m = 0; m < M; ++m) tot[m] = 0.0f;

    // contributions (kc, part): the workgroups touching segment (kc, rb), in order
    auto n_parts = [&](int kc) {
        const int sg = segment(ph, kc, rb);
        return cload(ph.seg_wg, 2 * sg + 1) - cload(ph.seg_wg, 2 * sg) + 1;
    };
    int ckc = 0, cp = 0;
    while (ckc <= kcl) {
        constexpr int B = 16;
        const uint64_t *src[B];
        bool valid[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            valid[u] = ckc <= kcl;
            if (valid[u]) {
                const int sg = segment(ph, ckc, rb);
                src[u] = P->partials + ((int64_t)(sg * P->parts + cp) * M) * 64 + lane;
                if (++cp == n_parts(ckc)) {
                    cp = 0;
                    ++ckc;
                }
            } else {
                src[u] = src[0];
            }
        }
        uint64_t v[B][M];
#pragma unroll
        for (int u = 0; u < B; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m) v[u][m] = load_shared(src[u] + m * 64);
        // re-poll every stale word together: one round trip per round
        int64_t spins = 0;
        for (;;) {
            bool stale = false;
#pragma unroll
            for (int u = 0; u < B; ++u)
#pragma unroll
                for (int m = 0; m < M; ++m) stale |= valid[u] && tag_of(v[u][m]) != tag;
            if (!wave_any(stale) || gave_up(P, spins)) break;
#pragma unroll
            for (int u = 0; u < B; ++u)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (valid[u] && tag_of(v[u][m]) != tag) v[u][m] = load_shared(src[u] + m * 64);
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            if (valid[u]) {
#pragma unroll
                for (int m = 0; m < M; ++m) tot[m] += __uint_as_float((uint32_t)v[u][m]);
            }
        }
    }
    const SeqOp op = cload(P->ops, op_of_rb(P, ph, rb));
    const int rbl = rb - op.rb_base;
    const int n = rbl * 64 + lane;
    const float unscale = 1.0f / (float)(1 << L::kAccShift);
    float yv[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t yb = f32_to_bf16_bits(s_act[m] * (tot[m] * unscale));
        const uint32_t hi = (uint32_t)__shfl_xor((int)yb, 1, 64);
        const uint32_t pair = yb | (hi << 16);
        if (!(lane & 1) && n < op.N) {
            const int64_t idx = (int64_t)m * (op.N >> 1) + (n >> 1);
            op.out[idx] = pair;
            if (op.xt) store_shared(op.xt + idx, tagged(pair, tag));
        }
        yv[m] = n < min(op.N, op.stats_cols) ? bf16_bits_to_f32(yb) : 0.0f;
    }
    if (op.stats_cols > 0) publish_stats<M>(P, op.stats_rec + rbl, yv, tag, lane);
}

// ---------------------------------------------------------------- the kernel

template <int BITS>
struct Slot {
    v4i w[Layout<BITS>::kSlabs];
    v2u sc;
    uint32_t hdr;   // the run header if this tile opens a run, else 0
};

// Tiles in flight per wave.  A wave can have at most 63 vector loads
// outstanding and a tile takes kSlabs + 1 of them (W4: 12 tiles, W6: 9);
// larger M trims the ring to stay within 512 registers.
template <int BITS, int M>
constexpr int ring_depth() {
    return BITS == 4 ? (M < 4 ? 12 : 10) : (M < 3 ? 9 : (M < 4 ? 8 : 7));
}
static_assert(ring_depth<4, 1>() * (Layout<4>::kSlabs + 1) <= 63, "vmcnt limit");
static_assert(ring_depth<6, 1>() * (Layout<6>::kSlabs + 1) <= 63, "vmcnt limit");

// Issue side: a cursor over the wave's run list.  Everything here is
// wave-uniform and read with scalar loads, so waiting on a tile never waits
// on a plan read.
struct Issue {
    const SeqRun *runs;
    int next, count;       // next run to open; runs of this wave
    int left;              // tiles left in the open run
    const uint8_t *src;    // next tile
};

template <int BITS>
__device__ __forceinline__ void issue(Issue &is, const uint8_t *dummy, int lane, Slot<BITS> &s) {
    uint32_t hdr = 0;
    if (is.left == 0) {
        if (is.next < is.count) {
            const SeqRun r = cload(is.runs, is.next);
            ++is.next;
            is.src = r.src;
            is.left = (int)r.n;
            hdr = r.hdr;
        } else {                       // past the end: keep the ring's load count fixed
            is.src = dummy;
            is.left = 1;
        }
    }
    s.hdr = hdr;
    load_tile<BITS>(is.src, lane, s.w, s.sc);
    is.src += Layout<BITS>::kTileBytes;
    --is.left;
}

// Park the open run's partial (segment sums of 4 rows x M per lane, reduced
// over the wave's k slices) in its LDS slot; lane l holds row l.
template <int M>
__device__ __forceinline__ void close_segment(int slot, float (&facc)[4][M], float *lp_w, int lane) {
    if (slot < 0) return;
    float *dst = lp_w + slot * M * 64;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = slice_sum(facc[i][m]);
        dst[m * 64] = to_row_layout(f, lane);
    }
}

// Workgroup-wide exit from phase p: merge the waves' LDS partials of every
// segment the workgroup touched (in wave order), publish one tagged partial
// per (segment, workgroup), then finalise the row blocks whose last tile the
// workgroup owns.
template <int BITS, int M>
__device__ __noinline__ void leave_phase(const SeqPlan *P, int p, uint32_t gen, int wg, const float *lp,
                                         const float *s_act) {
    __syncthreads();
    const SeqPhase ph = cload(P->phases, p);
    const int lane = threadIdx.x & 63;
    const int j = uniform(threadIdx.x >> 6);
    const uint32_t tag = make_tag(gen, p);
    const int w0 = wg * kSeqWaves;
    const int w1 = min(w0 + kSeqWaves, ph.W) - 1;
    const int s0 = cload(ph.wg_seg, 2 * wg), s1 = cload(ph.wg_seg, 2 * wg + 1);
    for (int sg = s0 + j; sg <= s1; sg += kSeqWaves) {
        const int wa = max(w0, seg_first_owner(ph, sg));
        const int wb = min(w1, seg_last_owner(ph, sg));
        float v[M];
#pragma unroll
        for (int m = 0; m < M; ++m) v[m] = 0.0f;
        for (int ww = wa; ww <= wb; ++ww) {
            const float *src = lp + (((ww - w0) * P->slots + sg - first_segment(ph, ww)) * M) * 64 + lane;
#pragma unroll
            for (int m = 0; m < M; ++m) v[m] += src[m * 64];
        }
        const int part = wg - cload(ph.seg_wg, 2 * sg);
        uint64_t *dst = P->partials + ((int64_t)(sg * P->parts + part) * M) * 64 + lane;
#pragma unroll
        for (int m = 0; m < M; ++m) store_shared(dst + m * 64, tagged(__float_as_uint(v[m]), tag));
    }
    const int f0 = cload(ph.wg_fin, 2 * wg), fn = cload(ph.wg_fin, 2 * wg + 1);
    for (int i = j; i < fn; i += kSeqWaves) finalize_rb<BITS, M>(P, gen, p, f0 + i, s_act);
}

struct Compute {
    int active;   // phase whose prologue ran last
    int slot;     // LDS slot of the open run's segment; -1: none
    int q;        // LDS byte offset of the next tile's activation group
};

template <int BITS, int M>
__device__ __forceinline__ void compute(const SeqPlan *P, uint32_t gen, int wg, int lane, Compute &c,
                                        float (&facc)[4][M], const Slot<BITS> &s, int8_t *q_lds, int qs,
                                        float *lp, float *lp_w, float (*s_sh)[4], float (*r_sh)[4]) {
    if (s.hdr != 0) {   // the tile opens a run: close the previous segment, meet the run's phase
        close_segment<M>(c.slot, facc, lp_w, lane);
        const int phase = (int)(s.hdr & ((1u << kRunPhaseBits) - 1));
        while (c.active < phase) {
            if (c.active >= 0) leave_phase<BITS, M>(P, c.active, gen, wg, lp, s_sh[c.active & 1]);
            ++c.active;
            enter_phase<M>(P, c.active, gen, wg, q_lds, s_sh, r_sh);
        }
        c.slot = (int)((s.hdr >> kRunPhaseBits) & ((1u << kRunSlotBits) - 1));
        c.q = (int)((s.hdr >> (kRunPhaseBits + kRunSlotBits)) & ((1u << kRunGroupBits) - 1)) * kGroup;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < M; ++m) facc[i][m] = 0.0f;
    }
    int acc[4][M];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = 0;
    const int8_t *qg = q_lds + c.q + (lane >> 4) * 32;
    dot_tile<BITS, M>(s.w, [&](int m, int d) { return reinterpret_cast<const int *>(qg + m * qs)[d]; }, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float S = row_scale(s.sc, i);
#pragma unroll
        for (int m = 0; m < M; ++m) facc[i][m] = fmaf((float)acc[i][m], S, facc[i][m]);
    }
    c.q += kGroup;
}

template <int BITS, int M>
__global__ __launch_bounds__(kSeqThreads) void seq_kernel(const SeqPlan *__restrict__ P, uint32_t *err,
                                                          uint32_t gen) {
    extern __shared__ __align__(16) int8_t q_lds[];
    __shared__ float s_sh[2][4];
    __shared__ float r_sh[2][4];
    if (cload(&P->magic) != kPlanMagic) {   // workspace does not hold a prepared plan
        if (threadIdx.x == 0 && blockIdx.x == 0) store_shared(err, 2u);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int wi = uniform(threadIdx.x >> 6);
    const int wg = blockIdx.x;
    const int w = wg * kSeqWaves + wi;
    const int n_phases = cload(&P->n_phases);
    const int qs = cload(&P->q_stride);
    const int slots = cload(&P->slots);
    const uint8_t *dummy = cload(&P->dummy);

    external_stats<M>(P, w, lane, gen);

    const SeqWave wv = cload(cload(&P->wtab), w);
    Issue is;
    is.runs = cload(&P->runs) + wv.run_begin;
    is.next = 0;
    is.count = wv.run_count;
    is.left = 0;
    is.src = dummy;
    float *lp = reinterpret_cast<float *>(q_lds + M * qs);
    float *lp_w = lp + (wi * slots * M) * 64 + lane;
    Compute c;
    c.active = -1;
    c.slot = -1;
    c.q = 0;
    float facc[4][M];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) facc[i][m] = 0.0f;

    constexpr int D = ring_depth<BITS, M>();
    Slot<BITS> ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) issue<BITS>(is, dummy, lane, ring[i]);
    int left = wv.tiles;
    while (left > 0) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (left > 0) {
                compute<BITS, M>(P, gen, wg, lane, c, facc, ring[i], q_lds, qs, lp, lp_w, s_sh, r_sh);
                --left;
            }
            issue<BITS>(is, dummy, lane, ring[i]);
        }
    }
    // close the last segment and meet every remaining workgroup-wide prologue
    close_segment<M>(c.slot, facc, lp_w, lane);
    while (c.active < n_phases - 1) {
        if (c.active >= 0) leave_phase<BITS, M>(P, c.active, gen, wg, lp, s_sh[c.active & 1]);
        ++c.active;
        enter_phase<M>(P, c.active, gen, wg, q_lds, s_sh, r_sh);
    }
    leave_phase<BITS, M>(P, c.active, gen, wg, lp, s_sh[c.active & 1]);
}

}  // namespace

// ---------------------------------------------------------------- host side

hipError_t launch_sequence(int bits, int64_t M, int grid, int lds_bytes, const void *plan, uint32_t *err,
                           uint32_t gen, hipStream_t st) {
    void *args[] = {(void *)&plan, (void *)&err, (void *)&gen};
    const void *fn = nullptr;
#define MBQ_PICK(B, MM) fn = reinterpret_cast<const void *>(&seq_kernel<B, MM>)
    if (bits == 4) {
        switch (M) { case 1: MBQ_PICK(4, 1); break; case 2: MBQ_PICK(4, 2); break;
                     case 3: MBQ_PICK(4, 3); break; default: MBQ_PICK(4, 4); break; }
    } else {
        switch (M) { case 1: MBQ_PICK(6, 1); break; case 2: MBQ_PICK(6, 2); break;
                     case 3: MBQ_PICK(6, 3); break; default: MBQ_PICK(6, 4); break; }
    }
#undef MBQ_PICK
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kSeqThreads), args, (unsigned)lds_bytes, st);
}

}  // namespace mbq
