// Host side of the fused decode-step walk: turns an mbq_op list into the
// device plan the persistent kernel reads (see mbq_seq.h), and sizes the
// workspace.  Pure host code; no HIP call happens here.
#include <string.h>

#include <algorithm>
#include <map>
#include <vector>

#include "../../include/mbq.h"
#include "mbq_internal.h"
#include "mbq_kernels.h"
#include "mbq_seq.h"

namespace mbq {

namespace {

int64_t up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Tile ranges and chunking, mirroring the kernel's arithmetic.
struct PhaseGeom {
    int R, G, nkc, T, W;
    int chunk_len(int kc) const { return kc < nkc - 1 ? kChunkGroups : G - kChunkGroups * (nkc - 1); }
    int start(int w) const { return (int)(((int64_t)T * w) / W); }
    int owner(int t) const { return (int)((((int64_t)t + 1) * W - 1) / T); }
    void decode(int t, int &kc, int &rb) const {
        const int chunk_tiles = R * kChunkGroups;
        kc = t / chunk_tiles;
        rb = (t - kc * chunk_tiles) / chunk_len(kc);
    }
    int segment(int t) const {
        int kc, rb;
        decode(t, kc, rb);
        return kc * R + rb;
    }
};

}  // namespace

int64_t build_sequence_plan(const mbq_op *ops, int32_t n_ops, void *const *bufs, const int64_t *widths,
                            int32_t n_bufs, int64_t M, int n_cu, uint8_t *ws, SeqBuild *out) {
    if (!ops || !widths) return MBQ_ERR_NULL;
    if (n_ops < 1 || n_bufs < 1) return MBQ_ERR_PROGRAM;
    if (M < 1 || M > 4) return MBQ_ERR_SHAPE;
    for (int32_t b = 0; b < n_bufs; ++b)
        if (widths[b] < 8 || widths[b] % 8 || widths[b] > kMaxN) return MBQ_ERR_PROGRAM;
    const int bits = ops[0].bits;
    // ---- validate ops and cut phases
    struct Ph { int first, count; };
    std::vector<Ph> ph;
    for (int32_t i = 0; i < n_ops; ++i) {
        const mbq_op &o = ops[i];
        if (o.bits != 4 && o.bits != 6) return MBQ_ERR_BITS;
        if (o.bits != bits) return MBQ_ERR_PROGRAM;   // one bit width per walk
        if (!o.packed) return MBQ_ERR_NULL;
        if (((uintptr_t)o.packed & 255) != 0) return MBQ_ERR_ALIGN;
        if (o.prologue != MBQ_PRO_QUANT && o.prologue != MBQ_PRO_RMSNORM_QUANT) return MBQ_ERR_PROGRAM;
        if (o.K < kGroup || o.K % kGroup || o.K > ((int64_t)1 << 24) || o.N < 1 || o.N > kMaxN)
            return MBQ_ERR_SHAPE;
        if (o.in_buf < 0 || o.in_buf >= n_bufs || o.out_buf < 0 || o.out_buf >= n_bufs) return MBQ_ERR_PROGRAM;
        if (o.out_buf == o.in_buf) return MBQ_ERR_PROGRAM;
        if (o.K > widths[o.in_buf] || o.N != widths[o.out_buf]) return MBQ_ERR_PROGRAM;
        const bool joins = !ph.empty() && ops[ph.back().first].in_buf == o.in_buf &&
                           ops[ph.back().first].prologue == o.prologue && ops[ph.back().first].K == o.K;
        if (joins) {
            for (int j = ph.back().first; j < i; ++j)
                if (ops[j].out_buf == o.out_buf) return MBQ_ERR_PROGRAM;
            ph.back().count++;
        } else {
            ph.push_back(Ph{i, 1});
        }
    }
    const int n_ph = (int)ph.size();
    if (n_ph > kMaxPhases) return MBQ_ERR_PROGRAM;

    // ---- producers, stats records and external inputs
    std::vector<int> stats_cols(n_ops, 0), phase_of(n_ops, 0), in_prod(n_ph, -1), in_ext(n_ph, -1);
    std::vector<int> last_writer(n_bufs, -1);
    struct Ext { int buf; int64_t K; int64_t rec; int n_rb, rb_first; };
    std::vector<Ext> ext;
    for (int p = 0; p < n_ph; ++p) {
        const mbq_op &o0 = ops[ph[p].first];
        const int prod = last_writer[o0.in_buf];
        if (prod >= 0) {
            if (stats_cols[prod] != 0 && stats_cols[prod] != o0.K) return MBQ_ERR_PROGRAM;
            stats_cols[prod] = (int)o0.K;
            in_prod[p] = prod;
        } else {
            int e = -1;
            for (size_t j = 0; j < ext.size(); ++j)
                if (ext[j].buf == o0.in_buf && ext[j].K == o0.K) e = (int)j;
            if (e < 0) {
                ext.push_back(Ext{o0.in_buf, o0.K, 0, (int)((o0.K + 63) / 64), 0});
                e = (int)ext.size() - 1;
            }
            in_ext[p] = e;
        }
        for (int i = ph[p].first; i < ph[p].first + ph[p].count; ++i) {
            phase_of[i] = p;
            last_writer[ops[i].out_buf] = i;
        }
    }
    int64_t n_rec = 0, n_xt = 0;
    std::vector<int64_t> op_rec(n_ops, 0), op_xt(n_ops, -1);
    for (int i = 0; i < n_ops; ++i)
        if (stats_cols[i] > 0) {
            op_rec[i] = n_rec;
            n_rec += row_blocks(ops[i].N);
            op_xt[i] = n_xt;                       // tagged copy: M rows of N/2 words
            n_xt += M * (ops[i].N / 2);
        }
    int ext_rb = 0;
    for (Ext &e : ext) {
        e.rec = n_rec;
        e.rb_first = ext_rb;
        n_rec += e.n_rb;
        ext_rb += e.n_rb;
    }

    // ---- geometry, partial slots, LDS activation span
    const int grid = n_cu;
    const int waves = grid * kSeqWaves;
    std::vector<PhaseGeom> geo(n_ph);
    std::vector<std::vector<int>> rb_base(n_ph);
    int slots = 1, q_span = 128;
    for (int p = 0; p < n_ph; ++p) {
        PhaseGeom &g = geo[p];
        int64_t R = 0;
        for (int i = ph[p].first; i < ph[p].first + ph[p].count; ++i) {
            rb_base[p].push_back((int)R);
            R += row_blocks(ops[i].N);
        }
        if (R > kMaxN / kRows) return MBQ_ERR_SHAPE;
        g.R = (int)R;
        g.G = (int)(ops[ph[p].first].K / kGroup);
        g.nkc = (g.G + kChunkGroups - 1) / kChunkGroups;
        const int64_t T = R * g.G;
        if (T >= ((int64_t)1 << 31)) return MBQ_ERR_SHAPE;
        g.T = (int)T;
        g.W = (int)(T < waves ? T : waves);
        for (int w = 0; w < g.W; ++w) {
            const int t0 = g.start(w), t1 = g.start(w + 1) - 1;
            const int s = g.segment(t1) - g.segment(t0) + 1;
            if (s > slots) slots = s;
        }
        for (int wg = 0; wg * kSeqWaves < g.W; ++wg) {
            const int w1 = (wg + 1) * kSeqWaves < g.W ? (wg + 1) * kSeqWaves : g.W;
            const int t0 = g.start(wg * kSeqWaves), t1 = g.start(w1) - 1;
            int kc0, kc1, rb;
            g.decode(t0, kc0, rb);
            g.decode(t1, kc1, rb);
            int64_t hi = (int64_t)(kc1 + 1) * kChunkGroups * kGroup;
            if (hi > ops[ph[p].first].K) hi = ops[ph[p].first].K;
            const int span = (int)(hi - (int64_t)kc0 * kChunkGroups * kGroup);
            if (span > q_span) q_span = span;
        }
    }
    // workgroups touching one segment (memory partial slots per segment)
    int parts = 1;
    int64_t max_seg = 1;
    for (int p = 0; p < n_ph; ++p) {
        const PhaseGeom &g = geo[p];
        max_seg = std::max<int64_t>(max_seg, (int64_t)g.nkc * g.R);
        for (int kc = 0; kc < g.nkc; ++kc)
            for (int rb = 0; rb < g.R; ++rb) {
                const int t0 = kc * g.R * kChunkGroups + rb * g.chunk_len(kc);
                const int t1 = t0 + g.chunk_len(kc) - 1;
                parts = std::max(parts, g.owner(t1) / kSeqWaves - g.owner(t0) / kSeqWaves + 1);
            }
    }
    // ---- per-wave run lists: each wave's tile range of each phase, cut at
    // segment boundaries (a run's tiles are consecutive groups of one row
    // block, so they are contiguous in the packed matrix)
    const int64_t tile_bytes = bits == 4 ? Layout<4>::kTileBytes : Layout<6>::kTileBytes;
    std::vector<std::vector<SeqRun>> wruns(waves);
    std::vector<int> wtiles(waves, 0);
    for (int p = 0; p < n_ph; ++p) {
        const PhaseGeom &g = geo[p];
        for (int w = 0; w < g.W; ++w) {
            const int t0 = g.start(w), t1 = g.start(w + 1);
            if (t1 <= t0) continue;
            int kcw, rbw;
            g.decode(g.start(w / kSeqWaves * kSeqWaves), kcw, rbw);
            const int wg_g0 = kcw * kChunkGroups;          // first group the workgroup quantises
            const int seg0 = g.segment(t0);
            for (int t = t0; t < t1;) {
                int kc, rb;
                g.decode(t, kc, rb);
                const int len = g.chunk_len(kc);
                const int gi = t - kc * g.R * kChunkGroups - rb * len;
                const int n = std::min(len - gi, t1 - t);
                const int g0 = kc * kChunkGroups + gi;
                const int slot = kc * g.R + rb - seg0;
                const int gl = g0 - wg_g0;
                if (slot >= (1 << kRunSlotBits) || gl >= (1 << kRunGroupBits)) return MBQ_ERR_SHAPE;
                int op = ph[p].first;
                while (op + 1 < ph[p].first + ph[p].count && rb >= rb_base[p][op + 1 - ph[p].first]) ++op;
                SeqRun r;
                r.src = reinterpret_cast<const uint8_t *>(ops[op].packed) +
                        ((int64_t)(rb - rb_base[p][op - ph[p].first]) * g.G + g0) * tile_bytes;
                r.hdr = kRunStart | (uint32_t)p | ((uint32_t)slot << kRunPhaseBits) |
                        ((uint32_t)gl << (kRunPhaseBits + kRunSlotBits));
                r.n = (uint32_t)n;
                wruns[w].push_back(r);
                wtiles[w] += n;
                t += n;
            }
        }
    }
    int64_t n_runs = 0;
    for (int w = 0; w < waves; ++w) n_runs += (int64_t)wruns[w].size();

    const int q_stride = (int)up(q_span, 16);
    const int64_t lds = M * q_stride + (int64_t)kSeqWaves * slots * M * 64 * 4;
    if (lds > 150 * 1024) return MBQ_ERR_SHAPE;

    // ---- workspace layout
    const int64_t off_err = 0;
    const int64_t off_dummy = 256;
    const int64_t off_stats = off_dummy + 8192;
    const int64_t off_xt = up(off_stats + n_rec * kStatRecBytes, 256);
    const int64_t off_part = up(off_xt + n_xt * 8, 256);
    const int64_t off_plan = up(off_part + max_seg * parts * M * 64 * 8, 256);
    const int64_t off_ext = up(off_plan + (int64_t)sizeof(SeqPlan), 64);
    const int64_t off_phases = up(off_ext + (int64_t)ext.size() * sizeof(SeqExt), 64);
    const int64_t off_ops = up(off_phases + (int64_t)n_ph * sizeof(SeqPhase), 64);
    const int64_t off_wtab = up(off_ops + (int64_t)n_ops * sizeof(SeqOp), 64);
    const int64_t off_runs = up(off_wtab + (int64_t)waves * sizeof(SeqWave), 64);
    // per-phase tables: wave_start, wave_seg0, seg_owner, wg_k (int32)
    std::vector<int64_t> off_tab(n_ph);
    int64_t tab = up(off_runs + n_runs * (int64_t)sizeof(SeqRun), 64);
    for (int p = 0; p < n_ph; ++p) {
        off_tab[p] = tab;
        const int64_t ints = (geo[p].W + 1) + geo[p].W + 4LL * geo[p].nkc * geo[p].R + 6LL * grid;
        tab = up(tab + 4 * ints, 64);
    }
    const int64_t total = up(tab, 256);
    if (!out) return total;

    out->ws_bytes = total;
    out->grid = grid;
    out->lds_bytes = (int)lds;
    out->bits = bits;
    out->plan_offset = off_plan;
    out->blob.assign(total - off_plan, 0);
    if (!ws || !bufs) return total;

    uint8_t *blob = out->blob.data();
    auto dev = [&](int64_t off) { return ws + off; };
    SeqPlan plan;
    memset(&plan, 0, sizeof(plan));
    plan.magic = kPlanMagic;
    plan.n_phases = n_ph;
    plan.n_ops = n_ops;
    plan.n_ext = (int)ext.size();
    plan.n_ext_rb = ext_rb;
    plan.waves = waves;
    plan.slots = slots;
    plan.parts = parts;
    plan.q_stride = q_stride;
    plan.ops = reinterpret_cast<const SeqOp *>(dev(off_ops));
    plan.phases = reinterpret_cast<const SeqPhase *>(dev(off_phases));
    plan.ext = reinterpret_cast<const SeqExt *>(dev(off_ext));
    plan.err = reinterpret_cast<uint32_t *>(dev(off_err));
    plan.stats = dev(off_stats);
    plan.partials = reinterpret_cast<uint64_t *>(dev(off_part));
    plan.dummy = dev(off_dummy);
    plan.runs = reinterpret_cast<const SeqRun *>(dev(off_runs));
    plan.wtab = reinterpret_cast<const SeqWave *>(dev(off_wtab));
    memcpy(blob, &plan, sizeof(plan));
    {
        int64_t r0 = 0;
        for (int w = 0; w < waves; ++w) {
            SeqWave sw;
            sw.run_begin = (int32_t)r0;
            sw.run_count = (int32_t)wruns[w].size();
            sw.tiles = wtiles[w];
            sw.pad = 0;
            memcpy(blob + (off_wtab - off_plan) + w * sizeof(SeqWave), &sw, sizeof(sw));
            if (!wruns[w].empty())
                memcpy(blob + (off_runs - off_plan) + r0 * sizeof(SeqRun), wruns[w].data(),
                       wruns[w].size() * sizeof(SeqRun));
            r0 += (int64_t)wruns[w].size();
        }
    }
    for (size_t j = 0; j < ext.size(); ++j) {
        SeqExt e;
        memset(&e, 0, sizeof(e));
        e.in = reinterpret_cast<const uint32_t *>(bufs[ext[j].buf]);
        e.in_stride2 = (int32_t)(widths[ext[j].buf] / 2);
        e.K = (int32_t)ext[j].K;
        e.rec = ext[j].rec;
        e.n_rb = ext[j].n_rb;
        e.rb_first = ext[j].rb_first;
        memcpy(blob + (off_ext - off_plan) + j * sizeof(SeqExt), &e, sizeof(e));
    }
    for (int p = 0; p < n_ph; ++p) {
        const mbq_op &o0 = ops[ph[p].first];
        SeqPhase s;
        memset(&s, 0, sizeof(s));
        s.in = reinterpret_cast<const uint32_t *>(bufs[o0.in_buf]);
        s.in_stride2 = (int32_t)(widths[o0.in_buf] / 2);
        s.K = (int32_t)o0.K;
        s.G = geo[p].G;
        s.nkc = geo[p].nkc;
        s.prologue = o0.prologue;
        s.op_first = ph[p].first;
        s.op_count = ph[p].count;
        s.R = geo[p].R;
        s.W = geo[p].W;
        s.T = geo[p].T;
        s.in_nrec = (int32_t)((o0.K + 63) / 64);
        if (in_prod[p] >= 0) {
            s.in_phase = phase_of[in_prod[p]];
            s.in_rec = op_rec[in_prod[p]];
            s.in_xt = reinterpret_cast<const uint64_t *>(dev(off_xt)) + op_xt[in_prod[p]];
        } else {
            s.in_xt = nullptr;
            s.in_phase = -1;
            s.in_rec = ext[in_ext[p]].rec;
        }
        {
            const PhaseGeom &g = geo[p];
            int32_t *t = reinterpret_cast<int32_t *>(blob + (off_tab[p] - off_plan));
            int32_t *t_start = t, *t_seg0 = t + (g.W + 1), *t_own = t_seg0 + g.W, *t_wgk = t_own + 2 * g.nkc * g.R;
            int32_t *t_wgseg = t_wgk + 2 * grid;
            int32_t *t_segwg = t_wgseg + 2 * grid;
            int32_t *t_fin = t_segwg + 2 * g.nkc * g.R;
            for (int w = 0; w <= g.W; ++w) t_start[w] = g.start(w);
            for (int w = 0; w < g.W; ++w) t_seg0[w] = g.segment(g.start(w));
            for (int kc = 0; kc < g.nkc; ++kc)
                for (int rb = 0; rb < g.R; ++rb) {
                    const int t0 = kc * g.R * kChunkGroups + rb * g.chunk_len(kc);
                    const int t1 = t0 + g.chunk_len(kc) - 1;
                    t_own[2 * (kc * g.R + rb)] = g.owner(t0);
                    t_own[2 * (kc * g.R + rb) + 1] = g.owner(t1);
                }
            for (int wg = 0; wg < grid; ++wg) {
                int lo = 0, hi = 0;
                if (wg * kSeqWaves < g.W) {
                    const int w1 = (wg + 1) * kSeqWaves < g.W ? (wg + 1) * kSeqWaves : g.W;
                    const int t0 = g.start(wg * kSeqWaves), t1 = g.start(w1) - 1;
                    if (t1 >= t0) {
                        int kc0, kc1, rb;
                        g.decode(t0, kc0, rb);
                        g.decode(t1, kc1, rb);
                        lo = kc0 * kChunkGroups * kGroup;
                        const int64_t h = (int64_t)(kc1 + 1) * kChunkGroups * kGroup;
                        hi = (int)(h < o0.K ? h : o0.K);
                    }
                }
                t_wgk[2 * wg] = lo;
                t_wgk[2 * wg + 1] = hi;
            }
            for (int wg = 0; wg < grid; ++wg) {
                t_wgseg[2 * wg] = 0;
                t_wgseg[2 * wg + 1] = -1;
                t_fin[2 * wg] = 0;
                t_fin[2 * wg + 1] = 0;
                if (wg * kSeqWaves < g.W) {
                    const int w1 = (wg + 1) * kSeqWaves < g.W ? (wg + 1) * kSeqWaves : g.W;
                    const int t0 = g.start(wg * kSeqWaves), t1 = g.start(w1) - 1;
                    if (t1 >= t0) {
                        t_wgseg[2 * wg] = g.segment(t0);
                        t_wgseg[2 * wg + 1] = g.segment(t1);
                    }
                }
            }
            for (int sg = 0; sg < g.nkc * g.R; ++sg) {
                t_segwg[2 * sg] = t_own[2 * sg] / kSeqWaves;
                t_segwg[2 * sg + 1] = t_own[2 * sg + 1] / kSeqWaves;
            }
            for (int rb = 0; rb < g.R; ++rb) {    // finalising workgroups are non-decreasing in rb
                const int o = t_segwg[2 * ((g.nkc - 1) * g.R + rb) + 1];
                if (t_fin[2 * o + 1] == 0) t_fin[2 * o] = rb;
                t_fin[2 * o + 1]++;
            }
            const int32_t *dt = reinterpret_cast<const int32_t *>(dev(off_tab[p]));
            s.wave_start = dt;
            s.wave_seg0 = dt + (g.W + 1);
            s.seg_owner = dt + (g.W + 1) + g.W;
            s.wg_k = dt + (g.W + 1) + g.W + 2 * g.nkc * g.R;
            s.wg_seg = s.wg_k + 2 * grid;
            s.seg_wg = s.wg_seg + 2 * grid;
            s.wg_fin = s.seg_wg + 2 * g.nkc * g.R;
        }
        memcpy(blob + (off_phases - off_plan) + p * sizeof(SeqPhase), &s, sizeof(s));
        for (int i = ph[p].first; i < ph[p].first + ph[p].count; ++i) {
            SeqOp d;
            memset(&d, 0, sizeof(d));
            d.packed = reinterpret_cast<const uint8_t *>(ops[i].packed);
            d.out = reinterpret_cast<uint32_t *>(bufs[ops[i].out_buf]);
            d.N = (int32_t)ops[i].N;
            d.n_rb = (int32_t)row_blocks(ops[i].N);
            d.rb_base = rb_base[p][i - ph[p].first];
            d.stats_cols = stats_cols[i];
            d.stats_rec = op_rec[i];
            d.xt = op_xt[i] >= 0 ? reinterpret_cast<uint64_t *>(dev(off_xt)) + op_xt[i] : nullptr;
            memcpy(blob + (off_ops - off_plan) + i * sizeof(SeqOp), &d, sizeof(d));
        }
    }
    return total;
}

}  // namespace mbq
