// Host side of the fused decode-step walk: turns an mbq_op list into the
// device plan the persistent kernel reads (see mbq_seq.h), and sizes the
// workspace.  Pure host code; no HIP call happens here.
#include <stdlib.h>
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
    std::vector<int> st;   // [W + 1]: first tile of each wave's range
    int chunk_len(int kc) const { return kc < nkc - 1 ? kChunkGroups : G - kChunkGroups * (nkc - 1); }
    int start(int w) const { return st[w]; }
    int owner(int t) const { return (int)(std::upper_bound(st.begin(), st.end(), t) - st.begin()) - 1; }
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
    // Cut the T tiles into W = min(T, waves) contiguous ranges, the waves of
    // non-finalising workgroups weighted by w_other, every range non-empty.
    void cut(int waves, int grid, int M, bool full, double w_other) {
        W = T < waves ? T : waves;
        std::vector<double> cum(W + 1, 0.0);
        for (int w = 0; w < W; ++w) cum[w + 1] = cum[w] + (is_final_wg(w / kSeqWaves, grid, M, full) ? 1.0 : w_other);
        st.assign(W + 1, 0);
        for (int w = 1; w < W; ++w) {
            int v = (int)((double)T * cum[w] / cum[W] + 0.5);
            v = std::max(v, st[w - 1] + 1);
            v = std::min(v, T - (W - w));
            st[w] = v;
        }
        st[W] = T;
    }
};

// Share of a phase's tiles given to a wave of a non-finalising workgroup,
// relative to a finalising one.  It also decides where the ranges end, and so
// how many contributions a row block gets (whole tiles per wave keep them
// few); the values were measured on 9B- and 27B-shaped W4 walks.
//   - A quarter of the grid finalising (plain walks up to M = 3): 3.0, so the
//     finalisers stream a tenth of the tiles (2.6-3.8 % faster than 2.0 at
//     M = 1..2; 2.5-3.5 are within 1 % of each other).
//   - Half of the grid finalising: 1.0 below M = 3, 2.0 from M = 3 on, where
//     a finaliser gathers M words per contribution (2.0 cut 4-11 % at M =
//     3..8; 1.75 was worse than both 1.5 and 2.0).
// MBQ_SPLIT_WEIGHT overrides it.
double other_weight(int64_t M, bool quarter) {
    static const double env = [] {
        const char *e = getenv("MBQ_SPLIT_WEIGHT");
        const double v = e ? atof(e) : 0.0;
        return v > 0.05 && v < 20.0 ? v : 0.0;
    }();
    if (env > 0.0) return env;
    (void)M;
    // every workgroup finalising: equal shares; a subset finalising streams less
    return quarter ? 3.0 : 1.0;
}

}  // namespace

int64_t build_sequence_plan(const mbq_op *ops, int32_t n_ops, void *const *bufs, const int64_t *widths,
                            int32_t n_bufs, int64_t M, int n_cu, uint8_t *ws, SeqBuild *out) {
    if (!ops || !widths) return MBQ_ERR_NULL;
    if (n_ops < 1 || n_bufs < 1) return MBQ_ERR_PROGRAM;
    if (M < 1 || M > kMaxM) return MBQ_ERR_SHAPE;
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
        if (o.prologue < MBQ_PRO_QUANT || o.prologue > MBQ_PRO_SWIGLU_QUANT) return MBQ_ERR_PROGRAM;
        if (o.K < kGroup || o.K % kGroup || o.K > ((int64_t)1 << 24) || o.N < 1 || o.N > kMaxN)
            return MBQ_ERR_SHAPE;
        if (o.in_buf < 0 || o.in_buf >= n_bufs || o.out_buf < 0 || o.out_buf >= n_bufs) return MBQ_ERR_PROGRAM;
        if (o.out_buf == o.in_buf) return MBQ_ERR_PROGRAM;
        if (o.K > widths[o.in_buf] || o.N != widths[o.out_buf]) return MBQ_ERR_PROGRAM;
        const bool swiglu = o.prologue == MBQ_PRO_SWIGLU_QUANT, wnorm = o.prologue == MBQ_PRO_WRMSNORM_QUANT;
        if (swiglu && (o.in_buf2 < 0 || o.in_buf2 >= n_bufs || o.in_buf2 == o.out_buf || o.in_buf2 == o.in_buf ||
                       o.K > widths[o.in_buf2]))
            return MBQ_ERR_PROGRAM;
        if (wnorm && !o.norm_w) return MBQ_ERR_NULL;
        if (wnorm && ((uintptr_t)o.norm_w & 15) != 0) return MBQ_ERR_ALIGN;
        const mbq_op *f = ph.empty() ? nullptr : &ops[ph.back().first];
        const bool joins = f && f->in_buf == o.in_buf && f->prologue == o.prologue && f->K == o.K &&
                           (!swiglu || f->in_buf2 == o.in_buf2) && (!wnorm || f->norm_w == o.norm_w);
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
    bool full = false;
    for (int32_t i = 0; i < n_ops; ++i)
        full |= ops[i].prologue == MBQ_PRO_WRMSNORM_QUANT || ops[i].prologue == MBQ_PRO_SWIGLU_QUANT;

    // ---- producers, stats records and external inputs
    // Every consumer of an op must agree on the statistics it needs: the
    // columns (its K) and the weights of a weighted RMSNorm (max |y w|).  A
    // SwiGLU phase whose two inputs are written by the walk needs them written
    // by two ops of one phase with equal N, read by nothing else: the pair's
    // finaliser then hands over silu(gate) * up.  A SwiGLU phase whose two
    // inputs both come from before the launch gates them as it quantises.
    std::vector<int> stats_cols(n_ops, 0), phase_of(n_ops, 0), in_prod(n_ph, -1), in_ext(n_ph, -1);
    std::vector<int> uses(n_ops, 0), pair_of(n_ops, -1);   // pair_of[gate op] = its up op
    std::vector<char> pair_up(n_ops, 0);
    std::vector<const void *> stats_w(n_ops, nullptr);
    std::vector<int> last_writer(n_bufs, -1);
    struct Ext { int buf, buf2; int64_t K; const void *w; int64_t rec, xt; int n_rb, rb_first; };
    std::vector<Ext> ext;
    // Buffers some phase reads as an input written before the walk.  Phases
    // read such an input with plain loads when they enter, and the walk has no
    // ordering between that read and a write by a later, unrelated phase, so
    // an op that overwrites one of them is refused (the unfused call runs it).
    std::vector<char> ext_read(n_bufs, 0);
    for (int p = 0; p < n_ph; ++p) {
        const mbq_op &o0 = ops[ph[p].first];
        const bool swiglu = o0.prologue == MBQ_PRO_SWIGLU_QUANT;
        const void *cw = o0.prologue == MBQ_PRO_WRMSNORM_QUANT ? o0.norm_w : nullptr;
        const int prod = last_writer[o0.in_buf];
        const int prod2 = swiglu ? last_writer[o0.in_buf2] : -1;
        if (swiglu && (prod >= 0) != (prod2 >= 0)) return MBQ_ERR_PROGRAM;
        if (prod >= 0) {
            if (swiglu) {
                if (phase_of[prod] != phase_of[prod2] || ops[prod].N != ops[prod2].N) return MBQ_ERR_PROGRAM;
                if (uses[prod] || uses[prod2]) return MBQ_ERR_PROGRAM;
                pair_of[prod] = prod2;
                pair_up[prod2] = 1;
                uses[prod2]++;
            } else if (pair_of[prod] >= 0 || pair_up[prod]) {
                return MBQ_ERR_PROGRAM;
            }
            if (uses[prod] && (stats_cols[prod] != o0.K || stats_w[prod] != cw)) return MBQ_ERR_PROGRAM;
            uses[prod]++;
            stats_cols[prod] = (int)o0.K;
            stats_w[prod] = cw;
            in_prod[p] = prod;
        } else {
            const int buf2 = swiglu ? o0.in_buf2 : -1;
            int e = -1;
            for (size_t j = 0; j < ext.size(); ++j)
                if (ext[j].buf == o0.in_buf && ext[j].buf2 == buf2 && ext[j].K == o0.K && ext[j].w == cw) e = (int)j;
            if (e < 0) {
                ext.push_back(Ext{o0.in_buf, buf2, o0.K, cw, 0, -1, (int)((o0.K + 63) / 64), 0});
                e = (int)ext.size() - 1;
            }
            in_ext[p] = e;
            ext_read[o0.in_buf] = 1;
            if (buf2 >= 0) ext_read[buf2] = 1;
        }
        for (int i = ph[p].first; i < ph[p].first + ph[p].count; ++i) {
            if (ext_read[ops[i].out_buf]) return MBQ_ERR_PROGRAM;
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
        if (e.buf2 >= 0) {                         // gated values: M rows of K/2 words
            e.xt = n_xt;
            n_xt += M * (e.K / 2);
        }
        e.rec = n_rec;
        e.rb_first = ext_rb;
        n_rec += e.n_rb;
        ext_rb += e.n_rb;
    }

    // ---- geometry and per-wave run lists
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
        g.cut(waves, grid, (int)M, full, other_weight(M, quarter_finalise(grid, (int)M, full)));
        for (int w = 0; w < g.W; ++w) {
            const int t0 = g.start(w), t1 = g.start(w + 1) - 1;
            const int sc = g.segment(t1) - g.segment(t0) + 1;
            if (sc > slots) slots = sc;
        }
        for (int wg = 0; wg * kSeqWaves < g.W; ++wg) {
            const int t0 = g.start(wg * kSeqWaves), t1 = g.start(std::min((wg + 1) * kSeqWaves, g.W)) - 1;
            int kc0, kc1, rb;
            g.decode(t0, kc0, rb);
            g.decode(t1, kc1, rb);
            const int64_t hi = std::min<int64_t>((int64_t)(kc1 + 1) * kChunkGroups * kGroup, ops[ph[p].first].K);
            q_span = std::max(q_span, (int)(hi - (int64_t)kc0 * kChunkGroups * kGroup));
        }
    }
    if (slots > 255) return MBQ_ERR_SHAPE;
    // A run is a wave's part of one segment: consecutive groups of one row
    // block, so its tiles are contiguous in the packed matrix.
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
                if (gl >= (1 << kRunGroupBits)) return MBQ_ERR_SHAPE;
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
    if (n_runs >= ((int64_t)1 << 31)) return MBQ_ERR_SHAPE;

    // ---- contributions: segment (kc, rb) gets one partial per workgroup
    // touching it; a row block's partials are contiguous, in (kc, workgroup)
    // order.  Finalising units: a row block, or a gate row block together
    // with the same rows of its up block, whose partials follow the gate's so
    // that the unit's partials are one contiguous range.
    auto op_of = [&](int p, int rb) {
        int op = ph[p].first;
        while (op + 1 < ph[p].first + ph[p].count && rb >= rb_base[p][op + 1 - ph[p].first]) ++op;
        return op;
    };
    struct Unit { int rb, rb2; };
    std::vector<std::vector<Unit>> units(n_ph);
    std::vector<std::vector<int>> seg_c0(n_ph), seg_wg0(n_ph), rb_c0(n_ph), rb_nc(n_ph), unit_fin(n_ph);
    int part_stride = 1, seg_cap = 1, fin_cap = 1;
    for (int p = 0; p < n_ph; ++p) {
        const PhaseGeom &g = geo[p];
        const int nseg = g.nkc * g.R;
        seg_c0[p].assign(nseg, 0);
        seg_wg0[p].assign(nseg, 0);
        rb_c0[p].assign(g.R, 0);
        rb_nc[p].assign(g.R, 0);
        for (int rb = 0; rb < g.R; ++rb) {
            const int op = op_of(p, rb);
            if (pair_up[op]) continue;   // finalised with its gate block
            const int rb2 = pair_of[op] >= 0 ? rb_base[p][pair_of[op] - ph[p].first] + (rb - rb_base[p][op - ph[p].first])
                                             : -1;
            units[p].push_back(Unit{rb, rb2});
        }
        int c = 0;
        auto number = [&](int rb) {
            rb_c0[p][rb] = c;
            for (int kc = 0; kc < g.nkc; ++kc) {
                const int t0 = kc * g.R * kChunkGroups + rb * g.chunk_len(kc);
                const int t1 = t0 + g.chunk_len(kc) - 1;
                const int wga = g.owner(t0) / kSeqWaves, wgb = g.owner(t1) / kSeqWaves;
                seg_c0[p][kc * g.R + rb] = c;
                seg_wg0[p][kc * g.R + rb] = wga;
                c += wgb - wga + 1;
            }
            rb_nc[p][rb] = c - rb_c0[p][rb];
        };
        for (const Unit &u : units[p]) {
            number(u.rb);
            if (u.rb2 >= 0) number(u.rb2);
        }
        part_stride = std::max(part_stride, c);
        // the units are finalised by the finalising workgroups in turn
        {
            std::vector<int> fwg;
            for (int wg = 0; wg < grid; ++wg)
                if (is_final_wg(wg, grid, (int)M, full)) fwg.push_back(wg);
            unit_fin[p].assign(units[p].size(), 0);
            for (size_t u = 0; u < units[p].size(); ++u) unit_fin[p][u] = fwg[u % fwg.size()];
        }
        std::vector<int> nfin(grid, 0);
        for (size_t u = 0; u < units[p].size(); ++u) fin_cap = std::max(fin_cap, ++nfin[unit_fin[p][u]]);
        for (int wg = 0; wg * kSeqWaves < g.W; ++wg) {
            const int t0 = g.start(wg * kSeqWaves), t1 = g.start(std::min((wg + 1) * kSeqWaves, g.W)) - 1;
            if (t1 >= t0) seg_cap = std::max(seg_cap, g.segment(t1) - g.segment(t0) + 1);
        }
    }
    // Outputs are written with plain stores by the workgroup that finalises
    // each row block, and two phases' finalisers need not be ordered (nothing
    // may wait for an output no op reads).  A buffer written by several ops
    // is therefore accepted only when every row block of it is finalised by
    // the same workgroup each time: one workgroup, one L2, program order.
    {
        std::vector<std::vector<int>> rb_fin(n_ph);
        for (int p = 0; p < n_ph; ++p) {
            rb_fin[p].assign(geo[p].R, -1);
            for (size_t u = 0; u < units[p].size(); ++u) {
                rb_fin[p][units[p][u].rb] = unit_fin[p][u];
                if (units[p][u].rb2 >= 0) rb_fin[p][units[p][u].rb2] = unit_fin[p][u];
            }
        }
        std::vector<int> first_writer(n_bufs, -1);
        for (int i = 0; i < n_ops; ++i) {
            const int b = ops[i].out_buf, j = first_writer[b];
            if (j < 0) {
                first_writer[b] = i;
                continue;
            }
            const int pi = phase_of[i], pj = phase_of[j];
            const int bi = rb_base[pi][i - ph[pi].first], bj = rb_base[pj][j - ph[pj].first];
            for (int64_t r = 0; r < row_blocks(ops[i].N); ++r)
                if (rb_fin[pi][bi + r] != rb_fin[pj][bj + r]) return MBQ_ERR_PROGRAM;
        }
    }
    const int blk_bytes = (int)up(sizeof(SeqWgHead) + seg_cap * sizeof(SeqWgSeg) + fin_cap * sizeof(SeqFin), 16);
    const int fin_off = (int)(sizeof(SeqWgHead) + seg_cap * sizeof(SeqWgSeg));
    if ((int64_t)sizeof(SeqPhase) + blk_bytes > kMetaMaxBytes) return MBQ_ERR_SHAPE;

    // ---- LDS: activations, partial slots, two metadata slots, then the
    // compute waves' weight rings in what is left of the CU's 160 KiB (less
    // the kernel's static LDS: scales, shared-gather sums, control words)
    const int q_stride = (int)up(q_span, 16);
    const int64_t meta_bytes = up(sizeof(SeqPhase) + blk_bytes, 16);
    // ... plus the loader's run-record buffers and the per-slot run headers
    const int64_t lds_fixed = M * q_stride + (int64_t)kSeqWaves * slots * M * 64 * 4 + 2 * meta_bytes +
                              (int64_t)kSeqWaves * kRecBuf * (int64_t)sizeof(SeqRun) + kSeqWaves * kMaxRingSlots * 4;
    const int64_t lds_static = 2 * 2 * kMaxM * 4 + (int64_t)kSeqWaves * (full ? 2 : 1) * M * 64 * 4 + 16 * 4;
    const int64_t lds_avail = 160 * 1024 - 1024 - lds_static - lds_fixed;   // 1 KiB of slack for alignment
    const int64_t ring_slots = std::min<int64_t>(kMaxRingSlots, lds_avail / (kSeqWaves * tile_bytes));
    if (ring_slots < 2) return MBQ_ERR_SHAPE;
    const int64_t lds = lds_fixed + ring_slots * kSeqWaves * tile_bytes;

    // ---- workspace layout
    const int64_t off_err = 0;
    const int64_t off_dummy = 256;
    const int64_t off_stats = off_dummy + 8192;
    const int64_t off_xt = up(off_stats + (int64_t)kStatReplicas * n_rec * 3 * M * 8, 256);
    const int64_t off_part = up(off_xt + n_xt * 8, 256);
    const int64_t off_plan = up(off_part + 2 * (int64_t)part_stride * M * 64 * 8, 256);
    // the counters sit inside the plan blob, so preparing a plan clears them
    const int64_t off_cnt = up(off_plan + (int64_t)sizeof(SeqPlan), 64);
    const int64_t off_ext = up(off_cnt + 4 * (int64_t)kCounterStride * (n_ph + 1), 64);
    const int64_t off_phases = up(off_ext + (int64_t)ext.size() * sizeof(SeqExt), 64);
    const int64_t off_wtab = up(off_phases + (int64_t)n_ph * sizeof(SeqPhase), 64);
    const int64_t off_runs = up(off_wtab + (int64_t)waves * sizeof(SeqWave), 64);
    // the loader reads each wave's records up to a buffer (kRecBuf) past its
    // last run: zero records after the table keep those reads inside it
    const int64_t off_blocks = up(off_runs + (n_runs + kRecBuf) * (int64_t)sizeof(SeqRun), 64);
    const int64_t total = up(off_blocks + (int64_t)n_ph * grid * blk_bytes, 256);
    if (!out) return total;

    out->ws_bytes = total;
    out->grid = grid;
    out->lds_bytes = (int)lds;
    out->bits = bits;
    out->full = full;
    out->plan_offset = off_plan;
    out->blob.assign(total - off_plan, 0);
    if (!ws || !bufs) return total;

    uint8_t *blob = out->blob.data();
    auto dev = [&](int64_t off) { return ws + off; };
    auto put = [&](int64_t off, const void *src, size_t n) { memcpy(blob + (off - off_plan), src, n); };
    SeqPlan plan;
    memset(&plan, 0, sizeof(plan));
    plan.magic = kPlanMagic;
    plan.n_phases = n_ph;
    plan.n_ext = (int)ext.size();
    plan.n_ext_rb = ext_rb;
    plan.waves = waves;
    plan.grid = grid;
    plan.slots = slots;
    plan.q_stride = q_stride;
    plan.blk_bytes = blk_bytes;
    plan.seg_cap = seg_cap;
    plan.part_stride = part_stride;
    plan.full = full ? 1 : 0;
    plan.ring_slots = (int32_t)ring_slots;
    plan.phases = reinterpret_cast<const SeqPhase *>(dev(off_phases));
    plan.ext = reinterpret_cast<const SeqExt *>(dev(off_ext));
    plan.err = reinterpret_cast<uint32_t *>(dev(off_err));
    plan.epoch = reinterpret_cast<uint32_t *>(dev(off_err + 128));   // a line of its own, kept by prepare
    plan.stats = reinterpret_cast<uint64_t *>(dev(off_stats));
    plan.stat_stride = n_rec;
    plan.stat_rep = n_rec * 3 * M;
    plan.partials = reinterpret_cast<uint64_t *>(dev(off_part));
    plan.dummy = dev(off_dummy);
    plan.runs = reinterpret_cast<const SeqRun *>(dev(off_runs));
    plan.wtab = reinterpret_cast<const SeqWave *>(dev(off_wtab));
    plan.blocks = dev(off_blocks);
    plan.counters = reinterpret_cast<uint32_t *>(dev(off_cnt));
    put(off_plan, &plan, sizeof(plan));
    for (size_t j = 0; j < ext.size(); ++j) {
        SeqExt e;
        memset(&e, 0, sizeof(e));
        e.in = reinterpret_cast<const uint32_t *>(bufs[ext[j].buf]);
        e.in_stride2 = (int32_t)(widths[ext[j].buf] / 2);
        if (ext[j].buf2 >= 0) {
            e.in2 = reinterpret_cast<const uint32_t *>(bufs[ext[j].buf2]);
            e.in2_stride2 = (int32_t)(widths[ext[j].buf2] / 2);
            e.xt = reinterpret_cast<uint64_t *>(dev(off_xt)) + ext[j].xt;
        }
        e.norm_w = reinterpret_cast<const uint16_t *>(ext[j].w);
        e.K = (int32_t)ext[j].K;
        e.rec = ext[j].rec;
        e.n_rb = ext[j].n_rb;
        e.rb_first = ext[j].rb_first;
        put(off_ext + j * sizeof(SeqExt), &e, sizeof(e));
    }
    {
        int64_t r0 = 0;
        for (int w = 0; w < waves; ++w) {
            SeqWave sw;
            sw.run_begin = (int32_t)r0;
            sw.run_count = (int32_t)wruns[w].size();
            sw.tiles = wtiles[w];
            sw.pad = 0;
            put(off_wtab + w * sizeof(SeqWave), &sw, sizeof(sw));
            if (!wruns[w].empty()) put(off_runs + r0 * sizeof(SeqRun), wruns[w].data(), wruns[w].size() * sizeof(SeqRun));
            r0 += (int64_t)wruns[w].size();
        }
    }
    uint32_t *cnt_dev = reinterpret_cast<uint32_t *>(dev(off_cnt));
    uint64_t *xt_dev = reinterpret_cast<uint64_t *>(dev(off_xt));
    for (int p = 0; p < n_ph; ++p) {
        const mbq_op &o0 = ops[ph[p].first];
        const PhaseGeom &g = geo[p];
        SeqPhase s;
        memset(&s, 0, sizeof(s));
        s.in = reinterpret_cast<const uint32_t *>(bufs[o0.in_buf]);
        s.in_stride2 = (int32_t)(widths[o0.in_buf] / 2);
        s.K = (int32_t)o0.K;
        s.prologue = o0.prologue;
        if (o0.prologue == MBQ_PRO_WRMSNORM_QUANT) s.norm_w = reinterpret_cast<const uint32_t *>(o0.norm_w);
        s.in_nrec = (int32_t)((o0.K + 63) / 64);
        if (in_prod[p] >= 0) {
            s.in_phase = phase_of[in_prod[p]];
            s.in_rec = op_rec[in_prod[p]];
            s.in_xt = xt_dev + op_xt[in_prod[p]];
        } else {
            const Ext &e = ext[in_ext[p]];
            s.in_xt = e.xt >= 0 ? xt_dev + e.xt : nullptr;
            if (e.xt >= 0) s.in_stride2 = (int32_t)(e.K / 2);
            s.in_phase = -1;
            s.in_rec = e.rec;
        }
        s.wait_n = p >= 2 ? geo[p - 2].R : 0;
        s.wait_count = p >= 2 ? cnt_dev + (int64_t)(p - 2) * kCounterStride : nullptr;
        s.fin_count = cnt_dev + (int64_t)p * kCounterStride;
        put(off_phases + p * sizeof(SeqPhase), &s, sizeof(s));

        // per-workgroup blocks
        std::vector<std::vector<int>> fins(grid);
        for (size_t u = 0; u < units[p].size(); ++u) fins[unit_fin[p][u]].push_back((int)u);
        for (int wg = 0; wg < grid; ++wg) {
            std::vector<uint8_t> blk(blk_bytes, 0);
            SeqWgHead h;
            memset(&h, 0, sizeof(h));
            const int w0 = wg * kSeqWaves, w1 = std::min(w0 + kSeqWaves, g.W);   // waves [w0, w1)
            for (int j = 0; j < kSeqWaves; ++j)
                h.tiles[j] = w0 + j < g.W ? g.start(w0 + j + 1) - g.start(w0 + j) : 0;
            if (w0 < g.W && g.start(w1) > g.start(w0)) {
                const int t0 = g.start(w0), t1 = g.start(w1) - 1;
                int kc0, kc1, rb;
                g.decode(t0, kc0, rb);
                g.decode(t1, kc1, rb);
                h.k_lo = kc0 * kChunkGroups * kGroup;
                h.k_hi = (int)std::min<int64_t>((int64_t)(kc1 + 1) * kChunkGroups * kGroup, o0.K);
                const int s0 = g.segment(t0), s1 = g.segment(t1);
                for (int sg = s0; sg <= s1; ++sg) {
                    SeqWgSeg e;
                    e.cidx = seg_c0[p][sg] + (wg - seg_wg0[p][sg]);
                    const int kc = sg / g.R, srb = sg % g.R;
                    const int ts0 = kc * g.R * kChunkGroups + srb * g.chunk_len(kc);
                    const int ts1 = ts0 + g.chunk_len(kc) - 1;
                    for (int j = 0; j < kSeqWaves; ++j) {
                        const int w = w0 + j;
                        e.slot[j] = 0xFF;
                        if (w < w1 && g.start(w) <= ts1 && g.start(w + 1) > ts0)
                            e.slot[j] = (uint8_t)(sg - g.segment(g.start(w)));
                    }
                    memcpy(blk.data() + sizeof(SeqWgHead) + h.n_seg * sizeof(SeqWgSeg), &e, sizeof(e));
                    h.n_seg++;
                }
            }
            for (int u : fins[wg]) {
                const int rb = units[p][u].rb, rb2 = units[p][u].rb2;
                const int op = op_of(p, rb);
                const int rbl = rb - rb_base[p][op - ph[p].first];
                const int64_t N = ops[op].N;
                SeqFin f;
                memset(&f, 0, sizeof(f));
                f.out = reinterpret_cast<uint32_t *>(bufs[ops[op].out_buf]) + rbl * 32;
                f.xt = op_xt[op] >= 0 ? xt_dev + op_xt[op] + rbl * 32 : nullptr;
                f.stats = stats_cols[op] > 0
                              ? reinterpret_cast<uint64_t *>(dev(off_stats + (op_rec[op] + rbl) * 8))
                              : nullptr;
                f.row_words = (int32_t)(N / 2);
                f.rows = (int32_t)std::min<int64_t>(64, N - (int64_t)rbl * 64);
                f.stat_rows = (int32_t)std::max<int64_t>(
                    0, std::min<int64_t>(f.rows, std::min<int64_t>(N, stats_cols[op]) - (int64_t)rbl * 64));
                f.c0 = rb_c0[p][rb];
                f.nc = rb_nc[p][rb];
                if (rb2 >= 0) {   // its partials follow the gate block's
                    f.out2 = reinterpret_cast<uint32_t *>(bufs[ops[pair_of[op]].out_buf]) + rbl * 32;
                    f.nc_2 = rb_nc[p][rb2];
                }
                if (f.stats && stats_w[op]) f.norm_w = reinterpret_cast<const uint16_t *>(stats_w[op]) + rbl * 64;
                memcpy(blk.data() + fin_off + h.n_fin * sizeof(SeqFin), &f, sizeof(f));
                h.n_fin++;
            }
            memcpy(blk.data(), &h, sizeof(h));
            put(off_blocks + ((int64_t)p * grid + wg) * blk_bytes, blk.data(), blk_bytes);
        }
    }
    return total;
}

}  // namespace mbq
