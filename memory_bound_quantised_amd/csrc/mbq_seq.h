// Execution plan of the fused decode-step walk (one persistent kernel per
// step).  Built on the host from an mbq_op list, copied into the workspace,
// read by the kernel.  Internal to libmbq.
#pragma once

#include <stdint.h>

namespace mbq {

constexpr int kSeqWaves = 4;                   // waves per workgroup
constexpr int kSeqThreads = 64 * kSeqWaves;
constexpr int kChunkGroups = 8;                // k groups per k chunk (1024 k)
constexpr int kStatRecBytes = 128;             // one per (producer op, row block)
constexpr int kMaxPhases = 1000;             // < 2^kRunPhaseBits
constexpr uint64_t kPlanMagic = 0x6d62712d73657131ull;  // "mbq-seq1"

// Every value that one wave hands to another travels in a 64-bit word whose
// high half is the epoch tag of the phase that wrote it, so a single load
// both fetches and validates it.
//
// Stats record of one row block of an op's output (rows n < stats_cols), for
// activation row m: word 3m = max|y| bits, 3m+1 / 3m+2 = low / high half of
// the fp64 sum of y^2; each word's high half is the tag.
struct SeqOp {
    const uint8_t *packed;
    uint32_t *out;           // bf16 pairs; row m starts at word m * N / 2
    uint64_t *xt;            // tagged copy of out for the consumer: bf16 pair | tag << 32
    int32_t N;
    int32_t n_rb;            // row blocks of this op
    int32_t rb_base;         // first phase-level row block of this op
    int32_t stats_cols;      // rows n < stats_cols feed the stats records (0: none)
    int64_t stats_rec;       // index of this op's first stats record
};

struct SeqPhase {
    const uint32_t *in;      // bf16 pairs of the input rows (inputs written before the launch)
    const uint64_t *in_xt;   // tagged copy written by the producer op, or null
    int32_t in_stride2;      // input row stride in 32-bit words (and in tagged words)
    int32_t K, G, nkc, prologue;
    int32_t op_first, op_count;
    int32_t R;               // row blocks over all ops of the phase
    int32_t W;               // waves with work (min(total waves, T))
    int32_t T;               // tiles, ordered (k chunk, row block, group)
    int32_t in_nrec;         // stats records describing the input: ceil(K / 64)
    int32_t in_phase;        // phase that writes them (-1: computed at kernel start)
    int64_t in_rec;          // first of them
    // Host-computed tables (integer division is slow on the GPU):
    const int32_t *wave_start;   // [W + 1]: first tile of each wave's range
    const int32_t *wave_seg0;    // [W]: segment (k chunk * R + row block) of that first tile
    const int32_t *seg_owner;    // [nkc * R][2]: waves owning the segment's first and last tile
    const int32_t *wg_k;         // [workgroups][2]: columns [k_lo, k_hi) a workgroup quantises
    const int32_t *wg_seg;       // [workgroups][2]: first and last segment the workgroup's tiles touch
                                 // (last < first: none)
    const int32_t *seg_wg;       // [nkc * R][2]: workgroups owning the segment's first and last tile
    const int32_t *wg_fin;       // [workgroups][2]: first row block and count of row blocks whose
                                 // last tile the workgroup owns (it finalises them)
};

// One run of a wave's walk: consecutive tiles of one segment (k chunk x row
// block), contiguous in memory.  hdr packs what the compute side needs when
// the run starts: bits 0-9 phase, 10-17 the wave's LDS partial slot, 18-29
// the run's first group relative to the workgroup's first quantised column
// (in groups), bit 31 set.
struct SeqRun {
    const uint8_t *src;      // first tile
    uint32_t hdr;
    uint32_t n;              // tiles (1 .. kChunkGroups)
};
constexpr uint32_t kRunStart = 1u << 31;
constexpr int kRunPhaseBits = 10, kRunSlotBits = 8, kRunGroupBits = 12;

struct SeqWave {             // one wave's slice of the run table
    int32_t run_begin, run_count, tiles, pad;
};

struct SeqExt {              // an input no op of the walk writes: stats at kernel start
    const uint32_t *in;
    int32_t in_stride2, K;
    int64_t rec;
    int32_t n_rb, rb_first;  // its row-block records are blocks rb_first.. of the pre-pass
};

struct SeqPlan {
    uint64_t magic;
    int32_t n_phases, n_ops, n_ext, n_ext_rb;
    int32_t waves;           // total waves of the launch
    int32_t slots;           // LDS partial slots per wave (segments one wave's range touches)
    int32_t q_stride;        // LDS bytes per activation row
    int32_t parts;           // memory partial slots per segment (workgroups touching one segment)
    const SeqOp *ops;
    const SeqPhase *phases;
    const SeqExt *ext;
    uint32_t *err;           // nonzero after a wait gave up
    uint8_t *stats;          // stats records
    uint64_t *partials;      // [segment][part][m][lane]: value bits | tag << 32
    const uint8_t *dummy;    // readable tile-sized area for loads past a stream's end
    const SeqRun *runs;      // every wave's runs, wave after wave, each in walk order
    const SeqWave *wtab;     // [waves]
};

}  // namespace mbq
