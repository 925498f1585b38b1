// Execution plan of the fused decode-step walk (one persistent kernel per
// step).  Built on the host from an mbq_op list, copied into the workspace,
// read by the kernel.  Internal to libmbq.
#pragma once

#include <stdint.h>

namespace mbq {

constexpr int kSeqWaves = 4;                   // compute waves per workgroup
constexpr int kSeqThreads = 64 * kSeqWaves;    // their threads (the loaders' come after)
constexpr int kSeqLoaders = 2;                 // loader waves per workgroup, each feeding kSeqWaves / kSeqLoaders
constexpr int kSeqFed = kSeqWaves / kSeqLoaders;
constexpr int kSeqBlock = kSeqThreads + 64 * kSeqLoaders;

// Every workgroup finalises: the row blocks of a phase are dealt to all
// workgroups in turn, so each gathers at most a block or two per wave and
// the hand-over's gathers are spread over the whole chip.  (Weight loads go
// through the loader waves, so a finalising workgroup's polls queue behind
// no weight loads of its own compute waves.)
#ifndef MBQ_FIN_EVERY
#define MBQ_FIN_EVERY 1   // workgroups wg with wg % MBQ_FIN_EVERY == MBQ_FIN_EVERY - 1 finalise
#endif
__host__ __device__ inline bool quarter_finalise(int grid, int M, bool full) { return MBQ_FIN_EVERY > 1; }
__host__ __device__ inline bool is_final_wg(int wg, int grid, int M, bool full) {
    return grid < MBQ_FIN_EVERY || wg % MBQ_FIN_EVERY == MBQ_FIN_EVERY - 1;
}
constexpr int kChunkGroups = 8;                // k groups per k chunk (1024 k)
constexpr int kCounterStride = 32;             // u32 words between phase counters (one 128-B line each)
constexpr int kStatReplicas = 8;               // copies of the stats records, one per XCD
constexpr int kMaxPhases = 1000;               // < 2^kRunPhaseBits
constexpr int kMetaMaxBytes = 4096;           // phase record + workgroup block, per LDS slot
constexpr int kMaxRingSlots = 16;              // weight-ring tiles per compute wave, at most
constexpr int kRecBuf = 64;                    // run records the loader buffers per compute wave (LDS)
constexpr int kRecHalf = kRecBuf / 2;          // read this far ahead, half a buffer at a time
constexpr uint64_t kPlanMagic = 0x6d62712d73657134ull;  // "mbq-seq4"

// Every value that one wave hands to another travels in a 64-bit word whose
// high half is the epoch tag of the phase that wrote it, so a single load
// both fetches and validates it.
//
// Stats record of one row block of an op's output (rows n < stats_cols), for
// activation row m: word 3m = max|y| bits (max|y w| when the consumer applies
// a weighted RMSNorm with weights w), 3m+1 / 3m+2 = low / high half of
// the fp64 sum of y^2; each word's high half is the tag.  The records are
// stored word-major (word c of record r at stats[c * stat_stride + r]) so that
// a wave reading 64 consecutive records fetches contiguous memory, and in
// kStatReplicas copies (copy k at stats + k * stat_rep): every workgroup polls
// every record, and a workgroup reads the copy of its XCD (workgroup index
// mod 8), so no line is polled by more than one eighth of the grid.

struct SeqPhase {            // 72 bytes
    const uint32_t *in;      // bf16 pairs of the input rows (inputs written before the launch)
    // Tagged copy of the input, or null: written by the producer op (for a
    // SwiGLU input, by the gate/up pair's finaliser, or by the kernel-start
    // pass when both halves come from before the launch: the gated values).
    const uint64_t *in_xt;
    const uint32_t *norm_w;  // weighted RMSNorm: the norm's weights as bf16 pairs, else null
    int32_t in_stride2;      // input row stride in 32-bit words (and in tagged words)
    int32_t K, prologue;
    int32_t in_nrec;         // stats records describing the input: ceil(K / 64)
    int64_t in_rec;          // first of them
    int32_t in_phase;        // phase that writes them (-1: computed at kernel start)
    // The partial area is shared by phases of equal parity: before storing
    // partials, wait until the phase two back has finalised all wait_n of its
    // row blocks (*wait_count counts them).
    int32_t wait_n;
    const uint32_t *wait_count;
    uint32_t *fin_count;     // this phase's count of finalised row blocks
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

// Per (phase, workgroup) block: everything the workgroup needs to enter and
// leave the phase, prefetched into LDS one phase ahead.
struct SeqWgHead {
    int32_t k_lo, k_hi;      // input columns the workgroup quantises ([k_lo, k_hi), may be empty)
    int32_t n_seg, n_fin;    // entries below
    int32_t tiles[kSeqWaves];   // tiles of each of its waves in this phase
};
struct SeqWgSeg {            // a segment the workgroup's tiles touch
    int32_t cidx;            // its contribution (partial slot) in the phase's partial area
    uint8_t slot[kSeqWaves]; // each wave's LDS slot holding a part of it (0xFF: none)
};
struct SeqFin {              // a row block the workgroup finalises (64 bytes)
    uint32_t *out;           // its first bf16 pair in output row 0
    // A gate row block paired with the same rows of the up projection (both
    // ops of one phase, read only by one SwiGLU consumer): out2 is the up
    // block's first pair, and xt and stats describe silu(gate) * up.  Else null.
    uint32_t *out2;
    uint64_t *xt;            // same in the tagged copy, or null
    uint64_t *stats;         // word 0 of its stats record, or null
    const uint16_t *norm_w;  // consumer's RMSNorm weights at these rows (stats hold max |y w|), or null
    int32_t row_words;       // output row stride in pairs (N / 2)
    int32_t rows;            // valid rows (<= 64, even)
    int32_t stat_rows;       // rows feeding the stats (0 .. rows)
    int32_t c0, nc;          // its contributions, summed in this order
    int32_t nc_2;            // the up block's contributions, next in the area (pairs only)
};

struct SeqExt {              // an input no op of the walk writes: stats at kernel start
    const uint32_t *in;
    // SwiGLU consumer: the up input, and where the gated values silu(in) * in2
    // go (tagged, row stride K / 2 words), which the stats then describe; else null.
    const uint32_t *in2;
    uint64_t *xt;
    const uint16_t *norm_w;  // weighted-RMSNorm consumer: its weights (stats hold max |x w|), else null
    int32_t in_stride2, in2_stride2, K, pad;
    int64_t rec;
    int32_t n_rb, rb_first;  // its row-block records are blocks rb_first.. of the pre-pass
};

static_assert(sizeof(SeqPhase) == 72 && sizeof(SeqFin) == 64 && sizeof(SeqExt) == 64, "plan record sizes");

struct SeqPlan {
    uint64_t magic;
    int32_t n_phases, n_ext, n_ext_rb;
    int32_t waves;           // waves of the launch
    int32_t grid;            // workgroups
    int32_t slots;           // LDS partial slots per wave (segments one wave's range touches)
    int32_t q_stride;        // LDS bytes per activation row
    int32_t blk_bytes;       // bytes of one (phase, workgroup) block
    int32_t seg_cap;         // SeqWgSeg entries per block
    int32_t part_stride;     // contributions per parity half of the partial area
    // 1: the walk has weighted RMSNorms or SwiGLU inputs and runs the form of
    // the kernel that handles them (the other form carries none of their
    // instructions or registers); 0: only the plain and weightless-norm prologues
    int32_t full;
    int32_t ring_slots;      // LDS ring slots (tiles) per compute wave
    const SeqPhase *phases;
    const SeqExt *ext;
    uint32_t *err;           // nonzero after a wait gave up
    // Launches of the walk on this workspace so far: every workgroup reads it
    // at the start (its tags are those of epoch + 1) and the last workgroup
    // to exit advances it, so each launch -- a graph replay included -- has
    // tags of its own.  Preparing a plan leaves it alone: words of an earlier
    // plan's launches keep older tags.
    uint32_t *epoch;
    uint64_t *stats;         // stats records, word-major
    int64_t stat_stride;     // records (words per stats word index)
    int64_t stat_rep;        // words per copy of the records
    uint64_t *partials;      // [phase & 1][contribution][m][lane]: value bits | tag << 32
    const uint8_t *dummy;    // readable tile-sized area for loads past a stream's end
    const SeqRun *runs;      // every wave's runs, wave after wave, each in walk order
    const SeqWave *wtab;     // [waves]
    const uint8_t *blocks;   // [phase][workgroup] blocks of blk_bytes
    uint32_t *counters;      // [n_phases] finalised row blocks, then the exit count, each
                             // kCounterStride words apart; the last workgroup to exit clears them
};

}  // namespace mbq
