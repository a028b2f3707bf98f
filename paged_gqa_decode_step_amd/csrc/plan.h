// Launch planning of libsa: the fixed split table, the balanced kernel's
// wavefront count, which kernel a call uses and the workspace it needs.
// Everything here depends only on the dims and the window (never on
// seq_lens, which live on the device, nor on timing), and it sets the launch
// configuration of every kernel.  Included by the C-ABI layer only.
#pragma once

#include <limits.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sa.h"
#include "sa_internal.h"

namespace {

using sa::kHeadDim;

// T: new tokens (query tokens) per sequence
int query_tokens(const sa_dims* d) { return d->num_query_tokens > 0 ? d->num_query_tokens : 1; }

// Fixed split table (no autotuning, so the result of a call never depends on
// timing).  A partition is 32 * 2^k slots, at most kMaxTableSlice blocks and
// at most kMaxPartTokens slots, and never longer than the context capacity
// (a 128-slot ring is one partition).  It halves, down to kMinPartTokens,
// while a call would have fewer than kMinWaves partition wavefronts.  A split
// call whose grid of kBurstSteps-step partitions is at most one wavefront per
// SIMD takes those instead (the static kernel then loads a whole partition at
// once).  Chosen from measured sweeps on MI355X: long partitions keep the
// partial traffic and the combine small; batch-1 calls trade some of that
// for parallelism.
constexpr int kMaxPartTokens = 1024;
constexpr int kMinPartTokens = 256;
constexpr long kMinWaves = 128;
// The fused mode (the last partition of a (b, g) merges the partials) is
// never the default: measured on MI355X, the device-scope fence every
// partition then needs costs more than the separate combine launch.
// Balanced kernel: at most kStreamWaves wavefronts (4 per compute unit of an
// MI355X, one per SIMD: measured faster than 6 or 8 per unit on every large
// workload, since fewer, longer streams leave fewer partials and unit
// switches while two steps in flight per wavefront still keep HBM busy),
// rounded down to a multiple of kWaveQuantum above it (counts between, such
// as 1280, 1664 or 1920, measured 5-8% slower), at most kMaxSegsPerUnit per
// (sequence, KV head) so a
// few long units do not turn into hundreds of partials each, and at least
// kMinStreamSteps 32-slot steps of work each, for batches of up to
// kMaxStreamSeqs sequences (its per-sequence table lives in LDS).
#ifndef SA_STREAM_WAVES
#define SA_STREAM_WAVES 1024
#endif
constexpr long kStreamWaves = SA_STREAM_WAVES;
constexpr long kWaveQuantum = 512;
constexpr long kMaxSegsPerUnit = 128;
constexpr long kMinStreamSteps = 8;
constexpr int kMaxStreamSeqs = 2048;

struct Plan {
    int32_t splits;
    int32_t part_tokens;
};

// Assumes check_dims passed.
Plan plan(const sa_dims* d, int32_t window) {
    const int bs = d->block_size;
    const long cap = (long)d->max_blocks_per_seq * bs;
    const long max_n = window > 0 ? (window < cap ? window : cap) : cap;
    const int gran = bs > sa::kStepTokens ? bs : sa::kStepTokens;
    int pmax = sa::kMaxTableSlice * bs;
    if (pmax > kMaxPartTokens && kMaxPartTokens >= gran) pmax = kMaxPartTokens;
    int P;
    if (d->num_splits > 0) {
        long want = (max_n + d->num_splits - 1) / d->num_splits;
        want = (want + gran - 1) / gran * gran;
        P = (int)(want < gran ? gran : (want > pmax ? pmax : want));
    } else {
        const long units = (long)(d->num_seqs > 0 ? d->num_seqs : 1) * d->num_kv_heads;
        P = pmax;
        while (P / 2 >= gran && P / 2 >= max_n) P /= 2;          // one partition covers it
        while (P / 2 >= gran && P / 2 >= kMinPartTokens &&
               units * ((max_n + P - 1) / P) < kMinWaves)
            P /= 2;
        // A call that is split anyway takes burst partitions when their grid
        // fits (a call of one partition a unit needs no merge at all): of 4
        // steps when that grid fits too, keeps the merge to at most
        // kCombineFourWaves partials a row, and leaves the one-wavefront
        // merge (kCombineOneWave partials) only for a grid of fewer than half
        // the wavefronts; else of 8 steps.  Measured on MI355X (us, 8-step vs
        // 4-step partitions): batch 1 x 1024 6.92 / 5.87, 1 x 4096 7.95 /
        // 7.13, 1 x 8192 8.47 / 8.27, 2 x 2048 7.43 / 7.09, 2 x 8192 11.61 /
        // 11.34, 4 x 4096 11.54 / 11.29; kept at 8 steps: 8 x 2048 11.24 /
        // 11.57 (the wider merge), 1 x 16384 11.71 / 12.30 (128 partials a
        // row).
        // The widest merges (more than kCombineFourWaves partials a row) on a
        // static grid of half to one wavefront per SIMD: partitions of two
        // table slices halve the partials and keep half the SIMDs or more
        // busy (measured: batch 1 x 131072 45.53 -> 44.94 us, its
        // tensor-parallel share 45.64 -> 45.12).  The static MFMA kernel
        // walks a partition's slices in turn; the vector-ALU engine reads one
        // slice a partition, so it keeps them.
        {
            const long s1 = (max_n + P - 1) / P, s2 = (max_n + 2L * P - 1) / (2L * P);
            if (P == pmax && d->variant != SA_VARIANT_VALU && s1 > sa::kCombineFourWaves &&
                units * s1 <= kStreamWaves && 2 * units * s2 >= kStreamWaves)
                P *= 2;
        }
        const int pb = sa::kBurstSteps * sa::kStepTokens;
        const int p4 = 4 * sa::kStepTokens;
        if (max_n > P && pb >= gran && pb <= pmax &&
            units * ((max_n + pb - 1) / pb) <= kStreamWaves) {
            const long s8 = (max_n + pb - 1) / pb, s4 = (max_n + p4 - 1) / p4;
            P = pb;
            if (p4 >= gran && units * s4 <= kStreamWaves && s4 <= sa::kCombineFourWaves &&
                (s4 <= sa::kCombineOneWave || s8 > sa::kCombineOneWave ||
                 units * s8 < kStreamWaves / 2))
                P = p4;
        }
    }
    Plan p;
    p.part_tokens = P;
    p.splits = (int32_t)((max_n + P - 1) / P);
    return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout.  The completion counters of the fused combine sit at a
// fixed place, offset 0, in a region nothing else ever writes: every call
// returns the counters it used to zero, so a workspace zeroed once stays
// valid for any later call, whatever its dims or split count.
constexpr int kCounterSlots = 1 << 18;   // (sequence, KV head) pairs a fused call may have
constexpr size_t kCounterBytes = (size_t)kCounterSlots * sizeof(int32_t);

struct WorkspaceLayout {
    size_t part_o, part_lse, counters, unit_seg, total;
};

// kBalanced: the balanced kernel and a merge launch; kBalancedLastMerges: the
// balanced kernel, the last wavefront to finish a split unit merging it
// (measured slower on every workload, so never the default: the counted
// arrival and the agent-coherent reads cost more than the launch)
enum class Mode { kStatic, kFused, kBalanced, kBalancedLastMerges };

// floats of one segment slot of the balanced kernel's own merge (16 values
// and an lse per lane)
constexpr size_t kSegFloats = 17 * 64;

// Upper bound on the balanced kernel's steps for these dims: every unit at
// the table's capacity (the lengths live on the device).
long stream_steps_upper(const sa_dims* d, int32_t window) {
    const long cap = (long)d->max_blocks_per_seq * d->block_size;
    const long max_n = window > 0 ? (window < cap ? window : cap) : cap;
    return (long)d->num_seqs * d->num_kv_heads * ((max_n + sa::kStepTokens - 1) / sa::kStepTokens);
}

// Wavefronts of the balanced kernel for these dims (an upper bound on the
// work is all the host knows).
long stream_waves(const sa_dims* d, int32_t window) {
    const long t_upper = stream_steps_upper(d, window);
    long nw = (t_upper + kMinStreamSteps - 1) / kMinStreamSteps;
    const long seg_cap = (long)d->num_seqs * d->num_kv_heads * kMaxSegsPerUnit;
    if (nw > seg_cap) nw = seg_cap;
    if (nw > kStreamWaves) nw = kStreamWaves;
    if (nw > kWaveQuantum) nw -= nw % kWaveQuantum;
    return nw < 1 ? 1 : nw;
}

// The static kernel loads every step of its partition at once (a burst)
// when partitions are exactly kBurstSteps or 4 steps and the grid is at most
// one wavefront per SIMD (the burst kernels hold all those steps in
// registers, so they run one wavefront per SIMD): one round trip of K/V per
// partition, for calls too small to keep HBM busy with pipelined
// wavefronts.  The burst covers exactly the partition's steps: the 8-step
// burst on the ring layer's 4-step partitions, with four unused loads each,
// measured slower than the pipeline (7.40 vs 6.59 us), the 4-step burst
// faster (6.43 vs 6.53 us, bit-identical output).  Returns the register
// depth: kBurstSteps or 4 for a burst, 2 for the two-step pipeline.
#ifndef SA_STATIC_BURST
#define SA_STATIC_BURST 1
#endif
int static_depth(const sa_dims* d, const Plan& p) {
    if (!SA_STATIC_BURST ||
        (long long)d->num_seqs * d->num_kv_heads * p.splits > kStreamWaves)
        return 2;
    if (p.part_tokens == sa::kBurstSteps * sa::kStepTokens) return sa::kBurstSteps;
    if (p.part_tokens == 4 * sa::kStepTokens) return 4;
    return 2;
}
bool static_burst(const sa_dims* d, const Plan& p) {
    return static_depth(d, p) == sa::kBurstSteps;
}

// Which kernel a call with these dims uses (assumes check_dims passed).
Mode choose_mode(const sa_dims* d, int32_t window, const Plan& p) {
    // the balanced kernel keeps its per-sequence table in LDS and walks steps
    // in 32-bit arithmetic
    const bool fits_stream = d->num_seqs <= kMaxStreamSeqs &&
                             stream_steps_upper(d, window) <= INT_MAX &&
                             (long long)d->num_seqs * d->num_kv_heads <= kCounterSlots;
    switch (d->variant) {
        case SA_VARIANT_MFMA_BALANCED:
            return fits_stream ? Mode::kBalanced : Mode::kStatic;
        case SA_VARIANT_MFMA_BALANCED_LAST_MERGES:
            return fits_stream ? Mode::kBalancedLastMerges : Mode::kStatic;
        case SA_VARIANT_MFMA_FUSED:
            return (long long)d->num_seqs * d->num_kv_heads <= kCounterSlots ? Mode::kFused
                                                                             : Mode::kStatic;
        case SA_VARIANT_MFMA_TWO_PASS:
        case SA_VARIANT_VALU:
            return Mode::kStatic;
        default: {
            // One static partition needs no merge at all.  Nor is the balanced
            // kernel worth its fixed costs when the static grid is burst
            // partitions, or holds between half and one wavefront per SIMD:
            // the length scan before any load (the static kernel issues its
            // first loads with the length's), and the merge's segment records
            // (the static merge knows where every partial is and reads them
            // all in one round trip).  Every partition then runs at once
            // (measured on MI355X: batch 1 x 8192 8.4 vs 9.7 us, batch 1 x
            // 131072 45.6 vs 47.4 us, 0.2-2.8 us faster from batch 8 x 8192 to
            // 64 x 2048); with fewer, longer partitions the GPU is not kept
            // busy, with more the balanced kernel's even split wins.
            if (d->num_splits > 0 || p.splits == 1 || !fits_stream) return Mode::kStatic;
            if (static_burst(d, p)) return Mode::kStatic;
            const long parts = (long)d->num_seqs * d->num_kv_heads * p.splits;
            if (parts >= kStreamWaves / 2 && parts <= kStreamWaves) return Mode::kStatic;
            return Mode::kBalanced;
        }
    }
}

WorkspaceLayout workspace_layout(const sa_dims* d, int32_t window, const Plan& p, Mode m) {
    WorkspaceLayout w{};
    size_t rows, lse;        // partial rows of D floats, and lse entries
    if (m == Mode::kBalancedLastMerges) {
        // two segment slots per wavefront, counters in front
        w.counters = 0;
        w.part_o = kCounterBytes;
        w.total = w.part_o + align256((size_t)stream_waves(d, window) * 2 * kSegFloats *
                                      sizeof(float));
        w.part_lse = w.unit_seg = w.total;
        return w;
    }
    if (m == Mode::kBalanced) {
        const size_t slots = (size_t)stream_waves(d, window) * 2 * query_tokens(d) *
                             (d->num_q_heads / d->num_kv_heads);
        rows = slots;
        lse = slots;
    } else {
        if (p.splits <= 1) return w;
        rows = (size_t)d->num_seqs * query_tokens(d) * d->num_q_heads * p.splits;
        lse = rows;
    }
    w.counters = 0;
    w.part_o = kCounterBytes;
    w.part_lse = w.part_o + align256(rows * kHeadDim * sizeof(float));
    w.unit_seg = w.part_lse + align256(lse * sizeof(float));
    w.total = w.unit_seg + align256((size_t)d->num_seqs * d->num_kv_heads * 2 * sizeof(int32_t));
    return w;
}

}  // namespace
