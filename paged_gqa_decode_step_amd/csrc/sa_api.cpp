// C-ABI layer of libsa: argument checks, the fixed split table, launches.
//
// Nothing here allocates, frees or synchronises; every call checks its
// arguments completely before it enqueues any kernel on the caller's stream.
#include <limits.h>
#include <stdint.h>
#include <math.h>

#include "../../include/sa.h"
#include "sa_internal.h"

namespace {

using sa::kHeadDim;

// Fixed split table (no autotuning, so the result of a call never depends on
// timing).  A partition is 32 * 2^k slots, at most kMaxTableSlice blocks and
// at most kMaxPartTokens slots, and never longer than the context capacity
// (a 128-slot ring is one partition).  It halves, down to kMinPartTokens,
// while a call would have fewer than kMinWaves partition wavefronts.  Chosen
// from measured sweeps on MI355X: long partitions keep the partial traffic
// and the combine small; batch-1 calls trade some of that for parallelism.
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

// 16-byte vector accesses need 16-byte aligned bases (null passes: the
// null checks are separate)
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
template <typename... P>
bool all_aligned16(const P*... p) { return (aligned16(p) && ...); }

int log2_exact(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return (1 << l) == x ? l : -1;
}

// T: new tokens (query tokens) per sequence
int query_tokens(const sa_dims* d) { return d->num_query_tokens > 0 ? d->num_query_tokens : 1; }

int check_dims(const sa_dims* d, int32_t window) {
    if (!d) return SA_ERR_INVALID_ARG;
    if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
        d->max_blocks_per_seq < 1 || d->num_blocks < 1 || d->num_splits < 0 ||
        d->head_dim < 1 || d->block_size < 1 || d->num_query_tokens < 0)
        return SA_ERR_INVALID_ARG;
    if (d->head_dim != kHeadDim) return SA_ERR_UNSUPPORTED;
    if (d->num_q_heads % d->num_kv_heads) return SA_ERR_UNSUPPORTED;
    // (query tokens) x (heads per KV head) columns fill one 16-column MFMA tile
    if ((long long)query_tokens(d) * (d->num_q_heads / d->num_kv_heads) > sa::kMaxGroup)
        return SA_ERR_UNSUPPORTED;
    if (query_tokens(d) > 1 && window > 0) return SA_ERR_UNSUPPORTED;   // a W-slot ring
    const int l = log2_exact(d->block_size);
    if (l < 3 || l > 6) return SA_ERR_UNSUPPORTED;
    if (d->variant < SA_VARIANT_DEFAULT || d->variant > SA_VARIANT_MFMA_BALANCED)
        return SA_ERR_INVALID_ARG;
    if (window > 0 && (window + d->block_size - 1) / d->block_size > d->max_blocks_per_seq)
        return SA_ERR_INVALID_ARG;
    if ((long long)d->num_blocks * d->num_kv_heads * d->block_size * kHeadDim > (1LL << 40))
        return SA_ERR_INVALID_ARG;
    // a sequence's capacity in tokens, and slot arithmetic past it by one
    // partition, stay in the device's 32-bit ints
    if ((long long)d->max_blocks_per_seq * d->block_size > (1LL << 30)) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

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
constexpr int kCounterSlots = 1 << 16;   // (sequence, KV head) pairs a fused call may have
constexpr size_t kCounterBytes = (size_t)kCounterSlots * sizeof(int32_t);

struct WorkspaceLayout {
    size_t part_o, part_lse, counters, unit_seg, total;
};

enum class Mode { kStatic, kFused, kBalanced };

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

// Which kernel a call with these dims uses (assumes check_dims passed).
Mode choose_mode(const sa_dims* d, int32_t window, const Plan& p) {
    // the balanced kernel keeps its per-sequence table in LDS and walks steps
    // in 32-bit arithmetic
    const bool fits_stream =
        d->num_seqs <= kMaxStreamSeqs && stream_steps_upper(d, window) <= INT_MAX;
    switch (d->variant) {
        case SA_VARIANT_MFMA_BALANCED:
            return fits_stream ? Mode::kBalanced : Mode::kStatic;
        case SA_VARIANT_MFMA_FUSED:
            return (long long)d->num_seqs * d->num_kv_heads <= kCounterSlots ? Mode::kFused
                                                                             : Mode::kStatic;
        case SA_VARIANT_MFMA_TWO_PASS:
        case SA_VARIANT_VALU:
            return Mode::kStatic;
        default:
            // one static partition needs no merge at all; beyond that the
            // balanced kernel keeps every compute unit equally busy
            if (d->num_splits > 0 || p.splits == 1 || !fits_stream) return Mode::kStatic;
            return Mode::kBalanced;
    }
}

WorkspaceLayout workspace_layout(const sa_dims* d, int32_t window, const Plan& p, Mode m) {
    WorkspaceLayout w{};
    size_t rows, lse;        // partial rows of D floats, and lse entries
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

bool grid_fits(const sa_dims* d, int32_t splits) {
    return (long long)d->num_seqs * d->num_kv_heads * splits < INT_MAX &&
           (long long)d->num_seqs * query_tokens(d) * d->num_q_heads < INT_MAX;
}

sa::DecodeArgs decode_args(const sa_dims* d, int32_t window, const Plan& p) {
    sa::DecodeArgs a{};
    a.B = d->num_seqs;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.G = d->num_q_heads / d->num_kv_heads;
    a.T = query_tokens(d);
    a.bs_log2 = log2_exact(d->block_size);
    a.mbs = d->max_blocks_per_seq;
    a.num_blocks = d->num_blocks;
    a.window = window > 0 ? window : 0;
    a.num_splits = p.splits;
    a.part_tokens = p.part_tokens;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kHeadDim));
    return a;
}

int to_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

}  // namespace

extern "C" {

int sa_kv_append(const sa_bf16* k_new, const sa_bf16* v_new, sa_bf16* k_cache,
                 sa_bf16* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                 int32_t window, const sa_dims* dims, void* stream) {
    int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    if (dims->num_seqs == 0) return SA_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !seq_lens)
        return SA_ERR_INVALID_ARG;
    if (!all_aligned16(k_new, v_new, k_cache, v_cache)) return SA_ERR_INVALID_ARG;
    if ((long long)dims->num_seqs * dims->num_kv_heads >= INT_MAX) return SA_ERR_INVALID_ARG;
    sa::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.B = dims->num_seqs;
    a.Hkv = dims->num_kv_heads;
    a.bs_log2 = log2_exact(dims->block_size);
    a.mbs = dims->max_blocks_per_seq;
    a.num_blocks = dims->num_blocks;
    a.window = window > 0 ? window : 0;
    a.T = query_tokens(dims);
    return to_status(sa::launch_kv_append(a, (hipStream_t)stream));
}

int32_t sa_decode_num_splits(const sa_dims* dims, int32_t window) {
    const int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    return plan(dims, window).splits;
}

size_t sa_decode_workspace_bytes(const sa_dims* dims, int32_t window) {
    if (check_dims(dims, window) != SA_OK) return 0;
    const Plan p = plan(dims, window);
    return workspace_layout(dims, window, p, choose_mode(dims, window, p)).total;
}

}  // extern "C"

namespace {

// Attention, and with k_new/v_new the KV append in the same launch.
int decode(const sa_bf16* q, const sa_bf16* k_new, const sa_bf16* v_new,
           const sa_bf16* k_cache, const sa_bf16* v_cache, const int32_t* block_table,
           const int32_t* seq_lens, const float* sinks, int32_t window, const sa_rope* rope,
           sa_bf16* out, const sa_dims* dims, void* workspace, size_t workspace_bytes,
           void* stream) {
    int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    if (dims->num_seqs == 0) return SA_OK;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
        return SA_ERR_INVALID_ARG;
    if (!all_aligned16(q, k_cache, v_cache, out, k_new, v_new, workspace))
        return SA_ERR_INVALID_ARG;
    if (rope && (!rope->cos_table || !rope->sin_table || rope->max_positions < 1 ||
                 (rope->style != SA_ROPE_HALF && rope->style != SA_ROPE_INTERLEAVED) || !k_new ||
                 !all_aligned16(rope->cos_table, rope->sin_table)))
        return SA_ERR_INVALID_ARG;
    const bool valu = dims->variant == SA_VARIANT_VALU;
    if (valu && (dims->num_q_heads / dims->num_kv_heads > 8 || k_new || query_tokens(dims) > 1))
        return SA_ERR_UNSUPPORTED;
    if (rope && query_tokens(dims) > 1) return SA_ERR_UNSUPPORTED;
    const Plan p = plan(dims, window);
    if (!grid_fits(dims, p.splits)) return SA_ERR_INVALID_ARG;
    const Mode mode = choose_mode(dims, window, p);
    const bool with_rope = rope != nullptr;
    auto launch_static = [valu, with_rope](const sa::DecodeArgs& args, hipStream_t strm) {
        return valu ? sa::launch_decode_valu(args, strm)
                    : sa::launch_decode_mfma(args, with_rope, strm);
    };
    const WorkspaceLayout wl = workspace_layout(dims, window, p, mode);
    if (wl.total && (!workspace || workspace_bytes < wl.total)) return SA_ERR_WORKSPACE;

    sa::DecodeArgs a = decode_args(dims, window, p);
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.sinks = sinks;
    a.out = out;
    if (k_new) {
        a.k_new = k_new;
        a.v_new = v_new;
        a.k_store = const_cast<uint16_t*>(k_cache);
        a.v_store = const_cast<uint16_t*>(v_cache);
    }
    if (rope) {
        a.rope_cos = rope->cos_table;
        a.rope_sin = rope->sin_table;
        a.rope_max_pos = rope->max_positions;
        a.rope_style = rope->style == SA_ROPE_HALF ? sa::kRopeHalf : sa::kRopeInterleaved;
    }
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    if (mode == Mode::kBalanced) {
        a.part_o = (float*)(ws + wl.part_o);
        a.part_lse = (float*)(ws + wl.part_lse);
        a.unit_seg = (int32_t*)(ws + wl.unit_seg);
        a.num_waves = (int32_t)stream_waves(dims, window);
        return to_status(sa::launch_decode_stream(a, with_rope, s));
    }
    if (p.splits == 1) {
        a.mode = sa::kWriteOut;
        return to_status(launch_static(a, s));
    }
    a.part_o = (float*)(ws + wl.part_o);
    a.part_lse = (float*)(ws + wl.part_lse);
    a.counters = (int32_t*)(ws + wl.counters);
    if (mode == Mode::kFused) {
        a.mode = sa::kFusedCombine;
        return to_status(sa::launch_decode_mfma(a, with_rope, s));
    }
    a.mode = sa::kWritePartials;
    st = to_status(launch_static(a, s));
    if (st != SA_OK) return st;
    sa::CombineArgs c{};
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.sinks = sinks;
    c.out = out;
    c.B = a.B * a.T;              // partial / out rows (b*T + t)*Hq + h
    c.Hq = a.Hq;
    c.num_splits = p.splits;
    return to_status(sa::launch_combine(c, s));
}

}  // namespace

extern "C" {

int sa_decode_attention(const sa_bf16* q, const sa_bf16* k_cache, const sa_bf16* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const float* sinks, int32_t window, sa_bf16* out,
                        const sa_dims* dims, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return decode(q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, sinks, window,
                  nullptr, out, dims, workspace, workspace_bytes, stream);
}

int sa_decode_attention_append(const sa_bf16* q, const sa_bf16* k_new, const sa_bf16* v_new,
                               sa_bf16* k_cache, sa_bf16* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const float* sinks, int32_t window, sa_bf16* out,
                               const sa_dims* dims, void* workspace, size_t workspace_bytes,
                               void* stream) {
    const int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    if (dims->num_seqs == 0) return SA_OK;
    if (!k_new || !v_new) return SA_ERR_INVALID_ARG;
    return decode(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, sinks, window,
                  nullptr, out, dims, workspace, workspace_bytes, stream);
}

int sa_decode_attention_append_rope(const sa_bf16* q, const sa_bf16* k_new, const sa_bf16* v_new,
                                    sa_bf16* k_cache, sa_bf16* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const float* sinks, int32_t window, const sa_rope* rope,
                                    sa_bf16* out, const sa_dims* dims, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    const int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    if (dims->num_seqs == 0) return SA_OK;
    if (!k_new || !v_new || !rope) return SA_ERR_INVALID_ARG;
    return decode(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, sinks, window, rope,
                  out, dims, workspace, workspace_bytes, stream);
}

int sa_decode_partials(const sa_bf16* q, const sa_bf16* k_cache, const sa_bf16* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens, int32_t window,
                       float* part_o, float* part_lse, const sa_dims* dims, void* stream) {
    int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    if (dims->num_seqs == 0) return SA_OK;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !part_o || !part_lse)
        return SA_ERR_INVALID_ARG;
    if (!all_aligned16(q, k_cache, v_cache, part_o)) return SA_ERR_INVALID_ARG;
    if (dims->variant == SA_VARIANT_VALU) return SA_ERR_UNSUPPORTED;
    const Plan p = plan(dims, window);
    if (!grid_fits(dims, p.splits)) return SA_ERR_INVALID_ARG;
    sa::DecodeArgs a = decode_args(dims, window, p);
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.mode = sa::kWritePartials;
    return to_status(sa::launch_decode_mfma(a, false, (hipStream_t)stream));
}

int sa_combine(const float* part_o, const float* part_lse, const float* sinks,
               int32_t num_splits, sa_bf16* out, const sa_dims* dims, void* stream) {
    if (!dims) return SA_ERR_INVALID_ARG;
    if (dims->num_seqs < 0 || dims->num_q_heads < 1 || num_splits < 1 ||
        dims->num_query_tokens < 0)
        return SA_ERR_INVALID_ARG;
    if (dims->head_dim != kHeadDim) return SA_ERR_UNSUPPORTED;
    if (dims->num_seqs == 0) return SA_OK;
    if (!part_o || !part_lse || !out) return SA_ERR_INVALID_ARG;
    if ((long long)dims->num_seqs * query_tokens(dims) * dims->num_q_heads >= INT_MAX)
        return SA_ERR_INVALID_ARG;
    sa::CombineArgs c{};
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.sinks = sinks;
    c.out = out;
    c.B = dims->num_seqs * query_tokens(dims);
    c.Hq = dims->num_q_heads;
    c.num_splits = num_splits;
    return to_status(sa::launch_combine(c, (hipStream_t)stream));
}

int sa_read_bandwidth_probe(const void* data, size_t bytes, uint32_t* sink, void* stream) {
    if (!sink || (bytes && !data) || bytes % 16) return SA_ERR_INVALID_ARG;
    if (bytes == 0) return SA_OK;
    return to_status(sa::launch_read_probe(data, bytes, sink, (hipStream_t)stream));
}

const char* sa_status_string(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARG: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported shape";
        case SA_ERR_WORKSPACE: return "workspace missing or too small";
        case SA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
