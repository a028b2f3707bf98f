// C-ABI layer of libsa: argument checks and launches (the launch planning,
// split table and workspace layout, is plan.h).
//
// Nothing here allocates, frees or synchronises; every call checks its
// arguments completely before it enqueues any kernel on the caller's stream.
#include <limits.h>
#include <stdint.h>
#include <math.h>

#include "../../include/sa.h"
#include "plan.h"
#include "sa_internal.h"

static_assert(SA_SCRATCH_BYTES == sa::kScratchBytes, "the header states the scratch size");

namespace {

using sa::kHeadDim;

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

int check_dims(const sa_dims* d, int32_t window) {
    if (!d) return SA_ERR_INVALID_ARG;
    if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
        d->max_blocks_per_seq < 1 || d->num_blocks < 1 || d->num_splits < 0 ||
        d->head_dim < 1 || d->block_size < 1 || d->num_query_tokens < 0)
        return SA_ERR_INVALID_ARG;
    if (d->head_dim != kHeadDim) return SA_ERR_UNSUPPORTED;
    // the kernels read only the split-K / chunked-V pools; plain-row pools
    // (or a caller that never set the field) would be read as garbage
    if (d->cache_layout != SA_LAYOUT_K2_V8) return SA_ERR_UNSUPPORTED;
    if (d->num_q_heads % d->num_kv_heads) return SA_ERR_UNSUPPORTED;
    // (query tokens) x (heads per KV head) columns fill one 16-column MFMA tile
    if ((long long)query_tokens(d) * (d->num_q_heads / d->num_kv_heads) > sa::kMaxGroup)
        return SA_ERR_UNSUPPORTED;
    if (query_tokens(d) > 1 && window > 0) return SA_ERR_UNSUPPORTED;   // a W-slot ring
    const int l = log2_exact(d->block_size);
    if (l < 3 || l > 6) return SA_ERR_UNSUPPORTED;
    if (d->variant < SA_VARIANT_DEFAULT || d->variant > SA_VARIANT_MFMA_BALANCED_LAST_MERGES)
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

// Attention, and with k_new/v_new the KV append in the same launch.  With
// lib_scratch the call takes its workspace from the library's own device
// array instead of `workspace` (which is then ignored): after every argument
// check, so a bad call still touches no HIP state.
int decode(const sa_bf16* q, const sa_bf16* k_new, const sa_bf16* v_new,
           const sa_bf16* k_cache, const sa_bf16* v_cache, const int32_t* block_table,
           const int32_t* seq_lens, const float* sinks, int32_t window, const sa_rope* rope,
           sa_bf16* out, const sa_dims* dims, void* workspace, size_t workspace_bytes,
           void* stream, bool lib_scratch = false) {
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
    const int depth = static_depth(dims, p);
    auto launch_static = [valu, with_rope, depth](const sa::DecodeArgs& args, hipStream_t strm) {
        return valu ? sa::launch_decode_valu(args, strm)
                    : sa::launch_decode_mfma(args, with_rope, depth, strm);
    };
    const WorkspaceLayout wl = workspace_layout(dims, window, p, mode);
    if (lib_scratch) {
        if (wl.total > sa::kScratchBytes) return SA_ERR_SCRATCH;
        workspace = nullptr;
        workspace_bytes = 0;
        if (wl.total) {
            if (sa::scratch_pointer(&workspace) != hipSuccess) return SA_ERR_HIP;
            workspace_bytes = sa::kScratchBytes;
        }
    }
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
    if (mode == Mode::kBalanced || mode == Mode::kBalancedLastMerges) {
        const bool fused = mode == Mode::kBalancedLastMerges;
        a.part_o = (float*)(ws + wl.part_o);
        if (fused) {
            a.counters = (int32_t*)(ws + wl.counters);
        } else {
            a.part_lse = (float*)(ws + wl.part_lse);
            a.unit_seg = (int32_t*)(ws + wl.unit_seg);
        }
        a.num_waves = (int32_t)stream_waves(dims, window);
        return to_status(sa::launch_decode_stream(a, with_rope, fused, s));
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
        return to_status(sa::launch_decode_mfma(a, with_rope, depth, s));
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

int sa_decode_attention_append_noalloc(const sa_bf16* q, const sa_bf16* k_new,
                                       const sa_bf16* v_new, sa_bf16* k_cache, sa_bf16* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const float* sinks, int32_t window, sa_bf16* out,
                                       const sa_dims* dims, void* stream) {
    const int st = check_dims(dims, window);
    if (st != SA_OK) return st;
    if (dims->num_seqs == 0) return SA_OK;
    if (!k_new || !v_new) return SA_ERR_INVALID_ARG;
    return decode(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, sinks, window,
                  nullptr, out, dims, nullptr, 0, stream, /*lib_scratch=*/true);
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
    return to_status(sa::launch_decode_mfma(a, false, static_depth(dims, p), (hipStream_t)stream));
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
    if (!sink || (bytes && !data) || bytes % 16 || !aligned16(data)) return SA_ERR_INVALID_ARG;
    if (bytes == 0) return SA_OK;
    return to_status(sa::launch_read_probe(data, bytes, sink, (hipStream_t)stream));
}

int sa_read_tiles_probe(const void* data, size_t bytes, const int32_t* tiles, int64_t ntiles,
                        int32_t waves, uint32_t* sink, void* stream) {
    if (!sink || ntiles < 0 || waves < 1 || waves > 65535 || !aligned16(data))
        return SA_ERR_INVALID_ARG;
    if (ntiles == 0) return SA_OK;
    if (!data || !tiles || bytes < 2048 || bytes / 2048 > INT_MAX || ntiles > INT_MAX)
        return SA_ERR_INVALID_ARG;
    return to_status(sa::launch_tile_probe(data, bytes, tiles, ntiles, waves, sink,
                                           (hipStream_t)stream));
}

const char* sa_status_string(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARG: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported shape";
        case SA_ERR_WORKSPACE: return "workspace missing or too small";
        case SA_ERR_HIP: return "HIP launch failed";
        case SA_ERR_SCRATCH:
            return "call needs more device scratch than the library's fixed array "
                   "(SA_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
