// Internal interface between the C-ABI layer (sa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Launch a kernel and return the status of this launch alone (hipGetLastError
// after a triple-chevron launch would also report an error some earlier call
// left on the calling thread).  The arguments are converted to the kernel's
// parameter types.
template <typename T> struct same_type { using type = T; };
template <typename... P>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, typename same_type<P>::type... args) {
    void* ptrs[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
}

constexpr int kHeadDim = 64;       // D handled by the kernels
constexpr int kMaxGroup = 16;      // query columns per KV head: (query tokens) x (heads
                                   // per KV head) fill one 16-column MFMA tile
constexpr int kStepTokens = 32;    // tokens per inner step of the partition kernels
constexpr int kMaxTableSlice = 64; // block-table entries one partition may span
constexpr int kBurstSteps = 8;     // steps of a partition the burst kernels load at once
// widths of the static merge (combine_kernel): one wavefront merges a row of
// up to kCombineOneWave partials, four wavefronts up to kCombineFourWaves,
// eight any more (16 at a time each: measured 0.1-0.2 us faster than sixteen
// wavefronts on rows of 128 partials)
constexpr int kCombineOneWave = 8;
constexpr int kCombineFourWaves = 64;

struct AppendArgs {
    const uint16_t* k_new;
    const uint16_t* v_new;
    uint16_t* k_cache;
    uint16_t* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int32_t B, Hkv, bs_log2, mbs, num_blocks, window;
    int32_t T;                // new tokens per sequence (positions L-T .. L-1)
};

// What a partition kernel does with its result.
enum PartitionMode : int32_t {
    kWriteOut = 0,        // S == 1: apply the sink, write bf16 out
    kWritePartials = 1,   // write (o, lse) partials; empty partitions write lse = -inf
    kFusedCombine = 2,    // write partials; the last partition of a (b, g) merges them
};

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const float* sinks;       // may be null
    const uint16_t* k_new;    // non-null: append the new token in the same launch
    const uint16_t* v_new;
    uint16_t* k_store;        // the caches again, writable (with k_new)
    uint16_t* v_store;
    uint16_t* out;            // kWriteOut, kFusedCombine
    float* part_o;            // kWritePartials, kFusedCombine
    float* part_lse;
    int32_t* counters;        // kFusedCombine, balanced kernel with its merge inside:
                              // [B*Hkv] arrivals, zero between calls
    int32_t* unit_seg;        // balanced kernel: [B*Hkv][2] = (first partial slot, last
                              // wavefront) of each unit with a step, for its combine
    int32_t num_waves;        // balanced kernel: wavefronts in the grid
    int32_t B, Hq, Hkv, G;
    int32_t T;                // query tokens per sequence (1, or several: causal,
                              // kernels built for it); q / out rows (b*T + t)*Hq + h
    int32_t bs_log2, mbs, num_blocks, window;
    int32_t num_splits;       // S
    int32_t part_tokens;      // P: slots per partition (multiple of 32 and of bs)
    int32_t mode;             // PartitionMode
    float scale_log2;         // log2(e) / sqrt(D)
    // rotary embedding of q and k_new at position L-1 (kernels built with it)
    const float* rope_cos;    // [rope_max_pos][D/2]
    const float* rope_sin;
    int32_t rope_max_pos;
    int32_t rope_style;       // kRopeHalf or kRopeInterleaved
};

constexpr int kRopeHalf = 0;          // pairs (i, i + D/2)
constexpr int kRopeInterleaved = 1;   // pairs (2i, 2i + 1)

struct CombineArgs {
    const float* part_o;
    const float* part_lse;
    const float* sinks;       // may be null
    uint16_t* out;
    int32_t B, Hq, num_splits;
};

// Bytes of the library-owned device scratch (one array per GPU) that the
// no-allocation entry point uses instead of a caller's workspace.
constexpr size_t kScratchBytes = (size_t)32 << 20;
// Device address of that array on the calling thread's current device (looked
// up with hipGetSymbolAddress on the first call on a device, then kept).
hipError_t scratch_pointer(void** out);

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
// rope: the kernels built with the rotary embedding of q and k_new; a.T > 1:
// the kernels built for several causal query tokens per sequence
// burst: the kernels that load every step of a partition of at most 8 steps
// at once (for grids of short partitions)
hipError_t launch_decode_mfma(const DecodeArgs& a, bool rope, int depth, hipStream_t stream);
// fused_merge: the last wavefront of a split unit merges it (part_o holds the
// segments, counters the arrivals); otherwise a merge launch follows, reading
// part_o / part_lse and the unit records in unit_seg
hipError_t launch_decode_stream(const DecodeArgs& a, bool rope, bool fused_merge,
                                hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_read_probe(const void* data, size_t bytes, unsigned* sink, hipStream_t stream);
hipError_t launch_tile_probe(const void* data, size_t bytes, const int* tiles, long long ntiles,
                             int waves, unsigned* sink, hipStream_t stream);

}  // namespace sa
