// A plain streaming read of a device buffer: the practical HBM read ceiling
// that the decode kernels are compared against.  Every 16-byte piece is read
// once, with the non-temporal hint the decode kernels' K/V loads carry, and
// every 32-bit word is folded into an XOR so the reads cannot be dropped and
// the result can be checked.
#include "sa_internal.h"

namespace sa {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kPerThread = 32;               // 16-byte loads per lane
constexpr size_t kMaxProbeBlocks = size_t(1) << 24;

// Workgroup w reads the contiguous 128 KiB [w*256*32, (w+1)*256*32) pieces
// (lane-contiguous 4 KiB per load instruction, 32 instructions), all loads
// issued before any is used; the grid covers the buffer in one round.  Many
// short workgroups, each on one contiguous stretch, measured fastest of the
// forms tried (long grid-stride loops, or pieces spread across the buffer,
// reached 6.4-7.0 TB/s against 7.2 here).
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* p, size_t n16,
                                                                   unsigned* sink) {
    const size_t step = (size_t)gridDim.x * kProbeThreads * kPerThread;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * kProbeThreads * kPerThread + threadIdx.x; i < n16;
         i += step) {
        u32x4_t v[kPerThread];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const size_t j = i + (size_t)k * kProbeThreads;
            v[k] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) acc ^= v[k];
    }
    unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0 && x != 0u) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_read_probe(const void* data, size_t bytes, unsigned* sink, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t per_block = (size_t)kProbeThreads * kPerThread;
    size_t blocks = (n16 + per_block - 1) / per_block;
    if (blocks > kMaxProbeBlocks) blocks = kMaxProbeBlocks;    // then lanes loop
    return launch(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                  reinterpret_cast<const u32x4_t*>(data), n16, sink);
}

}  // namespace sa

// ---------------------------------------------------------------------------
// Scattered-tile read: the decode kernels' access pattern with no arithmetic.
//
// tiles[0..ntiles) are tile numbers; tile k is the 2 KiB at data + k * 2048
// (one (block, KV head) piece of a pool at block size 16).  Wavefront w of
// `waves` one-wavefront workgroups reads the contiguous stretch [w*ntiles /
// waves, (w+1)*ntiles / waves) of the list, as the balanced decode kernel walks
// its steps: 8 KiB steps (four tiles: a K and a V piece of two blocks),
// three steps of loads in flight, the tile numbers of 64 tiles loaded with one
// load per lane and handed to each tile's lanes by a cross-lane read (as the
// decode kernels read block-table slices).  Every 32-bit word read is XORed
// into *sink, so the reads cannot be dropped and the result can be checked.
// ---------------------------------------------------------------------------
namespace sa {
namespace {

constexpr int kTileBytes = 2048;
constexpr int kTilesPerStep = 4;          // 8 KiB a step
constexpr int kTilesPerSlice = 64;        // tile numbers fetched at once (one a lane)
constexpr int kStepsPerSlice = kTilesPerSlice / kTilesPerStep;

struct TileStep {
    u32x4_t v[kTilesPerStep * 2];         // two 16-byte loads a lane per 2 KiB tile
};

__global__ __launch_bounds__(64) void tile_probe_kernel(const char* base, const int* tiles,
                                                        long long ntiles, int waves, int max_tile,
                                                        unsigned* sink) {
    const int lane = threadIdx.x;
    const long long w = blockIdx.x;
    const long long t0 = w * ntiles / waves;
    const long long t1 = (w + 1) * ntiles / waves;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (long long g = t0; g < t1; g += kTilesPerSlice) {
        // this slice's tile numbers, one a lane (lanes past the stretch take
        // its last tile, which the loads may read again but never fold in),
        // clamped into the buffer
        const long long last = t1 - 1;
        const int id = min(max(tiles[min(g + lane, last)], 0), max_tile);
        const int n = (int)min((long long)kTilesPerSlice, t1 - g);      // wave-uniform
        auto load = [&](int s, TileStep& r) {
#pragma unroll
            for (int c = 0; c < kTilesPerStep; ++c) {
                const int k = min(s * kTilesPerStep + c, n - 1);
                const int tid = __shfl(id, k);
                const u32x4_t* p =
                    reinterpret_cast<const u32x4_t*>(base + (size_t)(unsigned)tid * kTileBytes) +
                    lane;
                r.v[2 * c] = __builtin_nontemporal_load(p);
                r.v[2 * c + 1] = __builtin_nontemporal_load(p + 64);
            }
        };
        auto use = [&](int s, const TileStep& r) {
#pragma unroll
            for (int c = 0; c < kTilesPerStep; ++c) {
                if (s * kTilesPerStep + c < n) {          // wave-uniform: a tile read once
                    acc ^= r.v[2 * c];
                    acc ^= r.v[2 * c + 1];
                }
            }
        };
        TileStep A, B, C;
        load(0, A);
        load(1, B);
#pragma unroll
        for (int s = 0; s < kStepsPerSlice; s += 3) {
            if (s + 2 < kStepsPerSlice) load(s + 2, C);
            __builtin_amdgcn_sched_barrier(0);
            use(s, A);
            if (s + 3 < kStepsPerSlice) load(s + 3, A);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < kStepsPerSlice) use(s + 1, B);
            if (s + 4 < kStepsPerSlice) load(s + 4, B);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 2 < kStepsPerSlice) use(s + 2, C);
        }
    }
    unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
    if (lane == 0 && x != 0u) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_tile_probe(const void* data, size_t bytes, const int* tiles, long long ntiles,
                             int waves, unsigned* sink, hipStream_t stream) {
    const int max_tile = (int)(bytes / kTileBytes) - 1;
    return launch(tile_probe_kernel, dim3((unsigned)waves), dim3(64), 0, stream,
                  reinterpret_cast<const char*>(data), tiles, ntiles, waves, max_tile, sink);
}

}  // namespace sa
