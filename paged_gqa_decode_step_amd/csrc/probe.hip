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
