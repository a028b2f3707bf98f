// KV append: the new tokens' K and V go to their paged blocks or ring slots.
//
// SimpleLLM README, optimisation table: the fused decode-attention kernel
// also performs the KV append; full-attention layers keep a paged cache and
// sliding-window layers a ring buffer.  Position p of sequence b lives in
// slot p (paged) or p mod W (ring); the slot's block comes from the block
// table.  Inside a block K is stored [2][bs][32] (each half of a row, 32
// dimensions, slot-major) and V [bs/8][D][8] (transposed in chunks of 8
// slots).  With T new tokens per sequence (a query tile; paged layers only)
// token t sits at position L-T+t; one token is position L-1.
//
// One 64-lane wavefront per (sequence, KV head), token by token: lanes 0..7
// store the K row as eight 16-byte stores (four per 64-byte half); all 64
// lanes store one 2-byte V element each (the V column of the slot).  A bit
// copy; no arithmetic on the values.
#include "sa_internal.h"

namespace sa {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void kv_append_kernel(const AppendArgs a) {
    const int lane = threadIdx.x;
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    const int L = a.seq_lens[b];
    const int bs = 1 << a.bs_log2;
    // new token t of the sequence sits at position L - T + t (one token: L - 1)
    for (int t = 0; t < a.T; ++t) {
        const int p = L - a.T + t;
        if (p < 0) continue;
        const int slot = a.window > 0 ? p % a.window : p;
        const int j = slot >> a.bs_log2;
        if (j >= a.mbs) continue;                                // beyond the table row
        const int blk = a.block_table[(size_t)b * a.mbs + j];
        if (blk < 0 || blk >= a.num_blocks) continue;            // never write wild
        const int off = slot & (bs - 1);
        const size_t head_base = ((size_t)blk * a.Hkv + g) * (size_t)(bs * kHeadDim);
        const size_t src = (((size_t)b * a.T + t) * a.Hkv + g) * kHeadDim;
        if (lane < kHeadDim / 8) {
            const u32x4_t k = *reinterpret_cast<const u32x4_t*>(a.k_new + src + lane * 8);
            // dims 8*lane .. +7: half lane/4, 16-byte piece lane%4 of it
            const size_t kdst = head_base + ((size_t)(lane >> 2) * bs + off) * 32 + (lane & 3) * 8;
            *reinterpret_cast<u32x4_t*>(a.k_cache + kdst) = k;
        }
        a.v_cache[head_base + ((size_t)(off >> 3) * kHeadDim + lane) * 8 + (off & 7)] =
            a.v_new[src + lane];
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    return launch(kv_append_kernel, dim3(a.B * a.Hkv), dim3(64), 0, stream, a);
}

}  // namespace sa
