// Log-sum-exp combine of split-K partials with the attention sink.
//
// The flash-decoding split of the decode step (the tutorial setup page's
// FlashAttention chapter names the tiled online softmax this rests on; the
// SimpleLLM README's fused decode-attention row is where the sink comes
// from): every partition j of (b, h) leaves o_j (its own softmax average of
// V) and lse_j = log sum e^s over its slots.  With M = max(max_j lse_j, sigma_h)
//     out = sum_j e^(lse_j - M) o_j / (sum_j e^(lse_j - M) + e^(sigma_h - M)).
// Partials with lse = -inf (empty partitions) carry no weight and are never
// read.  One wavefront per (b, h); lane = dimension, so every partial row is
// one coalesced 256-byte load.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (bh >= a.B * a.Hq) return;
    const int h = bh % a.Hq;
    const int S = a.num_splits;
    const float* lse = a.part_lse + (size_t)bh * S;
    const float sig = a.sinks ? a.sinks[h] : -INFINITY;
    float M = sig;
    for (int j = 0; j < S; ++j) M = fmaxf(M, lse[j]);
    float out = 0.f;
    if (M != -INFINITY) {
        float num = 0.f;
        float den = __builtin_amdgcn_exp2f((sig - M) * kLog2e);
        const float* po = a.part_o + (size_t)bh * S * kHeadDim + lane;
#pragma unroll 4
        for (int j = 0; j < S; ++j) {
            const float l = lse[j];
            if (l == -INFINITY) continue;
            const float w = __builtin_amdgcn_exp2f((l - M) * kLog2e);
            den += w;
            num += w * po[(size_t)j * kHeadDim];
        }
        out = num / den;
    }
    const __bf16 o = (__bf16)out;
    a.out[(size_t)bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, o);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)((a.B * a.Hq + 3) / 4);
    hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
