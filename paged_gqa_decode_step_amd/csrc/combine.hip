// Log-sum-exp combine of split-K partials with the attention sink.
//
// The flash-decoding split of the decode step (the tutorial setup page's
// FlashAttention chapter names the tiled online softmax this rests on; the
// SimpleLLM README's fused decode-attention row is where the sink comes
// from): every partition j of (b, h) leaves o_j (its own softmax average of
// V) and lse_j = log sum e^s over its slots.  With M = max(max_j lse_j, sigma_h)
//     out = sum_j e^(lse_j - M) o_j / (sum_j e^(lse_j - M) + e^(sigma_h - M)).
// Partials with lse = -inf (empty partitions) carry no weight: whatever their
// o holds (NaN included) never reaches the output.
//
// One workgroup per (b, h).  Up to kOneWaveSplits partitions, one wavefront
// reads every lse and o row at once (lane = dimension) and merges them: one
// round trip.  Beyond that, WAVES wavefronts: every wavefront finds M over all
// partials (lanes stride over them), then merges the partials j = w,
// w + WAVES, ... with lane = dimension, so each partial row is one coalesced
// 256-byte load and WAVES rows are in flight at once; the per-wave sums meet
// in LDS.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kOneWaveSplits = 8;   // partitions up to which one wavefront merges a row

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void combine_kernel(const CombineArgs a) {
    __shared__ float s_num[WAVES][64];
    __shared__ float s_den[WAVES];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int bh = blockIdx.x;
    const int h = bh % a.Hq;
    const int S = a.num_splits;
    const float* lse = a.part_lse + (size_t)bh * S;
    const float sig = a.sinks ? a.sinks[h] : -INFINITY;

    if (WAVES == 1) {
        // S <= kOneWaveSplits: every partial's lse (the row's, so the same on
        // all lanes) and o are read at once, one round trip; an empty
        // partition's o is read but selected away, whatever its bits
        float l[kOneWaveSplits], o[kOneWaveSplits];
#pragma unroll
        for (int j = 0; j < kOneWaveSplits; ++j) {
            l[j] = -INFINITY;
            o[j] = 0.f;
            if (j < S) {
                l[j] = lse[j];
                o[j] = a.part_o[((size_t)bh * S + j) * kHeadDim + lane];
            }
        }
        float M = sig;
#pragma unroll
        for (int j = 0; j < kOneWaveSplits; ++j) M = fmaxf(M, l[j]);
        if (M == -INFINITY) {                   // nothing attended and no sink
            a.out[(size_t)bh * kHeadDim + lane] = 0;
            return;
        }
        float num = 0.f, den = __builtin_amdgcn_exp2f((sig - M) * kLog2e);
#pragma unroll
        for (int j = 0; j < kOneWaveSplits; ++j) {
            const bool live = l[j] != -INFINITY;
            const float wt = live ? __builtin_amdgcn_exp2f((l[j] - M) * kLog2e) : 0.f;
            den += wt;
            num += live ? wt * o[j] : 0.f;
        }
        const __bf16 ob = (__bf16)(num / den);
        a.out[(size_t)bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, ob);
        return;
    }

    float M = sig;
    for (int j = lane; j < S; j += 64) M = fmaxf(M, lse[j]);
    M = wave_max(M);
    if (M == -INFINITY) {                     // nothing attended and no sink
        if (w == 0) a.out[(size_t)bh * kHeadDim + lane] = 0;
        return;
    }
    float num = 0.f, den = 0.f;
    const float* po = a.part_o + (size_t)bh * S * kHeadDim + lane;
#pragma unroll 8
    for (int j = w; j < S; j += WAVES) {
        const float l = lse[j];
        if (l == -INFINITY) continue;
        const float wt = __builtin_amdgcn_exp2f((l - M) * kLog2e);
        den += wt;
        num += wt * po[(size_t)j * kHeadDim];
    }
    if (WAVES > 1) {
        s_num[w][lane] = num;
        if (lane == 0) s_den[w] = den;
        __syncthreads();
        if (w != 0) return;
        num = 0.f;
        den = 0.f;
#pragma unroll
        for (int i = 0; i < WAVES; ++i) {
            num += s_num[i][lane];
            den += s_den[i];
        }
    }
    den += __builtin_amdgcn_exp2f((sig - M) * kLog2e);
    const __bf16 o = (__bf16)(num / den);
    a.out[(size_t)bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, o);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.B * a.Hq);
    if (a.num_splits <= kOneWaveSplits)
        return launch(combine_kernel<1>, grid, dim3(64), 0, stream, a);
    else if (a.num_splits <= 64)
        return launch(combine_kernel<4>, grid, dim3(256), 0, stream, a);
    else
        return launch(combine_kernel<16>, grid, dim3(1024), 0, stream, a);
}

}  // namespace sa
