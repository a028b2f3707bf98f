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
// One workgroup per (b, h) of WAVES wavefronts.  Wavefront w merges
// partitions w*CHUNK .. in chunks of CHUNK, reading every lse and o row of a
// chunk at once (lane = dimension, so each partial row is one coalesced
// 256-byte load; past the last partition nothing is read): one memory round
// trip when S <= WAVES x CHUNK.  The wavefronts' running (max, numerator,
// denominator) meet in LDS.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int WAVES, int CHUNK>
__global__ __launch_bounds__(64 * WAVES) void combine_kernel(const CombineArgs a) {
    __shared__ float s_num[WAVES][64];
    __shared__ float s_den[WAVES];
    __shared__ float s_max[WAVES];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int bh = blockIdx.x;
    const int h = bh % a.Hq;
    const int S = a.num_splits;
    const float* lse = a.part_lse + (size_t)bh * S;
    const float* po = a.part_o + (size_t)bh * S * kHeadDim + lane;
    const float sig = a.sinks ? a.sinks[h] : -INFINITY;

    // running merge of this wavefront's partitions: sum_j e^(l_j - M) o_j and
    // sum_j e^(l_j - M); partitions with lse = -inf carry no weight and their
    // o (whatever its bits) is selected away
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int j0 = w * CHUNK; j0 < S; j0 += WAVES * CHUNK) {
        float l[CHUNK], o[CHUNK];
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
            l[c] = -INFINITY;
            o[c] = 0.f;
            if (j0 + c < S) {            // wave-uniform; the loads still all go out first
                l[c] = lse[j0 + c];
                o[c] = po[(size_t)(j0 + c) * kHeadDim];
            }
        }
        float M2 = M;
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) M2 = fmaxf(M2, l[c]);
        if (M2 == -INFINITY) continue;   // nothing live yet
        const float r = __builtin_amdgcn_exp2f((M - M2) * kLog2e);   // 0 while M = -inf
        float cn = 0.f, cd = 0.f;
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
            const bool live = l[c] != -INFINITY;
            const float wt = live ? __builtin_amdgcn_exp2f((l[c] - M2) * kLog2e) : 0.f;
            cn += live ? wt * o[c] : 0.f;
            cd += wt;
        }
        num = num * r + cn;
        den = den * r + cd;
        M = M2;
    }
    if (WAVES > 1) {
        s_num[w][lane] = num;
        if (lane == 0) {
            s_den[w] = den;
            s_max[w] = M;
        }
        __syncthreads();
        if (w != 0) return;
        M = -INFINITY;
#pragma unroll
        for (int i = 0; i < WAVES; ++i) M = fmaxf(M, s_max[i]);
        num = 0.f;
        den = 0.f;
#pragma unroll
        for (int i = 0; i < WAVES; ++i) {
            if (s_max[i] == -INFINITY) continue;    // a wavefront with nothing live
            const float r = __builtin_amdgcn_exp2f((s_max[i] - M) * kLog2e);
            num += s_num[i][lane] * r;
            den += s_den[i] * r;
        }
    }
    // the sink joins the denominator only
    const float M2 = fmaxf(M, sig);
    if (M2 == -INFINITY) {                         // nothing attended and no sink
        a.out[(size_t)bh * kHeadDim + lane] = 0;
        return;
    }
    const float r = __builtin_amdgcn_exp2f((M - M2) * kLog2e);
    den = den * r + __builtin_amdgcn_exp2f((sig - M2) * kLog2e);
    const __bf16 ob = (__bf16)(num * r / den);
    a.out[(size_t)bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, ob);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.B * a.Hq);
    if (a.num_splits <= kCombineOneWave)
        return launch(combine_kernel<1, kCombineOneWave>, grid, dim3(64), 0, stream, a);
    else if (a.num_splits <= kCombineFourWaves)
        return launch(combine_kernel<4, kCombineFourWaves / 4>, grid, dim3(256), 0, stream, a);
    else
        return launch(combine_kernel<8, 16>, grid, dim3(512), 0, stream, a);
}

}  // namespace sa
