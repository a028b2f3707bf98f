// Decode attention on the vector ALU only (no MFMA): the comparison point for
// the MFMA inner loop.  Same static split, same epilogues and combine, same
// masking rules; only the arithmetic engine differs.
//
// What is computed is the decode-attention definition of the SimpleLLM
// README's fused-kernel row (sinks, sliding window, GQA) over the paged cache
// or ring: scores s_p = q_h . K_p / sqrt(D), an online softmax, and
// sum_p e^(s_p-m) V_p, the sink joining only the final normaliser.
//
// Per 32-slot step, for the G <= 8 query heads of one KV group:
//   QK^T: lane l = (slot t = l/2, half = l%2) loads its half K row (64 B;
//         the K pool keeps each half of a block's rows slot-major, [2][bs][32],
//         so the wave reads whole cache lines) and forms
//         the eight half dot products with v_dot2_f32_bf16 from the queries
//         it keeps in registers; one lane swap completes each score.
//   max:  per head over the 32 slots, five lane-xor steps.
//   P:    e^(s - m) as bf16 pairs into LDS ([head][slot pair]).
//   PV:   lane = dimension d loads its V^T run of slots base..base+31, four
//         16-byte chunks (the V pool is transposed inside a block in chunks of
//         8 slots, so slot pairs are adjacent bf16) and
//         accumulates p . v with v_dot2_f32_bf16 against the broadcast P
//         pairs.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kGmax = 8;      // query heads per KV head this engine serves

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
    return __builtin_bit_cast(unsigned, v);
}

template <int BSL>
__global__ __launch_bounds__(64) void decode_valu_kernel(const DecodeArgs a) {
    __shared__ unsigned s_p[kGmax][16];     // P as bf16 pairs: [head][slot pair]
    constexpr int bs = 1 << BSL;
    const int lane = threadIdx.x;
    const int t = lane >> 1, half = lane & 1;   // QK role
    const int d = lane;                          // PV role: one dimension per lane
    const int units = a.B * a.Hkv;
    const int split = blockIdx.x / units;
    const int bg = blockIdx.x - split * units;
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    const int G = a.G;

    int n = a.seq_lens[b];
    if (a.window > 0) n = min(n, a.window);
    n = max(0, min(n, a.mbs << BSL));
    const int P = a.part_tokens;
    const int t0 = split * P;
    const size_t bh0 = (size_t)b * a.Hq + g * G;
    if (t0 >= n) {
        if (a.mode == kWritePartials) {
            if (lane < G) a.part_lse[(bh0 + lane) * a.num_splits + split] = -INFINITY;
        } else if (split == 0) {
            for (int h = 0; h < G; ++h) a.out[(bh0 + h) * kHeadDim + d] = 0;
        }
        return;
    }
    const int t1 = min(n, t0 + P);

    // queries: heads h < G, dims 32*half .. +31 as 16 bf16 pairs
    unsigned qr[kGmax][16];
#pragma unroll
    for (int h = 0; h < kGmax; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (h < G)
                v = *reinterpret_cast<const u32x4_t*>(a.q + (bh0 + h) * kHeadDim + 32 * half + 8 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) qr[h][4 * i + e] = v[e];
        }
    }

    // block-table slice of the partition, one entry per lane (<= 64 blocks)
    const int32_t* bt_row = a.block_table + (size_t)b * a.mbs;
    const int blk0 = t0 >> BSL;
    const int nblk = ((t1 - 1) >> BSL) - blk0 + 1;
    int tbl = 0;
    if (lane < nblk) tbl = min(max(bt_row[blk0 + lane], 0), a.num_blocks - 1);
    const unsigned blk_stride = (unsigned)(a.Hkv * bs * kHeadDim * 2);
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)g * bs * kHeadDim * 2;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)g * bs * kHeadDim * 2;

    float acc[kGmax], m[kGmax], lsum[kGmax];
#pragma unroll
    for (int h = 0; h < kGmax; ++h) {
        acc[h] = 0.f;
        m[h] = -INFINITY;
        lsum[h] = 0.f;
    }
    const int last_chunk = (t1 - 1) & ~7;

    for (int base = t0; base < t1; base += kStepTokens) {
        // K: half row of slot base + t (redirected to t1-1 past the end)
        const int slot = min(base + t, t1 - 1);
        const unsigned kblk = (unsigned)__builtin_amdgcn_ds_bpermute(((slot >> BSL) - blk0) << 2, tbl);
        const char* kp = kbase + (size_t)kblk * blk_stride +
                         ((unsigned)(half * bs + (slot & (bs - 1))) * 32) * 2;
        u32x4_t kr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kr[i] = *reinterpret_cast<const u32x4_t*>(kp + 16 * i);
        // V^T: dim d, slots base + 8c .. +7 for c = 0..3 (chunks past the end
        // redirected to the last live one and zeroed below)
        u32x4_t vr[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ch = min(base + 8 * c, last_chunk);
            const int vblk = __builtin_amdgcn_readlane(tbl, (ch >> BSL) - blk0);
            const char* vp = vbase + (size_t)(unsigned)vblk * blk_stride +
                             ((unsigned)((ch & (bs - 1)) >> 3) * kHeadDim + d) * 16;
            vr[c] = *reinterpret_cast<const u32x4_t*>(vp);
        }

        // scores of slot base + t for every head
        float s[kGmax];
#pragma unroll
        for (int h = 0; h < kGmax; ++h) {
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) x = dot2(qr[h][4 * i + e], kr[i][e], x);
            x += __shfl_xor(x, 1);                    // the other half of the row
            s[h] = base + t < t1 ? x * a.scale_log2 : -INFINITY;
        }
        // running max per head over the 32 slots
        float alpha[kGmax];
#pragma unroll
        for (int h = 0; h < kGmax; ++h) {
            float mx = s[h];
#pragma unroll
            for (int o = 2; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float m_new = fmaxf(m[h], mx);      // finite: slot base is live
            alpha[h] = __builtin_amdgcn_exp2f(m[h] - m_new);
            m[h] = m_new;
            const float p = __builtin_amdgcn_exp2f(s[h] - m_new);
            lsum[h] = lsum[h] * alpha[h] + p;         // this lane's slot; summed at the end
            const float p_next = __shfl_down(p, 2);   // slot t + 1 (lane + 2)
            if (half == 0 && (t & 1) == 0) s_p[h][t >> 1] = pack_bf16(p, p_next);
        }
        __syncthreads();
        // zero V of slots past the end (only in the last step)
        if (base + kStepTokens > t1) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int sl = base + 8 * c + 2 * w;
                    const unsigned mask = (sl < t1 ? 0x0000FFFFu : 0u) | (sl + 1 < t1 ? 0xFFFF0000u : 0u);
                    vr[c][w] &= mask;
                }
        }
        // PV for dimension d
#pragma unroll
        for (int h = 0; h < kGmax; ++h) {
            float x = acc[h] * alpha[h];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int w = 0; w < 4; ++w) x = dot2(s_p[h][4 * c + w], vr[c][w], x);
            acc[h] = x;
        }
        __syncthreads();
    }

    // per-head sums over the 32 slot lanes (the two halves hold equal values)
    float ltot[kGmax];
#pragma unroll
    for (int h = 0; h < kGmax; ++h) {
        float x = lsum[h];
#pragma unroll
        for (int o = 2; o < 64; o <<= 1) x += __shfl_xor(x, o);
        ltot[h] = x;
    }
    if (a.mode == kWriteOut) {
#pragma unroll
        for (int h = 0; h < kGmax; ++h) {
            if (h >= G) break;
            const float sig = a.sinks ? a.sinks[g * G + h] * kLog2e : -INFINITY;
            const float inv = 1.0f / (ltot[h] + __builtin_amdgcn_exp2f(sig - m[h]));
            const __bf16 o = (__bf16)(acc[h] * inv);
            a.out[(bh0 + h) * kHeadDim + d] = __builtin_bit_cast(uint16_t, o);
        }
        return;
    }
    const int S = a.num_splits;
#pragma unroll
    for (int h = 0; h < kGmax; ++h) {
        if (h >= G) break;
        a.part_o[((bh0 + h) * S + split) * kHeadDim + d] = acc[h] / ltot[h];
        if (lane == 0)
            a.part_lse[(bh0 + h) * S + split] = (m[h] + __builtin_amdgcn_logf(ltot[h])) * kLn2;
    }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream) {
    if (a.G > kGmax) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.B * a.Hkv * a.num_splits);
    switch (a.bs_log2) {
        case 3: return launch(decode_valu_kernel<3>, grid, dim3(64), 0, stream, a);
        case 4: return launch(decode_valu_kernel<4>, grid, dim3(64), 0, stream, a);
        case 5: return launch(decode_valu_kernel<5>, grid, dim3(64), 0, stream, a);
        case 6: return launch(decode_valu_kernel<6>, grid, dim3(64), 0, stream, a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sa
