// Decode attention, one split-K partition per 64-lane wavefront, on MFMA.
//
// What is computed (SimpleLLM README, optimisation table: one decode-attention
// kernel for sinks, sliding window and GQA over the paged cache / ring
// buffer; tutorial setup page, PagedAttention and FlashAttention chapters):
// for query head h of KV group g, scores s_p = q_h . K_p / sqrt(D) over the
// partition's slots, an online softmax over them, and sum_p e^(s_p-m) V_p.
// The per-head sink logit enters only the final normaliser (no value row).
//
// Work decomposition.  A workgroup is one wavefront and owns one
// (sequence b, KV head g, partition) triple.  It streams the partition's K and
// V once from HBM and serves all G <= 16 query heads of the group from the
// same registers: the group's queries form the 16-column operand of
// v_mfma_f32_16x16x32_bf16, so every K/V byte is read once per group, not
// once per query head.
//
// Per 32-slot step (2 blocks at bs = 16):
//   S^T[16 slots x 16 heads] = K[16 x 64] Q^T[64 x 16]   two M-tiles, 2 MFMAs each
//   O^T[64 dims x 16 heads] += V^T[64 x 32] P^T[32 x 16] four MFMAs
// Operand lanes: lane l = (c16 = l%16, q4 = l/16) supplies row/column c16 and
// the eight reduction elements of group q4.  The reduction index of both
// products is a free relabelling, so it is chosen to make every operand a
// single 16-byte load straight from the cache layout:
//   * QK^T reduces over dims: lane (c16, q4) holds dims 8*q4..+7 (kstep 0) and
//     32+8*q4..+7 (kstep 1) of its K row / of its query head;
//   * M-tile m row r holds slot base + 8*(r/4) + 4*m + r%4, so the S^T output
//     lane (head c16, q4) ends up with the scores of slots base+8*q4 .. +7;
//   * PV reduces over slots: that same lane feeds those eight probabilities
//     as its P^T column, and the V^T operand lane (dim row c16, q4) needs
//     V[dim][base+8*q4 .. +7], i.e. 16 contiguous bytes of the V^T block.
// No LDS, no barriers: cross-lane reductions of the softmax max/sum over the
// four q4 groups use v_permlane16_swap / v_permlane32_swap.
//
// Masking: only the last step of a partition can reach past its end t1.
// Chunks of 8 slots that start at or past t1 are redirected to the chunk
// holding t1-1 (an allocated block) for their loads; their scores become
// -inf and the V elements of slots >= t1 are zeroed, so stale or NaN data in
// a block tail can never reach the output.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// x[l] op x[l ^ 16] and x[l] op x[l ^ 32] without LDS: each swap gives every
// lane its own value in one result and its partner's in the other.
__device__ __forceinline__ float max_xor16(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
    return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Build-time tuning knobs (defaults are the measured best on MI355X):
//   SA_PIPE   register sets in the load pipeline (2: one step in flight
//             while the previous one computes);
//   SA_KV_NT  1: K/V loads carry the non-temporal hint (read-once data).
#ifndef SA_PIPE
#define SA_PIPE 2
#endif
#ifndef SA_KV_NT
#define SA_KV_NT 0
#endif
constexpr int kPipe = SA_PIPE;

__device__ __forceinline__ u32x4_t load16(const char* p) {
#if SA_KV_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#else
    return *reinterpret_cast<const u32x4_t*>(p);
#endif
}

struct StepRegs {
    u32x4_t k[4];   // [m*2 + kstep]
    u32x4_t v[4];   // dim tile j
};

__global__ __launch_bounds__(64) void decode_mfma_kernel(const DecodeArgs a) {
    const int lane = threadIdx.x;
    const int c16 = lane & 15;
    const int q4 = lane >> 4;
    const int units = a.B * a.Hkv;
    const int split = blockIdx.x / units;          // split-major: short sequences
    const int bg = blockIdx.x - split * units;     // leave early, late ids
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    const int h = g * a.G + c16;
    const bool head_ok = c16 < a.G;
    const int bs = 1 << a.bs_log2;

    int n = a.seq_lens[b];
    if (a.window > 0) n = min(n, a.window);
    n = max(0, min(n, a.mbs << a.bs_log2));
    const int P = a.part_tokens;
    const int t0 = split * P;

    if (t0 >= n) {
        if (a.mode == kWritePartials) {
            if (head_ok && q4 == 0)
                a.part_lse[((size_t)b * a.Hq + h) * a.num_splits + split] = -INFINITY;
        } else if (split == 0 && head_ok) {
            // nothing attended at all: the output is 0
            u32x2_t z = {0u, 0u};
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2_t*>(a.out + ((size_t)b * a.Hq + h) * kHeadDim +
                                            16 * j + 4 * q4) = z;
        }
        return;
    }
    const int t1 = min(n, t0 + P);

    // Block-table slice of this partition, one entry per lane.
    const int32_t* bt_row = a.block_table + (size_t)b * a.mbs;
    const int blk0 = t0 >> a.bs_log2;
    const int nblk = ((t1 - 1) >> a.bs_log2) - blk0 + 1;
    int tbl = 0;
    if (lane < nblk) {
        tbl = bt_row[blk0 + lane];
        tbl = min(max(tbl, 0), a.num_blocks - 1);
    }

    // Query operand: column c16 = head, dims 8*q4..+7 and 32+8*q4..+7.
    u32x4_t qop0 = {0u, 0u, 0u, 0u}, qop1 = {0u, 0u, 0u, 0u};
    if (head_ok) {
        const uint16_t* qp = a.q + ((size_t)b * a.Hq + h) * kHeadDim + 8 * q4;
        qop0 = *reinterpret_cast<const u32x4_t*>(qp);
        qop1 = *reinterpret_cast<const u32x4_t*>(qp + 32);
    }

    // Byte addressing: a (block, KV head) tile is bs*D bf16 in both pools.
    const unsigned blk_stride = (unsigned)(a.Hkv * bs * kHeadDim * 2);
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)g * bs * kHeadDim * 2;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)g * bs * kHeadDim * 2;
    const unsigned k_lane = (unsigned)((c16 & 3) * kHeadDim + 8 * q4) * 2;   // + slot row, dims
    const unsigned v_lane = (unsigned)(c16 * bs) * 2;                         // dim row c16
    const int last_chunk = (t1 - 1) & ~7;

    // Issue the 8 loads of step s (K: 2 M-tiles x 2 k-steps; V: 4 dim tiles).
    auto load_step = [&](int s, StepRegs& r) {
        const int base = t0 + (s << 5);
        int kc = base + ((c16 >> 2) << 3);           // 8-slot chunk of this lane's K rows
        int vc = base + (q4 << 3);                   // 8-slot chunk of this lane's V^T run
        kc = kc < t1 ? kc : last_chunk;
        vc = vc < t1 ? vc : last_chunk;
        const unsigned kblk = (unsigned)__builtin_amdgcn_ds_bpermute(((kc >> a.bs_log2) - blk0) << 2, tbl);
        const unsigned vblk = (unsigned)__builtin_amdgcn_ds_bpermute(((vc >> a.bs_log2) - blk0) << 2, tbl);
        const char* kp = kbase + (size_t)kblk * blk_stride +
                         ((unsigned)(kc & (bs - 1)) * kHeadDim * 2 + k_lane);
        const char* vp = vbase + (size_t)vblk * blk_stride + ((unsigned)(vc & (bs - 1)) * 2 + v_lane);
        r.k[0] = load16(kp);
        r.k[1] = load16(kp + 64);
        r.k[2] = load16(kp + 4 * kHeadDim * 2);
        r.k[3] = load16(kp + 4 * kHeadDim * 2 + 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) r.v[j] = load16(vp + (size_t)j * 16 * bs * 2);
    };

    f32x4_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max, log2 domain, per head (equal on its 4 lanes)
    float l_run = 0.f;         // this lane's share of the running sum

    auto compute_step = [&](int s, StepRegs& r) {
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        s0 = mfma(r.k[0], qop0, s0);
        s0 = mfma(r.k[1], qop1, s0);
        s1 = mfma(r.k[2], qop0, s1);
        s1 = mfma(r.k[3], qop1, s1);
        float t[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t[i] = s0[i] * a.scale_log2;
            t[4 + i] = s1[i] * a.scale_log2;
        }
        const int tok = t0 + (s << 5) + (q4 << 3);   // slot of t[0] on this lane
        if (tok + 8 > t1) {                           // only in a partition's last step
            const int valid = max(0, min(8, t1 - tok));
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e >= valid) t[e] = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const unsigned mask = (2 * w < valid ? 0x0000FFFFu : 0u) |
                                      (2 * w + 1 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
                for (int j = 0; j < 4; ++j) r.v[j][w] &= mask;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])),
                         fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
        mx = max_xor32(max_xor16(mx));
        const float m_new = fmaxf(m_run, mx);        // finite: every step has a live slot
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(t[e] - m_new);
            psum += p[e];
        }
        l_run = l_run * alpha + psum;
        const u32x4_t pop = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                             pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[j] *= alpha;
            acc[j] = mfma(r.v[j], pop, acc[j]);
        }
        m_run = m_new;
    };

    // Software pipeline over kPipe register sets: while step s computes, the
    // loads of the next kPipe-1 steps are in flight.  Steps go in groups of
    // kPipe; steps past the end are wholly masked (alpha = 1, p = 0) and
    // prefetches past the last step re-read it (a cache hit), so the loop
    // body has no branch around a load.
    const int nsteps = (t1 - t0 + kStepTokens - 1) / kStepTokens;
    const int last = nsteps - 1;
    StepRegs R[kPipe];
#pragma unroll
    for (int i = 0; i < kPipe - 1; ++i) load_step(min(i, last), R[i]);
    for (int s = 0; s < nsteps; s += kPipe) {
#pragma unroll
        for (int i = 0; i < kPipe; ++i) {
            load_step(min(s + i + kPipe - 1, last), R[(i + kPipe - 1) % kPipe]);
            // keep the prefetch ahead of this step's math in the schedule
            __builtin_amdgcn_sched_barrier(0);
            compute_step(s + i, R[i]);
        }
    }

    const float l_tot = sum_xor32(sum_xor16(l_run));
    const size_t bh = (size_t)b * a.Hq + h;

    if (a.mode == kWriteOut) {
        if (!head_ok) return;
        const float sig = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
        const float inv = 1.0f / (l_tot + __builtin_amdgcn_exp2f(sig - m_run));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x2_t o = {pack_bf16(acc[j][0] * inv, acc[j][1] * inv),
                               pack_bf16(acc[j][2] * inv, acc[j][3] * inv)};
            *reinterpret_cast<u32x2_t*>(a.out + bh * kHeadDim + 16 * j + 4 * q4) = o;
        }
        return;
    }

    // Partials: o = acc / l, lse = ln(sum e^s) = (m + log2 l) * ln 2.
    const int S = a.num_splits;
    if (head_ok) {
        const float inv = 1.0f / l_tot;
        float* po = a.part_o + (bh * S + split) * kHeadDim + 4 * q4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4_t*>(po + 16 * j) = acc[j] * inv;
        if (q4 == 0)
            a.part_lse[bh * S + split] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    if (a.mode != kFusedCombine) return;

    // Fused combine: the last partition of (b, g) to finish merges them all.
    const int nparts = (n + P - 1) / P;
    __threadfence();
    __syncthreads();
    int prev = 0;
    if (lane == 0) prev = atomicAdd(a.counters + bg, 1);
    prev = __shfl(prev, 0);
    if (prev != nparts - 1) return;
    __threadfence();
    if (lane == 0) a.counters[bg] = 0;               // ready for the next call
    if (!head_ok) return;

    const float sig = a.sinks ? a.sinks[h] : -INFINITY;   // natural log
    float M = sig;
    for (int j = 0; j < nparts; ++j) M = fmaxf(M, a.part_lse[bh * S + j]);
    f32x4_t num[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) num[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float den = __builtin_amdgcn_exp2f((sig - M) * kLog2e);
    for (int j = 0; j < nparts; ++j) {
        const float w = __builtin_amdgcn_exp2f((a.part_lse[bh * S + j] - M) * kLog2e);
        den += w;
        const float* po = a.part_o + (bh * S + j) * kHeadDim + 4 * q4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            num[jj] += w * *reinterpret_cast<const f32x4_t*>(po + 16 * jj);
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x2_t o = {pack_bf16(num[j][0] * inv, num[j][1] * inv),
                           pack_bf16(num[j][2] * inv, num[j][3] * inv)};
        *reinterpret_cast<u32x2_t*>(a.out + bh * kHeadDim + 16 * j + 4 * q4) = o;
    }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)a.B * a.Hkv * a.num_splits;
    hipLaunchKernelGGL(decode_mfma_kernel, dim3(grid), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
