// Decode attention with a static split: one wavefront per
// (sequence b, KV head g, partition of P slots).
//
// Partition `split` of (b, g) covers slots [split*P, min(n, (split+1)*P)) of
// the n attended slots (n = L for a paged layer, min(L, W) for a ring).  With
// one partition the wavefront applies the sink and writes bf16 out; otherwise
// it writes the partial (o, lse) that the combine kernel merges (the
// tutorial setup page's FlashAttention chapter names the tiled online
// softmax; the split-K partials are its flash-decoding form).  The fused
// mode lets the last partition of a (b, g) to finish merge the partials
// itself, behind a device-scope fence and an atomic counter.
//
// The per-step MFMA machinery lives in mfma_attend.h.
#include "mfma_attend.h"

namespace sa {
namespace {

using namespace mfma;

// DEPTH: the step pipeline (2), or a burst (4 or kBurst: every step of a
// partition of at most DEPTH steps loaded at once).
template <int BSL, bool ROPE, bool MULTI, int DEPTH>
__global__ __launch_bounds__(64) void decode_mfma_kernel(const DecodeArgs a) {
    const int lane = threadIdx.x;
    const int c16 = lane & 15;
    const int q4 = lane >> 4;
    const int units = a.B * a.Hkv;
    const int split = blockIdx.x / units;          // split-major: short sequences
    const int bg = blockIdx.x - split * units;     // leave early, late ids
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    const Col col = column(a, lane);
    const bool head_ok = col.ok;
    const int P = a.part_tokens;
    const int t0 = split * P;

    // The partition's slots follow from the grid alone, so the loads that
    // do not depend on the sequence's length (the query, the first table
    // slice, the new token's words) go out with the length's load, not after
    // its wait.
    u32x4_t qop0, qop1;
    if (!ROPE) load_query<false>(a, b, g, lane, qop0, qop1);
    Unit u = make_unit(a, b, g, lane);
    const RunStart pre = run_start<BSL>(u, t0, lane);

    const int L = a.seq_lens[b];
    int n = L;
    if (a.window > 0) n = min(n, a.window);
    n = max(0, min(n, a.mbs << a.bs_log2));
    const size_t bh = col_row(a, b, g, col);       // this lane's (token, head) row

    // A partition past the context attends one slot at t0 (inside its
    // table's allocated entries: a partition starts below the capacity) and
    // drops the result, instead of returning early: a branch here would let
    // the compiler sink the loads above past the length's wait.  Its run holds
    // no new token's slot (those lie below the context end), so it stores
    // nothing.
    const bool active = t0 < n;                    // wave-uniform
    const int t1 = active ? min(n, t0 + P) : t0 + 1;
    const int pos = ROPE && L > 0 ? rope_row(a, L) : 0;
    if (ROPE) load_query<true>(a, b, g, lane, qop0, qop1, pos);
    u.new_slot = MULTI ? -1 : new_token_slot(a, L, n);
    u.rope_pos = pos;
    u.L = L;
    State st;
    st.reset();
    attend<BSL, ROPE, MULTI, DEPTH>(a, u, t0, t1, qop0, qop1, st, pre);
    if (!active) {
        if (a.mode == kWritePartials) {
            if (head_ok && q4 == 0) a.part_lse[bh * a.num_splits + split] = -INFINITY;
        } else if (split == 0) {
            write_zero(a, b, g, lane);                // nothing attended at all
        }
        return;
    }
    const float l_tot = st.total();

    if (a.mode == kWriteOut) {
        write_out(a, b, g, lane, st, l_tot);
        return;
    }
    const int S = a.num_splits;
    write_partial(head_ok, bh, lane, st, l_tot, a.part_o + (size_t)split * kHeadDim,
                  (size_t)S * kHeadDim, a.part_lse + split, (size_t)S);
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

    const float sig = a.sinks ? a.sinks[g * a.G + col.h] : -INFINITY;   // natural log
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

template <bool ROPE, bool MULTI, int DEPTH>
hipError_t launch_static(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.B * a.Hkv * a.num_splits);
    switch (a.bs_log2) {
        case 3: return launch(decode_mfma_kernel<3, ROPE, MULTI, DEPTH>, grid, dim3(64), 0, stream, a);
        case 4: return launch(decode_mfma_kernel<4, ROPE, MULTI, DEPTH>, grid, dim3(64), 0, stream, a);
        case 5: return launch(decode_mfma_kernel<5, ROPE, MULTI, DEPTH>, grid, dim3(64), 0, stream, a);
        case 6: return launch(decode_mfma_kernel<6, ROPE, MULTI, DEPTH>, grid, dim3(64), 0, stream, a);
        default: return hipErrorInvalidValue;
    }
}

template <int DEPTH>
hipError_t launch_static_depth(const DecodeArgs& a, bool rope, hipStream_t stream) {
    if (a.T > 1) return rope ? hipErrorInvalidValue : launch_static<false, true, DEPTH>(a, stream);
    return rope ? launch_static<true, false, DEPTH>(a, stream)
                : launch_static<false, false, DEPTH>(a, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, bool rope, int depth, hipStream_t stream) {
    switch (depth) {
        case kBurst: return launch_static_depth<kBurst>(a, rope, stream);
        case 4: return launch_static_depth<4>(a, rope, stream);
        default: return launch_static_depth<2>(a, rope, stream);
    }
}

}  // namespace sa
