// Decode attention with balanced work: every wavefront gets the same number
// of 32-slot steps, whatever the mix of context lengths in the batch.
//
// The n_b attended slots of sequence b (n = L for a paged layer, min(L, W)
// for a ring) make ceil(n_b / 32) steps for each of its Hkv units
// (b, g).  Laying the units out one after another gives T steps in all;
// wavefront i of NW takes steps [i*T/NW, (i+1)*T/NW) and walks them unit by
// unit.  A unit it covers whole gets its bf16 output (with the sink)
// directly (a sequence with nothing to attend gets zeros from the wavefront
// that finished the sequence before it, or from wavefront 0); a unit it
// covers in part leaves a partial (o, lse), which only
// its first and last unit can need, so each wavefront owns two partial slots.
// combine_stream_kernel then merges, for each unit spread over wavefronts
// i0..i1, the slots those wavefronts left (the log-sum-exp merge of the
// flash-decoding split; the tutorial setup page's FlashAttention chapter
// names the online softmax it rests on).
//
// Every wavefront derives T and the unit layout itself from seq_lens (an
// inclusive scan in LDS), so there is no planning launch.
//
// Merging a unit spread over wavefronts i0..i1.  By default the wavefronts
// holding a unit's first and last steps record the unit's first partial
// slot and its last wavefront, and combine_stream_kernel merges in a launch
// of its own.  With FUSED (SA_VARIANT_MFMA_BALANCED_LAST_MERGES) each of them
// stores its segment (o, lse) with agent-coherent stores (sc1: written
// through this XCD's L2, so a wavefront on another XCD reads them) as soon as
// it has it, and once its whole range is done waits until those stores are
// complete and counts its arrivals on the units' counters with device-scope
// atomics; the wavefront that arrives last at a unit reads every segment
// with agent-coherent loads, merges them with the sink, writes the bf16
// output and returns the counter to zero.  That needs no device-scope fence
// (an L2 write-back) and no second launch, but measured slower than the
// merge launch on every workload (the write-back wait, the counted arrival
// and the merging wavefront's reads are dependent round trips, and a unit
// spread over many wavefronts is merged by one), so it is not the default.
// The per-step MFMA machinery is mfma_attend.h.
#include "mfma_attend.h"

namespace sa {
namespace {

using namespace mfma;

__device__ __forceinline__ int attended(const DecodeArgs& a, int L) {
    int n = a.window > 0 ? min(L, a.window) : L;
    return max(0, min(n, a.mbs << a.bs_log2));
}

// first step of wavefront i (T > 0)
__device__ __forceinline__ long long wave_start(long long i, long long T, long long NW) {
    return i * T / NW;
}

// wavefront holding step x: the i with wave_start(i) <= x < wave_start(i+1)
__device__ __forceinline__ int wave_of(long long x, long long T, long long NW) {
    return (int)(((x + 1) * NW - 1) / T);
}

// A segment of a unit in the fused merge: o = acc / l (16 values a lane) and
// the log2-domain lse of the lane's column, stored lane-major so each store
// and load instruction covers 256 contiguous bytes.
constexpr int kSegFloats = 17 * 64;

__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_segment(float* seg, int lane, const State& st, float l_tot) {
    // a column with no slot in the segment (several query tokens only) has
    // weight 0: lse = -inf, o = 0
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_agent(seg + (j * 4 + e) * 64 + lane, st.acc[j][e] * inv);
    store_agent(seg + 16 * 64 + lane, empty ? -INFINITY : st.m + __builtin_amdgcn_logf(l_tot));
}

// The last wavefront to arrive at a unit spread over wavefronts i0..i1 merges
// their segments (its own included, read back like the others) with the sink
// and writes the bf16 output.  Segment k is wavefront i0 + k's: in slot
// `first` for k = 0 (the unit may be that wavefront's second), else in slot
// 2 (i0 + k) (its first).
constexpr int kMergeChunk = 4;
__device__ __forceinline__ void merge_unit(const DecodeArgs& a, int b, int g, int lane, int i0,
                                           int i1, int first) {
    // running merge, log2 domain: out = num / (den + 2^(sigma - M)), all
    // scaled by 2^-M
    float M = -INFINITY;
    float num[16];
    float den = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) num[v] = 0.f;
    const int nseg = i1 - i0 + 1;
    for (int k0 = 0; k0 < nseg; k0 += kMergeChunk) {
        float lse[kMergeChunk], o[kMergeChunk][16];
#pragma unroll
        for (int c = 0; c < kMergeChunk; ++c) {
            const int k = k0 + c;               // wave-uniform
            lse[c] = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; ++v) o[c][v] = 0.f;
            if (k < nseg) {
                const float* seg =
                    a.part_o + (size_t)(k == 0 ? first : 2 * (i0 + k)) * kSegFloats;
                lse[c] = load_agent(seg + 16 * 64 + lane);
#pragma unroll
                for (int v = 0; v < 16; ++v) o[c][v] = load_agent(seg + v * 64 + lane);
            }
        }
#pragma unroll
        for (int c = 0; c < kMergeChunk; ++c) {
            if (lse[c] == -INFINITY) continue;  // not a segment, or an empty column
            const float M2 = fmaxf(M, lse[c]);
            const float r = __builtin_amdgcn_exp2f(M - M2);       // 0 while M = -inf
            const float w = __builtin_amdgcn_exp2f(lse[c] - M2);
#pragma unroll
            for (int v = 0; v < 16; ++v) num[v] = num[v] * r + w * o[c][v];
            den = den * r + w;
            M = M2;
        }
    }
    const Col c = column(a, lane);
    if (!c.ok) return;
    // the sink joins the denominator only
    const float sig = a.sinks ? a.sinks[g * a.G + c.h] * kLog2e : -INFINITY;
    const float M2 = fmaxf(M, sig);
    uint16_t* op = a.out + col_row(a, b, g, c) * kHeadDim + 4 * (lane >> 4);
    if (M2 == -INFINITY) {                      // nothing attended and no sink
        write_zero(a, b, g, lane);
        return;
    }
    const float r = __builtin_amdgcn_exp2f(M - M2);
    const float inv = 1.0f / (den * r + __builtin_amdgcn_exp2f(sig - M2));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x2_t ov = {pack_bf16(num[j * 4] * r * inv, num[j * 4 + 1] * r * inv),
                            pack_bf16(num[j * 4 + 2] * r * inv, num[j * 4 + 3] * r * inv)};
        *reinterpret_cast<u32x2_t*>(op + 16 * j) = ov;
    }
}

// Sequence b has nothing to attend: zero outputs, and (without FUSED) for
// each of its units a record (first slot in wavefront i, last wavefront i)
// that the combine kernel reads as "done".
template <bool FUSED>
__device__ __forceinline__ void finish_empty(const DecodeArgs& a, int b, int i, int lane) {
    for (int g = 0; g < a.Hkv; ++g) write_zero(a, b, g, lane);
    if (FUSED) return;
    // one record per KV head, however many heads there are (the workspace is
    // reused from call to call, so a record left out would be a stale one)
    for (int g = lane; g < a.Hkv; g += 64) {
        int* seg = a.unit_seg + 2 * (b * a.Hkv + g);
        seg[0] = 2 * i;
        seg[1] = i;
    }
}

// SA_STREAM_OCC > 0 asks the compiler for that many waves per SIMD.
#ifndef SA_STREAM_OCC
#define SA_STREAM_OCC 0
#endif

template <int BSL, bool ROPE, bool MULTI, bool FUSED>
__global__ __launch_bounds__(64)
#if SA_STREAM_OCC > 0
__attribute__((amdgpu_waves_per_eu(SA_STREAM_OCC, SA_STREAM_OCC)))
#endif
void decode_stream_kernel(const DecodeArgs a) {
    extern __shared__ int s_mem[];
    int* s_len = s_mem;            // seq_lens (n and the appended token's slot follow)
    int* s_end = s_mem + a.B;      // inclusive prefix of Hkv * steps, in steps
    const int lane = threadIdx.x;
    const int i = blockIdx.x;
    const int NW = a.num_waves;

    // per-sequence steps and their prefix sums
    int carry = 0;
    for (int base = 0; base < a.B; base += 64) {
        const int b = base + lane;
        const int L = b < a.B ? a.seq_lens[b] : 0;
        const int n = attended(a, L);
        int v = ((n + kStepTokens - 1) / kStepTokens) * a.Hkv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(v, off);
            if (lane >= off) v += t;
        }
        v += carry;
        if (b < a.B) {
            s_len[b] = L;
            s_end[b] = v;
        }
        carry = __shfl(v, 63);
    }
    __syncthreads();
    const long long T = carry;
    if (T == 0) {
        // nothing attended anywhere: every output is 0
        for (int bz = i; bz < a.B; bz += NW) finish_empty<FUSED>(a, bz, i, lane);
        return;
    }
    // the host launches this kernel only when sequences x KV heads x the
    // table's capacity in steps stays below 2^31, so the walk runs on 32-bit
    // wave-uniform values
    if (i == 0)                   // sequences before the first with a step
        for (int bz = 0; bz < a.B && s_end[bz] == 0; ++bz) finish_empty<FUSED>(a, bz, 0, lane);
    // The launch sizes NW from the table's capacity; with fewer steps than
    // that, only the first T wavefronts take part, so that every wavefront
    // in use holds at least one step and the wavefronts a unit spans are
    // consecutive ones that each left it a segment.
    const long long NWe = T < NW ? T : (long long)NW;
    if (i >= NWe) return;
    int x = (int)wave_start(i, T, NWe);
    const int x1 = (int)wave_start(i + 1, T, NWe);

    // sequence holding step x: the first b with s_end[b] > x
    int b;
    {
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_end[mid] > x) hi = mid; else lo = mid + 1;
        }
        b = __builtin_amdgcn_readfirstlane(lo);
    }
    int slot = 0;                 // 0: first unit of this wavefront, 1: last
    // (FUSED) segments stored in slot 0 / 1, whose arrivals are still to count
    int pend_b[2] = {0, 0}, pend_g[2] = {0, 0}, pend_start[2] = {0, 0}, pend_steps[2] = {1, 1};
    bool pend_on[2] = {false, false};
    while (x < x1) {
        const int L = __builtin_amdgcn_readfirstlane(s_len[b]);
        const int n = attended(a, L);
        const int steps = (n + kStepTokens - 1) / kStepTokens;
        const int end_b = __builtin_amdgcn_readfirstlane(s_end[b]);
        const int start_b = end_b - a.Hkv * steps;
        const int g = (x - start_b) / steps;
        const int ustart = start_b + g * steps;
        const int seg_end = min(x1, ustart + steps);
        const int s0 = x - ustart, s1 = seg_end - ustart;

        u32x4_t qop0, qop1;
        const int pos = ROPE ? rope_row(a, L) : 0;
        load_query<ROPE>(a, b, g, lane, qop0, qop1, pos);
        const Unit u = make_unit(a, b, g, lane, MULTI ? -1 : new_token_slot(a, L, n), pos, L);
        State st;
        st.reset();
        // one wavefront per SIMD: three steps in the register pipeline
        attend<BSL, ROPE, MULTI, 3>(a, u, s0 * kStepTokens, min(n, s1 * kStepTokens), qop0, qop1,
                                    st);
        const float l_tot = st.total();
        if (!FUSED && lane == 0) {
            int* seg = a.unit_seg + 2 * (b * a.Hkv + g);
            if (s0 == 0) seg[0] = 2 * i + slot;    // this wavefront's slot for the unit
            if (s1 == steps) seg[1] = i;
        }
        if (s0 == 0 && s1 == steps) {
            write_out(a, b, g, lane, st, l_tot);
        } else if (FUSED) {
            // a segment of a unit other wavefronts share: stored now, its
            // arrival counted once this wavefront's range is done (so the
            // stream never waits for the stores)
            store_segment(a.part_o + (size_t)(2 * i + slot) * kSegFloats, lane, st, l_tot);
            pend_b[slot] = b;
            pend_g[slot] = g;
            pend_start[slot] = ustart;
            pend_steps[slot] = steps;
            pend_on[slot] = true;
        } else {
            // partial slot: T*G rows, one per (query token, head) column
            const int ncol = a.T * a.G;
            const size_t sl = (size_t)(2 * i + slot) * ncol;
            write_partial((lane & 15) < ncol, lane & 15, lane, st, l_tot,
                          a.part_o + sl * kHeadDim, kHeadDim, a.part_lse + sl, 1);
        }
        slot = 1;
        x = seg_end;
        if (x >= end_b) {         // next sequence that has any step
            ++b;
            while (b < a.B && __builtin_amdgcn_readfirstlane(attended(a, s_len[b])) == 0) {
                finish_empty<FUSED>(a, b, i, lane);
                ++b;
            }
        }
    }
    if (!FUSED || !(pend_on[0] || pend_on[1])) return;
    // Count this wavefront's arrivals at the units it left segments of, once
    // every store of those segments is complete (agent-visible: they are
    // sc1); the wavefront that arrives last at a unit merges it.  Lanes 0 and
    // 1 count the two segments at once.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int old = -1;
    if (lane < 2 && pend_on[lane])
        old = __hip_atomic_fetch_add(a.counters + pend_b[lane] * a.Hkv + pend_g[lane], 1,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int old0 = __builtin_amdgcn_readlane(old, 0);
    const int old1 = __builtin_amdgcn_readlane(old, 1);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (!pend_on[p]) continue;
        const int us = pend_start[p];
        const int i0 = wave_of(us, T, NWe);
        const int i1 = wave_of(us + pend_steps[p] - 1, T, NWe);
        if ((p == 0 ? old0 : old1) != i1 - i0) continue;
        // the last to arrive: every segment's stores completed before its
        // arrival was counted.  The counter is this unit's alone until the
        // next call, which finds it at zero again.
        if (lane == 0)
            __hip_atomic_store(a.counters + pend_b[p] * a.Hkv + pend_g[p], 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        const int first = 2 * i0 + (wave_start(i0, T, NWe) == us ? 0 : 1);
        merge_unit(a, pend_b[p], pend_g[p], lane, i0, i1, first);
    }
}

// One workgroup per (b, h) of a unit spread over wavefronts i0 < i1: merge
// the partial slots those wavefronts left, with the sink.  Units done whole
// by one wavefront, and units with no step, were written by the partition
// kernel.  Two memory round trips: the unit's segment record, then its
// partials, CHUNK segments per wavefront at a time with every load issued
// before any is used (a chunk's loads sit under wave-uniform conditions with
// no wait between them, so a chunk is one round trip; past the last segment
// nothing is read and the weight is 0).  Chunks of 8: 16-wide chunks measured
// 0.4-1.3 us slower on batch-64 calls and 0.4 us on batch-1 and -8 calls.
constexpr int kCombineChunk = 8;
// segments per unit (if lengths were equal) up to which one wavefront merges
// a (b, h) row
constexpr int kOneWaveMergeSegs = 12;

template <int WAVES, int CHUNK>
__global__ __launch_bounds__(64 * WAVES) void combine_stream_kernel(const DecodeArgs a) {
    __shared__ float s_num[WAVES][64];
    __shared__ float s_den[WAVES];
    __shared__ float s_max[WAVES];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int bh = blockIdx.x;                  // out row (b*T + t)*Hq + h
    const int bt = bh / a.Hq;
    const int h = bh - bt * a.Hq;
    const int b = bt / a.T;
    const int tq = bt - b * a.T;
    const int g = h / a.G;
    const int hl = tq * a.G + (h - g * a.G);    // column of (tq, h) in a partial slot
    const int ncol = a.T * a.G;
    const int2 rec = *reinterpret_cast<const int2*>(a.unit_seg + 2 * (b * a.Hkv + g));
    // every unit's record is written by this call; the clamps only keep a
    // damaged one from reading past the partial slots
    const int first = min(max(rec.x, 0), 2 * a.num_waves - 1);
    const int i0 = first >> 1;
    const int i1 = min(max(rec.y, i0), a.num_waves - 1);
    if (i0 == i1) return;                         // written whole (or zero) by one wavefront
    const int nseg = i1 - i0 + 1;
    // segment k is wavefront i0 + k; its slot is `first` for k = 0, else 2*(i0+k)
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int k0 = w * CHUNK; k0 < nseg; k0 += WAVES * CHUNK) {
        float l[CHUNK], o[CHUNK];
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            const int k = k0 + j;
            l[j] = -INFINITY;
            o[j] = 0.f;
            if (k < nseg) {           // wave-uniform; the loads still all go out first
                const size_t sl = (size_t)(k == 0 ? first : 2 * (i0 + k)) * ncol + hl;
                l[j] = a.part_lse[sl];
                o[j] = a.part_o[sl * kHeadDim + lane];
            }
        }
        float M2 = M;
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) M2 = fmaxf(M2, k0 + j < nseg ? l[j] : -INFINITY);
        // no segment with a slot for this column yet (several query tokens:
        // segments before a token's position are empty): nothing to add
        if (M2 == -INFINITY) continue;
        const float r = __builtin_amdgcn_exp2f((M - M2) * kLog2e);   // 0 while M = -inf
        float cn = 0.f, cd = 0.f;
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            const float wt = k0 + j < nseg ? __builtin_amdgcn_exp2f((l[j] - M2) * kLog2e) : 0.f;
            cn += wt * o[j];
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
        for (int j = 0; j < WAVES; ++j) M = fmaxf(M, s_max[j]);
        num = 0.f;
        den = 0.f;
#pragma unroll
        for (int j = 0; j < WAVES; ++j) {
            if (s_max[j] == -INFINITY) continue;  // a wavefront with no segment
            const float r = __builtin_amdgcn_exp2f((s_max[j] - M) * kLog2e);
            num += s_num[j][lane] * r;
            den += s_den[j] * r;
        }
    }
    // the sink joins the denominator only
    const float sig = a.sinks ? a.sinks[h] : -INFINITY;
    const float M2 = fmaxf(M, sig);
    const float r = __builtin_amdgcn_exp2f((M - M2) * kLog2e);
    den = den * r + __builtin_amdgcn_exp2f((sig - M2) * kLog2e);
    const __bf16 o = (__bf16)(num * r / den);
    a.out[(size_t)bh * kHeadDim + lane] = __builtin_bit_cast(uint16_t, o);
}

template <bool ROPE, bool MULTI, bool FUSED>
hipError_t launch_stream_partitions(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)2 * a.B * sizeof(int);
    const dim3 grid(a.num_waves);
    switch (a.bs_log2) {
        case 3: return launch(decode_stream_kernel<3, ROPE, MULTI, FUSED>, grid, dim3(64), lds, stream, a);
        case 4: return launch(decode_stream_kernel<4, ROPE, MULTI, FUSED>, grid, dim3(64), lds, stream, a);
        case 5: return launch(decode_stream_kernel<5, ROPE, MULTI, FUSED>, grid, dim3(64), lds, stream, a);
        case 6: return launch(decode_stream_kernel<6, ROPE, MULTI, FUSED>, grid, dim3(64), lds, stream, a);
        default: return hipErrorInvalidValue;
    }
}

template <bool FUSED>
hipError_t launch_stream_variant(const DecodeArgs& a, bool rope, hipStream_t stream) {
    return a.T > 1 ? (rope ? hipErrorInvalidValue
                           : launch_stream_partitions<false, true, FUSED>(a, stream))
           : rope ? launch_stream_partitions<true, false, FUSED>(a, stream)
                  : launch_stream_partitions<false, false, FUSED>(a, stream);
}

}  // namespace

hipError_t launch_decode_stream(const DecodeArgs& a, bool rope, bool fused_merge,
                                hipStream_t stream) {
    if (fused_merge) return launch_stream_variant<true>(a, rope, stream);
    hipError_t e = launch_stream_variant<false>(a, rope, stream);
    if (e != hipSuccess) return e;
    // segments per unit if lengths were equal; picks the combine's width
    const long long units = (long long)a.B * a.Hkv;
    const long long per_unit = (a.num_waves + units - 1) / units + 1;
    const dim3 cgrid((unsigned)a.B * a.T * a.Hq);
    if (per_unit <= kOneWaveMergeSegs)
        return launch(combine_stream_kernel<1, kCombineChunk>, cgrid, dim3(64), 0, stream, a);
    else if (per_unit <= 64)
        return launch(combine_stream_kernel<4, kCombineChunk>, cgrid, dim3(256), 0, stream, a);
    else
        return launch(combine_stream_kernel<16, kCombineChunk>, cgrid, dim3(1024), 0, stream, a);
}

}  // namespace sa
