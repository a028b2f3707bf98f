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
// inclusive scan in LDS), so there is no planning launch.  The wavefronts
// holding a unit's first and last steps record, for the combine kernel, the
// unit's first partial slot and its last wavefront.  The per-step MFMA
// machinery is mfma_attend.h.
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

// Sequence b has nothing to attend: zero outputs, and for each of its units a
// record (first slot in wavefront i, last wavefront i) that the combine
// kernel reads as "done".
__device__ __forceinline__ void finish_empty(const DecodeArgs& a, int b, int i, int lane) {
    for (int g = 0; g < a.Hkv; ++g) write_zero(a, b, g, lane);
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

template <int BSL, bool ROPE, bool MULTI>
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
        for (int bz = i; bz < a.B; bz += NW) finish_empty(a, bz, i, lane);
        return;
    }
    // the host launches this kernel only when sequences x KV heads x the
    // table's capacity in steps stays below 2^31, so the walk runs on 32-bit
    // wave-uniform values
    if (i == 0)                   // sequences before the first with a step
        for (int bz = 0; bz < a.B && s_end[bz] == 0; ++bz) finish_empty(a, bz, 0, lane);
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
        if (lane == 0) {
            int* seg = a.unit_seg + 2 * (b * a.Hkv + g);
            if (s0 == 0) seg[0] = 2 * i + slot;    // this wavefront's slot for the unit
            if (s1 == steps) seg[1] = i;
        }
        if (s0 == 0 && s1 == steps) {
            write_out(a, b, g, lane, st, l_tot);
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
                finish_empty(a, b, i, lane);
                ++b;
            }
        }
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

template <bool ROPE, bool MULTI>
hipError_t launch_stream_partitions(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)2 * a.B * sizeof(int);
    const dim3 grid(a.num_waves);
    switch (a.bs_log2) {
        case 3: return launch(decode_stream_kernel<3, ROPE, MULTI>, grid, dim3(64), lds, stream, a);
        case 4: return launch(decode_stream_kernel<4, ROPE, MULTI>, grid, dim3(64), lds, stream, a);
        case 5: return launch(decode_stream_kernel<5, ROPE, MULTI>, grid, dim3(64), lds, stream, a);
        case 6: return launch(decode_stream_kernel<6, ROPE, MULTI>, grid, dim3(64), lds, stream, a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_stream(const DecodeArgs& a, bool rope, hipStream_t stream) {
    hipError_t e = a.T > 1 ? (rope ? hipErrorInvalidValue
                                   : launch_stream_partitions<false, true>(a, stream))
                 : rope ? launch_stream_partitions<true, false>(a, stream)
                        : launch_stream_partitions<false, false>(a, stream);
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
