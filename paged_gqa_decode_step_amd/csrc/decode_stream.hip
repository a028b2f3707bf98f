// Decode attention with balanced work: every wavefront gets the same number
// of 32-slot steps, whatever the mix of context lengths in the batch.
//
// The n_b attended slots of sequence b (n = L for a paged layer, min(L, W)
// for a ring) make ceil(n_b / 32) steps for each of its Hkv units
// (b, g).  Laying the units out one after another gives T steps in all;
// wavefront i of NW takes steps [i*T/NW, (i+1)*T/NW) and walks them unit by
// unit.  A unit it covers whole gets its bf16 output (with the sink)
// directly; a unit it covers in part leaves a partial (o, lse), which only
// its first and last unit can need, so each wavefront owns two partial slots.
// combine_stream_kernel then merges, for each unit spread over wavefronts
// i0..i1, the slots those wavefronts left (the log-sum-exp merge of the
// flash-decoding split; the tutorial setup page's FlashAttention chapter
// names the online softmax it rests on).
//
// Every wavefront derives T and the unit layout itself from seq_lens (an
// inclusive scan in LDS), so there is no planning launch; wavefront 0 also
// stores the per-sequence step prefix for the combine kernel.  The per-step
// MFMA machinery is mfma_attend.h.
#include "mfma_attend.h"

namespace sa {
namespace {

using namespace mfma;

__device__ __forceinline__ int attended(const DecodeArgs& a, int L) {
    int n = a.window > 0 ? min(L, a.window) : L;
    return max(0, min(n, a.mbs << a.bs_log2));
}

// first step of wavefront i, and the wavefront holding step x (T > 0)
__device__ __forceinline__ long long wave_start(long long i, long long T, long long NW) {
    return i * T / NW;
}
__device__ __forceinline__ long long wave_of(long long x, long long T, long long NW) {
    return ((x + 1) * NW - 1) / T;
}

// SA_STREAM_OCC > 0 asks the compiler for that many waves per SIMD.
#ifndef SA_STREAM_OCC
#define SA_STREAM_OCC 0
#endif

template <int BSL>
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
            if (i == 0) a.plan[b] = v;
        }
        carry = __shfl(v, 63);
    }
    __syncthreads();
    const long long T = carry;
    if (T == 0) {
        // nothing attended anywhere: every output is 0
        for (int u = i; u < a.B * a.Hkv; u += NW) write_zero(a, u / a.Hkv, u % a.Hkv, lane);
        return;
    }
    // step counts stay below 2^31 (sequences x KV heads x 2^26 slots / 32),
    // so the walk runs on 32-bit wave-uniform values
    int x = (int)wave_start(i, T, NW);
    const int x1 = (int)wave_start(i + 1, T, NW);
    if (x >= x1) return;

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
        load_query(a, b, g, lane, qop0, qop1);
        const Unit u = make_unit(a, b, g, lane, new_token_slot(a, L, n));
        State st;
        st.reset();
        attend<BSL>(u, s0 * kStepTokens, min(n, s1 * kStepTokens), qop0, qop1, st);
        const float l_tot = st.total();
        if (s0 == 0 && s1 == steps) {
            write_out(a, b, g, lane, st, l_tot);
        } else {
            const size_t sl = (size_t)(2 * i + slot) * a.G;
            write_partial(a.G, lane, st, l_tot, a.part_o + sl * kHeadDim, kHeadDim,
                          a.part_lse + sl, 1);
        }
        slot = 1;
        x = seg_end;
        if (x >= end_b) {         // next sequence that has any step
            ++b;
            while (b < a.B && __builtin_amdgcn_readfirstlane(attended(a, s_len[b])) == 0) ++b;
        }
    }
}

// One workgroup per (b, h) of a unit spread over wavefronts i0 < i1: merge
// the partial slots those wavefronts left, with the sink.  Units done whole
// by one wavefront were written by the partition kernel; units with no step
// get 0 here.  Each wavefront merges its share of the segments with a
// running maximum, so all of a segment's loads (lse and o row) can be in
// flight at once: two memory round trips in all (plan, then partials).
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void combine_stream_kernel(const DecodeArgs a) {
    __shared__ float s_num[WAVES][64];
    __shared__ float s_den[WAVES];
    __shared__ float s_max[WAVES];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int bh = blockIdx.x;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int g = h / a.G;
    const int hl = h - g * a.G;
    const long long T = a.plan[a.B - 1];
    const long long end_b = a.plan[b];
    const long long prev = b > 0 ? a.plan[b - 1] : 0;
    const int steps = (int)((end_b - prev) / a.Hkv);
    uint16_t* op = a.out + (size_t)bh * kHeadDim + lane;
    if (steps == 0) {
        if (w == 0) *op = 0;
        return;
    }
    const long long NW = a.num_waves;
    const long long us = prev + (long long)g * steps;
    const long long i0 = wave_of(us, T, NW);
    const long long i1 = wave_of(us + steps - 1, T, NW);
    if (i0 == i1) return;                         // written whole by one wavefront
    const int first_slot = wave_start(i0, T, NW) == us ? 0 : 1;
    const int nseg = (int)(i1 - i0 + 1);
    // segment k is wavefront i0 + k; its slot is 2*(i0+k) + (k == 0 ? first_slot : 0)
    float M = -INFINITY, num = 0.f, den = 0.f;
#pragma unroll 8
    for (int k = w; k < nseg; k += WAVES) {
        const size_t sl = (size_t)(2 * (i0 + k) + (k == 0 ? first_slot : 0)) * a.G + hl;
        const float l = a.part_lse[sl];
        const float o = a.part_o[sl * kHeadDim + lane];
        const float M2 = fmaxf(M, l);
        const float r = __builtin_amdgcn_exp2f((M - M2) * kLog2e);   // 0 while M = -inf
        const float wt = __builtin_amdgcn_exp2f((l - M2) * kLog2e);
        num = num * r + wt * o;
        den = den * r + wt;
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
    *op = __builtin_bit_cast(uint16_t, o);
}

}  // namespace

hipError_t launch_decode_stream(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)2 * a.B * sizeof(int);
    const dim3 grid(a.num_waves);
    switch (a.bs_log2) {
        case 3: hipLaunchKernelGGL(decode_stream_kernel<3>, grid, dim3(64), lds, stream, a); break;
        case 4: hipLaunchKernelGGL(decode_stream_kernel<4>, grid, dim3(64), lds, stream, a); break;
        case 5: hipLaunchKernelGGL(decode_stream_kernel<5>, grid, dim3(64), lds, stream, a); break;
        case 6: hipLaunchKernelGGL(decode_stream_kernel<6>, grid, dim3(64), lds, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // segments per unit if lengths were equal; picks the combine's width
    const long long units = (long long)a.B * a.Hkv;
    const long long per_unit = (a.num_waves + units - 1) / units + 1;
    const dim3 cgrid((unsigned)a.B * a.Hq);
    if (per_unit <= 8)
        hipLaunchKernelGGL(combine_stream_kernel<1>, cgrid, dim3(64), 0, stream, a);
    else if (per_unit <= 64)
        hipLaunchKernelGGL(combine_stream_kernel<4>, cgrid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(combine_stream_kernel<16>, cgrid, dim3(1024), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
