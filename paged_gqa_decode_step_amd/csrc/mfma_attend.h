// The inner loop of decode attention on MFMA, shared by the partition kernels.
//
// What is computed (SimpleLLM README, optimisation table: one decode-attention
// kernel for sinks, sliding window and GQA over the paged cache / ring
// buffer; tutorial setup page, PagedAttention and FlashAttention chapters):
// for query head h of KV group g, scores s_p = q_h . K_p / sqrt(D) over a run
// of slots, an online softmax over them, and sum_p e^(s_p-m) V_p.  The
// per-head sink logit enters only the final normaliser (no value row), which
// the callers apply.
//
// One 64-lane wavefront serves all G <= 16 query heads of a KV group from one
// read of each K/V tile: the group's queries form the 16-column operand of
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
//     32+8*q4..+7 (kstep 1) of its K row / of its query head; the K pool keeps
//     each half of a row (32 dims, 64 bytes) slot-major in its own half of the
//     block ([2][bs][32]), so a K load covers 4 runs of 4 consecutive slots'
//     64-byte halves, i.e. 8 whole cache lines;
//   * M-tile m row r holds slot base + 8*(r/4) + 4*m + r%4, so the S^T output
//     lane (head c16, q4) ends up with the scores of slots base+8*q4 .. +7;
//   * PV reduces over slots: that same lane feeds those eight probabilities
//     as its P^T column, and the V^T operand lane (dim row c16, q4) needs
//     V[dim][base+8*q4 .. +7], i.e. 16 contiguous bytes of the V pool, which
//     is transposed inside a block in chunks of 8 slots ([bs/8][D][8]).
// No LDS, no barriers: cross-lane reductions of the softmax max/sum over the
// four q4 groups use v_permlane16_swap / v_permlane32_swap.
//
// Masking: only the last step of a run can reach past its end t1.  Chunks of
// 8 slots that start at or past t1 are redirected to the chunk holding t1-1
// (an allocated block) for their loads; their scores become -inf and the V
// elements of slots >= t1 are zeroed, so stale or NaN data in a block tail
// can never reach the output.
#pragma once

#include <math.h>

#include "sa_internal.h"

// Build-time tuning knob (the default is the measured best on MI355X):
//   SA_KV_NT  1: K/V loads carry the non-temporal hint.  The K/V stream is
//             read once per call, so keeping it out of the caches leaves them
//             to the block table, queries and partials (measured +4-7% on
//             calls that do not fit the 256 MB Infinity Cache).
#ifndef SA_KV_NT
#define SA_KV_NT 1
#endif

namespace sa {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// How far (log2 units) a head's running max may rise above the reference max
// of the online softmax before the state is rescaled: probabilities stay below
// 2^8, far inside the range of the fp32 sums and of the bf16 P operand.
constexpr float kRescaleSlack = 8.0f;

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

// bf16 halves of a 32-bit word, widened exactly
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// Rotary embedding of one pair (x1, x2) by the angle with cosine c and sine s:
// (x1 c - x2 s, x2 c + x1 s), each product and each sum rounded to float32 on
// its own (no fused multiply-add), so the bf16 rounding that follows takes
// the same decision wherever it is computed.
__device__ __forceinline__ float rot_first(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
    return x1 * c - x2 * s;
}
__device__ __forceinline__ float rot_second(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
    return x2 * c + x1 * s;
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t load16(const char* p) {
#if SA_KV_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#else
    return *reinterpret_cast<const u32x4_t*>(p);
#endif
}

// K pool layout inside a (block, KV head): [2][bs][32], the row of a slot cut
// into two halves of 32 dimensions, each half slot-major.  An operand load
// instruction (16 slots x 32 dimensions) then reads whole cache lines; with
// plain rows ([bs][D]) it read half of 16 lines, which measured about 2% slower
// on long contexts.  Word w (dimensions 2w, 2w+1) of slot s's row is at byte
// k_word_offset(s, w).
template <int BS>
__device__ __forceinline__ unsigned k_word_offset(unsigned slot_in_block, unsigned w) {
    return ((w >> 4) * BS + slot_in_block) * 64 + (w & 15) * 4;
}

// V pool layout inside a (block, KV head): [bs/8][D][8], i.e. V transposed in
// chunks of 8 slots.  A chunk is D rows of 16 bytes (one dimension's 8 slots),
// so the PV operand (8 slots of one dimension) is one 16-byte load, and a
// token's column (one element in each of the 64 rows) spans 8 cache lines.
constexpr unsigned kVChunkBytes = kHeadDim * 8 * 2;
__device__ __forceinline__ unsigned v_elem_offset(unsigned slot_in_block, unsigned dim) {
    return ((slot_in_block >> 3) * kHeadDim + dim) * 16 + (slot_in_block & 7) * 2;
}

struct StepRegs {
    u32x4_t k[4];   // [m*2 + kstep]
    u32x4_t v[4];   // dim tile j
};

// Pipeline depth that issues every step of a short run at once (attend_run).
constexpr int kBurst = kBurstSteps;

// Online-softmax state of one wavefront: acc[j] lane (head c16, q4) holds dims
// 16j + 4*q4 .. +3 of that head; m is the reference max of the exponents
// (log2 domain, equal on the head's four lanes; at most kRescaleSlack below the
// running max); l is this lane's share of the running sum.
struct State {
    f32x4_t acc[4];
    float m;
    float l;
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
    }
    // sum of l over the head's four lanes
    __device__ __forceinline__ float total() const { return sum_xor32(sum_xor16(l)); }
};

// Where one (sequence, KV head) lives, and the lane's fixed offsets.  The
// block size is a template parameter (bs = 2^BSL) of the functions below so
// every in-block offset is an immediate of its load.
struct Unit {
    const char* kbase;       // K pool + g * (bs*D*2)
    const char* vbase;       // V pool + g * (bs*D*2)
    // the token appended by this launch: its slot (-1: none), its K and V rows
    // (k_new / v_new of this unit; q when nothing is appended, so that the
    // rows can be read unconditionally) and where the pools are written
    int new_slot;
    int rope_pos;            // position of the new token in the rotary tables
    int L, T, G;             // sequence length; query tokens (new slots L-T..L-1); heads
    bool appends;            // the launch appends (k_new given)
    const uint16_t* kn_row;  // token 0's rows; token t's are kn_stride elements further
    const uint16_t* vn_row;
    int kn_stride;
    char* kstore;            // writable K pool + g * (bs*D*2)
    char* vstore;
    const int32_t* bt_row;   // block table row of the sequence
    unsigned blk_stride;     // bytes per block across all KV heads
    unsigned k_lane;         // (c16 & 3) slots + 8*q4 dims of a half row, bytes
    unsigned v_lane;         // c16 dim rows of a chunk, bytes
    int bs_log2;
    int num_blocks;
    int mbs;                 // entries in a block-table row
    int c16, q4;
    float scale_log2;
};

// Slot of the token this launch appends for a sequence of length L with n
// attended slots (-1 when the launch appends nothing or the slot is past the
// table's capacity, where the separate append skips it too).
__device__ __forceinline__ int new_token_slot(const DecodeArgs& a, int L, int n) {
    if (!a.k_new || L <= 0) return -1;
    const int slot = a.window > 0 ? (L - 1) % a.window : L - 1;
    return slot < n ? slot : -1;
}

__device__ __forceinline__ Unit make_unit(const DecodeArgs& a, int b, int g, int lane,
                                          int new_slot = -1, int rope_pos = 0, int L = 0) {
    Unit u;
    const int bs = 1 << a.bs_log2;
    u.c16 = lane & 15;
    u.q4 = lane >> 4;
    u.bs_log2 = a.bs_log2;    // == BSL of the kernel instantiation
    u.num_blocks = a.num_blocks;
    u.mbs = a.mbs;
    u.blk_stride = (unsigned)(a.Hkv * bs * kHeadDim * 2);
    u.kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)g * bs * kHeadDim * 2;
    u.vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)g * bs * kHeadDim * 2;
    u.bt_row = a.block_table + (size_t)b * a.mbs;
    u.k_lane = (unsigned)((u.c16 & 3) * 32 + 8 * u.q4) * 2;
    u.v_lane = (unsigned)u.c16 * 16;   // dim row c16 of an 8-slot chunk, bytes
    u.scale_log2 = a.scale_log2;
    u.new_slot = new_slot;
    u.rope_pos = rope_pos;
    u.L = L;
    u.T = a.T;
    u.G = a.G;
    u.kn_stride = a.Hkv * kHeadDim;
    u.appends = a.k_new != nullptr;
    const size_t row = ((size_t)b * a.T * a.Hkv + g) * kHeadDim;
    u.kn_row = a.k_new ? a.k_new + row : a.q;
    u.vn_row = a.k_new ? a.v_new + row : a.q;
    u.kstore = reinterpret_cast<char*>(a.k_store) + (size_t)g * bs * kHeadDim * 2;
    u.vstore = reinterpret_cast<char*>(a.v_store) + (size_t)g * bs * kHeadDim * 2;
    return u;
}

// Query operand of head g*G + c16 (zero for c16 >= G): dims 8*q4..+7 and
// 32+8*q4..+7.
// The query column of a lane: c16 = t*G + h is query token t, head g*G + h of
// the unit (one token: t = 0, h = c16); columns past T*G are idle.
struct Col {
    bool ok;
    int t, h;
};
__device__ __forceinline__ Col column(const DecodeArgs& a, int lane) {
    const int c16 = lane & 15;
    Col c;
    c.t = c16 / a.G;
    c.h = c16 - c.t * a.G;
    c.ok = c.t < a.T;
    return c;
}
// q / out row of a column of unit (b, g)
__device__ __forceinline__ size_t col_row(const DecodeArgs& a, int b, int g, const Col& c) {
    return ((size_t)b * a.T + c.t) * a.Hq + g * a.G + c.h;
}

// Row of the rotary tables for a sequence of length L (> 0): position L-1,
// past the tables' last row their last row.
__device__ __forceinline__ int rope_row(const DecodeArgs& a, int L) {
    return min(L - 1, a.rope_max_pos - 1);
}

// The query operands of a unit: lane (c16, q4) holds head g*G + c16, dims
// 8q4..8q4+7 (qop0) and 32+8q4..32+8q4+7 (qop1); zero for c16 >= G.  With
// ROPE they are rotated at table row `pos`.  Both pairings keep each pair
// inside one lane: "half" pairs dim i with i+32, i.e. element e of qop0 with
// element e of qop1; "interleaved" pairs the two halves of each 32-bit word.
template <bool ROPE>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int b, int g, int lane,
                                           u32x4_t& qop0, u32x4_t& qop1, int pos = 0) {
    const int q4 = lane >> 4;
    qop0 = u32x4_t{0u, 0u, 0u, 0u};
    qop1 = u32x4_t{0u, 0u, 0u, 0u};
    const Col c = column(a, lane);
    if (c.ok) {
        const uint16_t* qp = a.q + col_row(a, b, g, c) * kHeadDim + 8 * q4;
        qop0 = *reinterpret_cast<const u32x4_t*>(qp);
        qop1 = *reinterpret_cast<const u32x4_t*>(qp + 32);
    }
    if (!ROPE) return;
    const float* cr = a.rope_cos + (size_t)pos * (kHeadDim / 2);
    const float* sr = a.rope_sin + (size_t)pos * (kHeadDim / 2);
    if (a.rope_style == kRopeHalf) {
        // pair i = 8q4 + e: x1 = element e of qop0, x2 = element e of qop1
        const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cr + 8 * q4);
        const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(cr + 8 * q4 + 4);
        const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sr + 8 * q4);
        const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(sr + 8 * q4 + 4);
        const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a1 = bf16_lo(qop0[w]), b1 = bf16_hi(qop0[w]);   // x1 of pairs 2w, 2w+1
            const float a2 = bf16_lo(qop1[w]), b2 = bf16_hi(qop1[w]);   // their x2
            qop0[w] = pack_bf16(rot_first(a1, a2, c[2 * w], sn[2 * w]),
                                rot_first(b1, b2, c[2 * w + 1], sn[2 * w + 1]));
            qop1[w] = pack_bf16(rot_second(a1, a2, c[2 * w], sn[2 * w]),
                                rot_second(b1, b2, c[2 * w + 1], sn[2 * w + 1]));
        }
    } else {
        // pair i = 4q4 + w (qop0 word w) and 16 + 4q4 + w (qop1 word w)
        const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cr + 4 * q4);
        const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(cr + 16 + 4 * q4);
        const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sr + 4 * q4);
        const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(sr + 16 + 4 * q4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float x1 = bf16_lo(qop0[w]), x2 = bf16_hi(qop0[w]);
            qop0[w] = pack_bf16(rot_first(x1, x2, c0[w], s0[w]), rot_second(x1, x2, c0[w], s0[w]));
            const float y1 = bf16_lo(qop1[w]), y2 = bf16_hi(qop1[w]);
            qop1[w] = pack_bf16(rot_first(y1, y2, c1[w], s1[w]), rot_second(y1, y2, c1[w], s1[w]));
        }
    }
}

// Block-table entries blk0 + lane of a unit, one per lane, clamped into the
// pool for the reads (lanes past the row's end repeat its last entry; they
// are never used), and whether the entry was inside the pool, which the
// append's stores require: an entry outside it is a caller error that the
// reads survive by the clamp and the append skips.  No branch around the
// load, so it is in flight with whatever precedes it.
struct TableSlice {
    int blk;
    int ok;
};
__device__ __forceinline__ TableSlice table_slice(const Unit& u, int blk0, int lane) {
    const int e = u.bt_row[min(blk0 + lane, u.mbs - 1)];
    return TableSlice{min(max(e, 0), u.num_blocks - 1), (e >= 0 && e < u.num_blocks) ? 1 : 0};
}

// Attend over slots [t0, t1) of one unit (t0 a multiple of 32, t1 > t0, and
// the run spanning at most kMaxTableSlice blocks, whose table entries tbl
// holds, with tbl_ok their validity for the append), folding into st.  kword / vval: this lane's word (lane & 31) of the
// new token's K row and its element `lane` of the V row.
template <int BSL, bool ROPE, bool MULTI, int DEPTH>
__device__ __forceinline__ void attend_run(const Unit& u, int t0, int t1, int tbl, int tbl_ok,
                                           unsigned kword, uint16_t vval, float2 kcos,
                                           float2 ksin, int rope_style, u32x4_t qop0,
                                           u32x4_t qop1, State& st) {
    const int c16 = u.c16, q4 = u.q4;
    constexpr int bs = 1 << BSL;
    const int blk0 = t0 >> BSL;
    const int last_chunk = (t1 - 1) & ~7;
    const int nsteps = (t1 - t0 + kStepTokens - 1) / kStepTokens;
    const bool has_new = !MULTI && u.new_slot >= t0 && u.new_slot < t1;   // wave-uniform
    // several query tokens: token t of a column sees slots below L - T + t + 1
    const int col_lim = MULTI ? min(t1, u.L - u.T + c16 / u.G + 1) : t1;
    // block of the new slot (any lane when there is none: bpermute wraps),
    // outside the branch so the table wait is not merged into the join below
    const unsigned nblk_id =
        (unsigned)__builtin_amdgcn_ds_bpermute(((u.new_slot >> BSL) - blk0) << 2, tbl);
    const int nblk_ok = __builtin_amdgcn_ds_bpermute(((u.new_slot >> BSL) - blk0) << 2, tbl_ok);

    // the 8 loads of step s (K: 2 M-tiles x 2 k-steps; V: 4 dim tiles)
    auto load_step = [&](int s, StepRegs& r) {
        const int base = t0 + (s << 5);
        int kc = base + ((c16 >> 2) << 3);           // 8-slot chunk of this lane's K rows
        int vc = base + (q4 << 3);                   // 8-slot chunk of this lane's V^T run
        kc = kc < t1 ? kc : last_chunk;
        vc = vc < t1 ? vc : last_chunk;
        const unsigned kblk =
            (unsigned)__builtin_amdgcn_ds_bpermute(((kc >> BSL) - blk0) << 2, tbl);
        const unsigned vblk =
            (unsigned)__builtin_amdgcn_ds_bpermute(((vc >> BSL) - blk0) << 2, tbl);
        const char* kp = u.kbase + (size_t)kblk * u.blk_stride +
                         ((unsigned)(kc & (bs - 1)) * 64 + u.k_lane);
        const char* vp = u.vbase + (size_t)vblk * u.blk_stride +
                         ((unsigned)((vc & (bs - 1)) >> 3) * kVChunkBytes + u.v_lane);
        r.k[0] = load16(kp);                      // M-tile 0, dims 0..31
        r.k[1] = load16(kp + bs * 64);            // M-tile 0, dims 32..63
        r.k[2] = load16(kp + 4 * 64);             // M-tile 1 (4 slots on)
        r.k[3] = load16(kp + 4 * 64 + bs * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) r.v[j] = load16(vp + (size_t)j * 16 * 16);
    };

    auto compute_step = [&](int s, StepRegs& r) {
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        s0 = mfma(r.k[0], qop0, s0);
        s0 = mfma(r.k[1], qop1, s0);
        s1 = mfma(r.k[2], qop0, s1);
        s1 = mfma(r.k[3], qop1, s1);
        float t[8];          // q.k; the scale joins in the exponent's fused multiply-add
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t[i] = s0[i];
            t[4 + i] = s1[i];
        }
        const int tok = t0 + (s << 5) + (q4 << 3);   // slot of t[0] on this lane
        if (MULTI && tok + 8 > col_lim) {             // the column's causal limit
            const int valid = max(0, min(8, col_lim - tok));
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e >= valid) t[e] = -INFINITY;
        }
        if (tok + 8 > t1) {                           // only in a run's last step
            const int valid = max(0, min(8, t1 - tok));
            if (!MULTI) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (e >= valid) t[e] = -INFINITY;
            }
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
        mx = max_xor32(max_xor16(mx)) * u.scale_log2;   // the scale is positive
        // The reference max st.m moves, and the state is rescaled, only when
        // some head's max rises more than kRescaleSlack above it; otherwise
        // the probabilities stay below 2^kRescaleSlack and most steps skip the
        // rescale (a wave-uniform branch).  A fresh state (m = -inf) takes the
        // first live step's max; a wholly masked step on a fresh state keeps
        // m = -inf and its probabilities are exp2(-inf) = 0.
        if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleSlack) != 0) {
            const float m_new = fmaxf(st.m, mx);
            const float alpha =
                __builtin_amdgcn_exp2f(st.m - (m_new == -INFINITY ? 0.f : m_new));
            st.l *= alpha;
#pragma unroll
            for (int j = 0; j < 4; ++j) st.acc[j] *= alpha;
            st.m = m_new;
        }
        const float m_ref = st.m == -INFINITY ? 0.f : st.m;
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(t[e], u.scale_log2, -m_ref));
            psum += p[e];
        }
        st.l += psum;
        const u32x4_t pop = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                             pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
#pragma unroll
        for (int j = 0; j < 4; ++j) st.acc[j] = mfma(r.v[j], pop, st.acc[j]);
    };

    // The append (the fused form of the KV append): the one run that holds
    // the new token's slot stores its K row and V column into the pools
    // before it issues the loads of the step holding that slot.  A
    // wavefront's memory operations to one address complete in program order
    // (and the compiler keeps the order: the pools are read and written
    // through pointers that may alias), so this run's loads of the slot
    // return the new row.  No other wavefront of this launch reads the slot.
    // When the slot is past the first step, the store goes after the first
    // step's loads (step 1 onwards is loaded later), so any wait on the store
    // overlaps with those loads.  (The V column is one 2-byte element in each
    // of 64 dim rows, 8 cache lines in the chunked layout; its cost grows with
    // the lines it dirties, and no later placement of the store measured
    // faster.)
    auto store_new = [&]() {
        const int lane = c16 + 16 * q4;
        const unsigned noff = (unsigned)(u.new_slot & (bs - 1));
        const size_t blk_off = (size_t)nblk_id * u.blk_stride;
        unsigned kw = kword;
        if (ROPE) {
            // the new key rotated at its position: word (lane & 31) holds dims
            // 2w, 2w+1; with "half" pairing their partners are word w ^ 16
            const unsigned other =
                (unsigned)__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, (int)kword);
            const float lo = bf16_lo(kword), hi = bf16_hi(kword);
            if (rope_style == kRopeHalf) {
                const float plo = bf16_lo(other), phi = bf16_hi(other);
                kw = (lane & 16) == 0
                         ? pack_bf16(rot_first(lo, plo, kcos.x, ksin.x),
                                     rot_first(hi, phi, kcos.y, ksin.y))
                         : pack_bf16(rot_second(plo, lo, kcos.x, ksin.x),
                                     rot_second(phi, hi, kcos.y, ksin.y));
            } else {
                kw = pack_bf16(rot_first(lo, hi, kcos.x, ksin.x), rot_second(lo, hi, kcos.x, ksin.x));
            }
        }
        // V column: lane = dim.  K row: word (lane & 31) of the row (the
        // upper half-wave stores the same words again).
        *reinterpret_cast<uint16_t*>(u.vstore + blk_off + v_elem_offset(noff, lane)) = vval;
        *reinterpret_cast<unsigned*>(u.kstore + blk_off + k_word_offset<bs>(noff, lane & 31)) =
            kw;
    };
    // the new slot's table entry outside the pool: no append (the reads
    // of the slot see the clamped block's contents, as for every slot)
    const bool stores_new = has_new && nblk_ok;                  // wave-uniform
    const bool new_first = stores_new && u.new_slot < t0 + kStepTokens;
    if (new_first) store_new();
    if (MULTI && u.appends && u.L - 1 >= t0 && u.L - u.T < t1) {
        // every new token whose slot lies in this run, before any load.  The
        // words of up to kAppendGroup tokens are read together (unconditional
        // loads: past the last token they re-read it), so a group costs one
        // round trip, not one per token.
        constexpr int kAppendGroup = 4;
        const int lane = c16 + 16 * q4;
        for (int tg = 0; tg < u.T; tg += kAppendGroup) {
            unsigned kws[kAppendGroup];
            uint16_t vvs[kAppendGroup];
#pragma unroll
            for (int j = 0; j < kAppendGroup; ++j) {
                const size_t row = (size_t)min(tg + j, u.T - 1) * u.kn_stride;
                kws[j] = reinterpret_cast<const unsigned*>(u.kn_row + row)[lane & 31];
                vvs[j] = (u.vn_row + row)[lane];
            }
#pragma unroll
            for (int j = 0; j < kAppendGroup; ++j) {
                const int slot = u.L - u.T + tg + j;         // wave-uniform
                if (tg + j >= u.T || slot < t0 || slot >= t1) continue;
                const unsigned nb =
                    (unsigned)__builtin_amdgcn_ds_bpermute(((slot >> BSL) - blk0) << 2, tbl);
                if (!__builtin_amdgcn_ds_bpermute(((slot >> BSL) - blk0) << 2, tbl_ok)) continue;
                const unsigned noff = (unsigned)(slot & (bs - 1));
                const size_t off = (size_t)nb * u.blk_stride;
                *reinterpret_cast<uint16_t*>(u.vstore + off + v_elem_offset(noff, lane)) = vvs[j];
                *reinterpret_cast<unsigned*>(u.kstore + off +
                                             k_word_offset<bs>(noff, lane & 31)) = kws[j];
            }
        }
    }

    if constexpr (DEPTH == kBurst || DEPTH == 4) {
        // Runs of up to DEPTH steps issue every step's loads at once (steps
        // past the run re-read its last chunk, which the clamp in load_step
        // keeps inside the run's blocks, and are never computed): one round
        // trip of K/V instead of a pipeline's several, for calls whose
        // partitions are short.  Longer runs take the two-step pipeline.
        if (nsteps <= DEPTH) {
            StepRegs R[DEPTH];
            load_step(0, R[0]);
            if (stores_new && !new_first) store_new();
#pragma unroll
            for (int s = 1; s < DEPTH; ++s) load_step(s, R[s]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < DEPTH; ++s)
                if (s < nsteps) compute_step(s, R[s]);
            return;
        }
    }
    if constexpr (DEPTH == 3) {
        // Three register sets: the loads of steps s+1 and s+2 are in flight
        // while step s computes (for a kernel that runs one wavefront per
        // SIMD, where the extra 32 registers cost no occupancy).  Runs of one
        // or two steps, and the one to four steps after the last whole
        // triple, are peeled so that no load reaches past the run or sits
        // under a branch that joins before its use.
        StepRegs A, B, C;
        if (nsteps == 1) {
            load_step(0, A);
            if (stores_new && !new_first) store_new();
            compute_step(0, A);
        } else if (nsteps == 2) {
            load_step(0, A);
            if (stores_new && !new_first) store_new();
            load_step(1, B);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(0, A);
            compute_step(1, B);
        } else {
            load_step(0, A);
            if (stores_new && !new_first) store_new();
            load_step(1, B);
            int s = 0;
            // steps s and s+1 are in flight at the top of each triple
            for (; s + 5 <= nsteps; s += 3) {
                load_step(s + 2, C);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(s, A);
                load_step(s + 3, A);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(s + 1, B);
                load_step(s + 4, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(s + 2, C);
            }
            const int r = nsteps - s;            // 2, 3 or 4 steps left
            if (r == 2) {
                compute_step(s, A);
                compute_step(s + 1, B);
            } else if (r == 3) {
                load_step(s + 2, C);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(s, A);
                compute_step(s + 1, B);
                compute_step(s + 2, C);
            } else {
                load_step(s + 2, C);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(s, A);
                load_step(s + 3, A);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(s + 1, B);
                compute_step(s + 2, C);
                compute_step(s + 3, A);
            }
        }
        return;
    }

    // Two register sets in ping-pong: the loads of step s+1 are in flight
    // while step s computes.  The loop covers whole pairs that still have a
    // next step to prefetch; the last one or two steps are peeled, so no load
    // ever reaches past the run and no load sits under a branch inside the
    // loop (a conditional load there would make the compiler wait for every
    // outstanding load at the join).
    StepRegs A, B;
    load_step(0, A);
    if (stores_new && !new_first) store_new();
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
        load_step(s + 1, B);
        __builtin_amdgcn_sched_barrier(0);    // keep the prefetch ahead of the math
        compute_step(s, A);
        load_step(s + 2, A);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(s + 1, B);
    }
    if (s + 1 < nsteps) {
        load_step(s + 1, B);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(s, A);
        compute_step(s + 1, B);
    } else {
        compute_step(s, A);
    }
}

// Attend over slots [t0, t1) of one unit in runs of at most kMaxTableSlice
// blocks (t0 a multiple of 32).  The first run's table slice and the new
// token's words are read here, with no branch, so they travel with the
// caller's query loads.
// DEPTH: register sets of the step pipeline (2, or 3 for one wavefront per SIMD),
// or a burst's (4 or kBurst: a run of at most DEPTH steps loaded at once).
// The loads that begin a unit's run of slots from t0: its first table slice
// and this lane's words of the new token's K and V rows.  None of them
// depends on the sequence's length, so a caller may issue them before it
// waits for that.
struct RunStart {
    TableSlice tbl;
    unsigned kword;
    uint16_t vval;
};
template <int BSL>
__device__ __forceinline__ RunStart run_start(const Unit& u, int t0, int lane) {
    RunStart r;
    r.tbl = table_slice(u, t0 >> BSL, lane);
    r.kword = reinterpret_cast<const unsigned*>(u.kn_row)[lane & 31];
    r.vval = u.vn_row[lane];
    return r;
}

template <int BSL, bool ROPE, bool MULTI = false, int DEPTH = 2>
__device__ __forceinline__ void attend(const DecodeArgs& a, const Unit& u, int t0, int t1,
                                       u32x4_t qop0, u32x4_t qop1, State& st,
                                       const RunStart& pre) {
    constexpr int run = kMaxTableSlice << BSL;
    const int lane = u.c16 + 16 * u.q4;
    TableSlice tbl = pre.tbl;
    const unsigned kword = pre.kword;
    const uint16_t vval = pre.vval;
    // cos / sin of the pairs of this lane's new-key word (read with no branch)
    float2 kcos = {1.f, 1.f}, ksin = {0.f, 0.f};
    if (ROPE) {
        const size_t row = (size_t)u.rope_pos * (kHeadDim / 2);
        const int w = lane & 31;
        if (a.rope_style == kRopeHalf) {          // pairs 2(w & 15), 2(w & 15) + 1
            kcos = *reinterpret_cast<const float2*>(a.rope_cos + row + 2 * (w & 15));
            ksin = *reinterpret_cast<const float2*>(a.rope_sin + row + 2 * (w & 15));
        } else {                                  // pair w
            kcos.x = a.rope_cos[row + w];
            ksin.x = a.rope_sin[row + w];
        }
    }
    for (int r0 = t0;;) {
        const int r1 = min(t1, r0 + run);
        attend_run<BSL, ROPE, MULTI, DEPTH>(u, r0, r1, tbl.blk, tbl.ok, kword, vval, kcos, ksin,
                                            a.rope_style, qop0, qop1, st);
        if (r1 >= t1) break;
        r0 = r1;
        tbl = table_slice(u, r0 >> BSL, lane);
    }
}
template <int BSL, bool ROPE, bool MULTI = false, int DEPTH = 2>
__device__ __forceinline__ void attend(const DecodeArgs& a, const Unit& u, int t0, int t1,
                                       u32x4_t qop0, u32x4_t qop1, State& st) {
    attend<BSL, ROPE, MULTI, DEPTH>(a, u, t0, t1, qop0, qop1, st,
                                    run_start<BSL>(u, t0, u.c16 + 16 * u.q4));
}

// bf16 output of the unit's heads with the sink in the denominator:
// out = acc / (l + e^(sigma - m)) (all in the log2 domain).
__device__ __forceinline__ void write_out(const DecodeArgs& a, int b, int g, int lane,
                                          const State& st, float l_tot) {
    const int q4 = lane >> 4;
    const Col c = column(a, lane);
    if (!c.ok) return;
    const float sig = a.sinks ? a.sinks[g * a.G + c.h] * kLog2e : -INFINITY;
    const float inv = 1.0f / (l_tot + __builtin_amdgcn_exp2f(sig - st.m));
    uint16_t* op = a.out + col_row(a, b, g, c) * kHeadDim + 4 * q4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x2_t o = {pack_bf16(st.acc[j][0] * inv, st.acc[j][1] * inv),
                           pack_bf16(st.acc[j][2] * inv, st.acc[j][3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + 16 * j) = o;
    }
}

// zeros for the unit's columns (nothing attended: the sink has no value row)
__device__ __forceinline__ void write_zero(const DecodeArgs& a, int b, int g, int lane) {
    const int q4 = lane >> 4;
    const Col c = column(a, lane);
    if (!c.ok) return;
    uint16_t* op = a.out + col_row(a, b, g, c) * kHeadDim + 4 * q4;
    const u32x2_t z = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2_t*>(op + 16 * j) = z;
}

// Partial of a run for this lane's column (when ok): o = acc / l (fp32, 64
// values at po + row*row_stride), lse = ln sum e^s = (m + log2 l) ln 2 at
// pl[row * lse_stride].
__device__ __forceinline__ void write_partial(bool ok, size_t row, int lane, const State& st,
                                              float l_tot, float* po, size_t row_stride,
                                              float* pl, size_t lse_stride) {
    const int q4 = lane >> 4;
    if (!ok) return;
    // a column with no slot in the run (a query token before the run's slots:
    // only with several query tokens) leaves o = 0 and lse = -inf, weight 0
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    float* p = po + row * row_stride + 4 * q4;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4_t*>(p + 16 * j) = st.acc[j] * inv;
    if (q4 == 0)
        pl[row * lse_stride] = empty ? -INFINITY : (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

}  // namespace mfma
}  // namespace sa
