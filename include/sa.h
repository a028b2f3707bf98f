/*
 * sa.h -- single-token decode attention over a paged / ring KV cache on
 * AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * Sources.  The SimpleLLM README (shadowgraph.io/naklecha/simple-llm),
 * optimisation table: one fused decode-attention kernel covers attention
 * sinks, sliding-window attention, GQA and the KV append; full-attention
 * layers keep a paged KV cache; sliding-window layers keep a ring buffer.
 * The "learn-llm-inference-from-scratch" setup page, file table: KV cache
 * (S05), PagedAttention (S06) and FlashAttention (S12) chapters.  The pages
 * print no formula; the definitions below are the standard ones for those
 * concepts.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer is DEVICE memory owned by the caller, except the
 *    `const sa_dims*`, which is host memory read during the call only.
 *    The library never allocates, frees or synchronises; it keeps no
 *    global mutable state (save the per-device address of the no-allocation
 *    call's scratch, set once under a lock) and is safe to call from several
 *    host threads.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *    null stream of the calling thread's current HIP device).  A return of
 *    SA_OK means the work was enqueued; a fault inside a kernel surfaces as a
 *    HIP error at the caller's next synchronisation.  Launches go to the
 *    calling thread's current device, which must be the device of `stream`
 *    and of every pointer passed.
 *  - Errors are negative SA_ERR_* codes returned before anything is
 *    launched; no call aborts or throws.  SA_ERR_HIP is the status of the
 *    call's own launches: an error an earlier HIP call left on the thread
 *    does not make a call fail.
 *  - q, out, k_new, v_new, k_cache, v_cache, part_o, the rotary tables and
 *    the workspace are read or written 16 bytes at a time and must be
 *    16-byte aligned (SA_ERR_INVALID_ARG otherwise).
 *  - Shapes: B sequences, Hq query heads, Hkv KV heads (Hq % Hkv == 0,
 *    Hq/Hkv <= 16), head_dim D == 64, block_size bs in {8, 16, 32, 64}.
 *  - GQA: query head h reads KV head h / (Hq/Hkv) (contiguous groups).
 *  - Layouts (row-major, innermost last; bf16 = IEEE bfloat16 bits):
 *      q, out          bf16 [B][Hq][D]
 *      k_new, v_new    bf16 [B][Hkv][D]
 *      k_cache         bf16 [num_blocks][Hkv][2][bs][32]
 *                      (each K row cut into two halves of 32 dims, each
 *                       half slot-major: slot s, dim d at [d/32][s][d%32])
 *      v_cache         bf16 [num_blocks][Hkv][bs/8][D][8]
 *                      (V transposed inside a block in chunks of 8 slots:
 *                       slot s, dim d at [s/8][d][s%8])
 *                      This pool layout is part of the contract: a caller
 *                      states it in sa_dims.cache_layout (SA_LAYOUT_K2_V8).
 *                      Pools of plain rows, [num_blocks][Hkv][bs][D] for K
 *                      and V (SA_LAYOUT_PLAIN, also what a zero-filled
 *                      sa_dims says), are refused with SA_ERR_UNSUPPORTED
 *                      rather than read wrongly.
 *      block_table     int32 [B][max_blocks_per_seq]
 *      seq_lens        int32 [B]
 *      sinks           fp32 [Hq] (may be NULL: no sink)
 *      part_o          fp32 [B][Hq][S][D]
 *      part_lse        fp32 [B][Hq][S]        (natural log)
 *  - seq_lens[b] = L is the context length AFTER this step's append: the
 *    new token is position L-1.  The same array feeds append and attention.
 *  - window <= 0: full-attention layer; position p lives in slot p.
 *    window  = W > 0: sliding-window layer kept as a ring of W slots;
 *    position p lives in slot p mod W and the query attends to positions
 *    [max(0, L-W), L), i.e. slots [0, min(L, W)).  ceil(W/bs) must not
 *    exceed max_blocks_per_seq.
 *  - Slot s of sequence b lives in block block_table[b][s / bs] at offset
 *    s % bs.  Only the table entries that cover attended slots are read.
 *    A context longer than max_blocks_per_seq*bs is cut to that capacity.
 *    Table entries outside [0, num_blocks) are clamped into range for the
 *    attention's reads, and an append whose slot's entry is outside writes
 *    nothing, in sa_kv_append and inside the attention launch alike (a
 *    caller error, but never a wild access).
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t sa_bf16;   /* bfloat16 bit pattern */

typedef struct sa_dims {
    int32_t num_seqs;            /* B   (0 is a no-op)                          */
    int32_t num_q_heads;         /* Hq                                          */
    int32_t num_kv_heads;        /* Hkv                                         */
    int32_t head_dim;            /* D: 64                                       */
    int32_t block_size;          /* bs: 8, 16, 32 or 64 tokens per block        */
    int32_t max_blocks_per_seq;  /* row stride of block_table; the capacity
                                    max_blocks_per_seq * bs is at most 2^30
                                    tokens (SA_ERR_UNSUPPORTED otherwise)      */
    int32_t num_blocks;          /* blocks in each pool                         */
    int32_t num_splits;          /* 0: the library's fixed split table;
                                    > 0: use at most this many split-K
                                    partitions per (sequence, KV head)         */
    int32_t variant;             /* 0: default kernels; see SA_VARIANT_*        */
    int32_t num_query_tokens;    /* T: new tokens per sequence (0 means 1).  With
                                    T > 1 (a query tile: speculative verify,
                                    chunked prefill) token t sits at position
                                    L-T+t and attends causally up to itself;
                                    q / out are [B][T][Hq][D], k_new / v_new
                                    [B][T][Hkv][D], partials [B][T][Hq][S][D].
                                    Needs window <= 0 and T*(Hq/Hkv) <= 16
                                    (SA_ERR_UNSUPPORTED otherwise); not with
                                    RoPE or SA_VARIANT_VALU.                   */
    int32_t cache_layout;        /* layout of k_cache / v_cache: must be
                                    SA_LAYOUT_K2_V8 for every call that takes
                                    the pools or sizes a call on them
                                    (SA_ERR_UNSUPPORTED otherwise; sa_combine
                                    ignores it)                                */
} sa_dims;

/* Pool layouts (sa_dims.cache_layout). */
enum {
    SA_LAYOUT_PLAIN = 0,   /* K and V [num_blocks][Hkv][bs][D]: not supported   */
    SA_LAYOUT_K2_V8 = 1    /* K [num_blocks][Hkv][2][bs][D/2] (two slot-major
                              halves), V [num_blocks][Hkv][bs/8][D][8] (chunks
                              of 8 slots): the layout the kernels read         */
};

enum {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = -1,    /* NULL pointer, negative or inconsistent size  */
    SA_ERR_UNSUPPORTED = -2,    /* D != 64, Hq % Hkv != 0, Hq/Hkv > 16, bs,
                                   capacity > 2^30 tokens, ...                  */
    SA_ERR_WORKSPACE = -3,      /* workspace missing or too small               */
    SA_ERR_HIP = -4,            /* the HIP runtime refused a launch             */
    SA_ERR_SCRATCH = -5         /* the no-allocation call needs more than the
                                   library's SA_SCRATCH_BYTES of scratch        */
};

/* Kernel variants (sa_dims.variant).  All give results within the same
 * tolerance; they exist so each design choice can be measured. */
enum {
    SA_VARIANT_DEFAULT = 0,
    SA_VARIANT_MFMA_TWO_PASS = 1, /* MFMA partitions, separate combine launch  */
    SA_VARIANT_MFMA_FUSED = 2,    /* MFMA partitions, combine by the last one  */
    SA_VARIANT_VALU = 3,          /* vector-ALU partitions (no MFMA)           */
    SA_VARIANT_MFMA_BALANCED = 4, /* MFMA, equal work per wavefront across the
                                     batch, merge launch for split units       */
    SA_VARIANT_MFMA_BALANCED_LAST_MERGES = 5 /* the same split; the last
                                     wavefront to finish a split unit merges it
                                     (agent-coherent stores and a device-scope
                                     counter instead of the merge launch)      */
};

/*
 * KV append (SimpleLLM README, optimisation table: the fused kernel's KV
 * append; paged-cache and ring-buffer rows for where the token goes).
 * For every sequence b with L = seq_lens[b] >= 1 and every KV head g, writes
 * k_new[b][g][:] to slot off of k_cache[blk][g] and v_new[b][g][:] to slot
 * off of v_cache[blk][g] (the layouts above), where slot s = L-1
 * (window <= 0) or (L-1) mod W,
 * blk = block_table[b][s / bs], off = s % bs.  A bit copy: nothing else in
 * either pool changes.  Sequences with L <= 0 are skipped.
 * Uses: num_seqs, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
 * num_blocks.
 */
int sa_kv_append(const sa_bf16* k_new, const sa_bf16* v_new,
                 sa_bf16* k_cache, sa_bf16* v_cache,
                 const int32_t* block_table, const int32_t* seq_lens,
                 int32_t window, const sa_dims* dims, void* stream);

/*
 * Split-K partitions S the attention call uses for these dims and window
 * (>= 1), or a negative SA_ERR_* code.  Deterministic: it depends only on
 * the dims, the window and num_splits, never on timing.
 */
int32_t sa_decode_num_splits(const sa_dims* dims, int32_t window);

/*
 * Device workspace bytes sa_decode_attention needs for these dims and window
 * (0 when it needs none, also returned for invalid dims).  The first 1 MiB
 * of a workspace holds completion counters: zero-fill the workspace once
 * before its first use; every call leaves those counters at zero again, so
 * one workspace of the largest size needed serves any sequence of calls on a
 * stream, whatever their dims.  Calls that may run at the same time need
 * workspaces of their own.
 */
size_t sa_decode_workspace_bytes(const sa_dims* dims, int32_t window);

/*
 * Decode attention (SimpleLLM README, optimisation table: sinks, sliding
 * window and GQA in one decode-attention kernel; paged cache and ring
 * buffer; the tutorial's PagedAttention and FlashAttention chapters for the
 * block-table read and the tiled online softmax).  For every sequence b and
 * query head h, with scores s_p = q[b][h] . K_p / sqrt(D) over the attended
 * positions p and sink logit sigma_h = sinks[h] (-inf if sinks is NULL):
 *
 *     M = max(max_p s_p, sigma_h)
 *     out[b][h] = sum_p e^(s_p - M) V_p / (sum_p e^(s_p - M) + e^(sigma_h - M))
 *
 * rounded to bf16 (round to nearest even); 0 where nothing is attended.
 * Accumulation is fp32.  Long contexts are cut into S split-K partitions
 * whose partials are merged with a log-sum-exp combine inside the call.
 * workspace: at least sa_decode_workspace_bytes(dims, window) bytes (may be
 * NULL when that is 0), zero-filled before first use.
 */
int sa_decode_attention(const sa_bf16* q, const sa_bf16* k_cache, const sa_bf16* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const float* sinks, int32_t window, sa_bf16* out,
                        const sa_dims* dims, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * The fused decode step (SimpleLLM README, optimisation table: one
 * decode-attention kernel that also does the KV append): exactly
 * sa_kv_append followed by sa_decode_attention with the same arguments, in
 * one launch (plus the merge launch when the call is split).  The wavefront
 * that attends the new token's slot stores k_new / v_new into the pools and
 * takes the new token's K and V from k_new / v_new, so the pools after the
 * call are bit-identical to those after sa_kv_append and the output is that
 * of sa_decode_attention on them.  A new token whose slot is past the
 * table's capacity is skipped, as by sa_kv_append.  Not available with
 * SA_VARIANT_VALU.
 */
int sa_decode_attention_append(const sa_bf16* q, const sa_bf16* k_new, const sa_bf16* v_new,
                               sa_bf16* k_cache, sa_bf16* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const float* sinks, int32_t window, sa_bf16* out,
                               const sa_dims* dims, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Exactly
 * sa_decode_attention_append without a workspace argument, with
 * bit-identical results.  What the call would keep in a workspace (split-K
 * partials, the balanced kernel's unit records, completion counters) goes to
 * a device array the library owns: SA_SCRATCH_BYTES bytes on each GPU,
 * created zero-filled with the library's code on that device and held until
 * the process ends.  The call allocates and frees nothing; on its first call
 * on a device it looks the array's address up (hipGetSymbolAddress) with
 * that device current and keeps it (under a lock: the only state the library
 * keeps).  A call whose sa_decode_workspace_bytes exceeds SA_SCRATCH_BYTES
 * returns SA_ERR_SCRATCH before launching anything.  Every call on one GPU
 * uses that GPU's one array and leaves its counters at zero, as it found
 * them; the rest is rewritten by each call before it is read.  Calls that
 * may overlap on one GPU (several streams, several host threads) race on the
 * array and must be serialised by the caller.
 */
#define SA_SCRATCH_BYTES ((size_t)32 << 20)
int sa_decode_attention_append_noalloc(const sa_bf16* q, const sa_bf16* k_new,
                                       const sa_bf16* v_new, sa_bf16* k_cache, sa_bf16* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const float* sinks, int32_t window, sa_bf16* out,
                                       const sa_dims* dims, void* stream);

/*
 * Rotary position embedding of the new token (SimpleLLM README, optimisation
 * table: RoPE as one fused kernel).  Pair i of a head vector's D dims is
 * turned by the angle whose cosine and sine are cos_table[p][i] and
 * sin_table[p][i] at the token's position p = L-1 (rows past the tables' end
 * use the last row):  (x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin), each
 * product and sum rounded to float32 on its own, the result rounded to bf16
 * (nearest, ties to even).  Pairing: SA_ROPE_HALF pairs dim i with dim
 * i + D/2; SA_ROPE_INTERLEAVED pairs dims 2i and 2i+1.  The tables are
 * device fp32 [max_positions][head_dim/2], 16-byte aligned, owned by the
 * caller.
 */
#define SA_ROPE_HALF 0
#define SA_ROPE_INTERLEAVED 1

typedef struct {
    const float* cos_table;
    const float* sin_table;
    int32_t max_positions;
    int32_t style;
} sa_rope;

/*
 * sa_decode_attention_append with the rotary embedding fused in: q and k_new
 * are taken unrotated and rotated at each sequence's position L-1; the
 * rotated key (and the unrotated v_new) are appended, and the attention uses
 * the rotated query.  The cache then holds rotated keys, as a model with
 * rotary embedding keeps it.  rope must be non-null and valid
 * (SA_ERR_INVALID_ARG otherwise); not available with SA_VARIANT_VALU.
 */
int sa_decode_attention_append_rope(const sa_bf16* q, const sa_bf16* k_new, const sa_bf16* v_new,
                                    sa_bf16* k_cache, sa_bf16* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const float* sinks, int32_t window, const sa_rope* rope,
                                    sa_bf16* out, const sa_dims* dims, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Split-K partials only, for a caller that merges them itself (for example
 * across devices that each hold part of a context).  With S =
 * sa_decode_num_splits(dims, window), partition j of (b, h) covers attended
 * slots [j*P, min(n, (j+1)*P)) for the library's partition length P, and
 *     part_lse[b][h][j] = log sum_p e^(s_p)          (-inf if empty)
 *     part_o[b][h][j][:] = sum_p e^(s_p) V_p / e^(part_lse)
 * No sink is applied.  part_o of an empty partition is left unwritten.
 */
int sa_decode_partials(const sa_bf16* q, const sa_bf16* k_cache, const sa_bf16* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int32_t window, float* part_o, float* part_lse,
                       const sa_dims* dims, void* stream);

/*
 * Log-sum-exp combine of split-K partials with the sink (the tutorial setup
 * page, file table, FlashAttention chapter (S12): the tiled online softmax
 * whose per-tile (o, lse) pairs merge this way; SimpleLLM README,
 * optimisation table, fused decode-attention row: the attention sink, which
 * joins the normaliser once and has no value row).  For num_splits partials
 * per (b, h):
 *     M = max(max_j part_lse[b][h][j], sigma_h)
 *     out[b][h] = sum_j e^(lse_j - M) part_o[b][h][j] / (sum_j e^(lse_j - M) + e^(sigma_h - M))
 * rounded to bf16; partials with lse = -inf carry no weight (whatever their
 * part_o holds, NaN included, never reaches out; the whole [B][Hq][S][D]
 * part_o must still be allocated); 0 where nothing remains.  This equals
 * the one-shot attention of sa_decode_attention when the partials cover the
 * attended positions in disjoint sets.  Uses num_seqs, num_q_heads,
 * head_dim and num_query_tokens of dims (rows (b*T + t)*Hq + h).  Errors:
 * SA_ERR_INVALID_ARG (NULL dims, part_o, part_lse or out with num_seqs > 0;
 * num_splits < 1; negative sizes), SA_ERR_UNSUPPORTED (head_dim != 64).
 */
int sa_combine(const float* part_o, const float* part_lse, const float* sinks,
               int32_t num_splits, sa_bf16* out, const sa_dims* dims, void* stream);

/*
 * Measurement helper, not a step of the decode path: reads `bytes` of device
 * memory at `data` once, as a plain streaming read (16-byte non-temporal
 * loads, the hint the decode kernels' K/V loads carry), and XORs every 32-bit
 * word of it into *sink (device memory; the caller sets its start value,
 * normally 0).  Its bandwidth is the practical HBM read ceiling the decode
 * kernels are compared against.  bytes must be a multiple of 16 (0 launches
 * nothing); data 16-byte aligned.
 */
int sa_read_bandwidth_probe(const void* data, size_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement helper, not a step of the decode path: the decode kernels'
 * read pattern with no arithmetic.  tiles[0..ntiles) are tile numbers; tile k
 * is the 2048 bytes at data + 2048 k (one (block, KV head) piece of a pool at
 * block size 16).  waves one-wavefront workgroups each read a contiguous
 * stretch of the list as the balanced decode kernel walks its steps: 8 KiB
 * (four tiles) a step, three steps of loads in flight, non-temporal 16-byte
 * loads, the tile numbers fetched 64 at a time.  Every 32-bit word of every
 * listed tile is XORed into *sink once per listing.  Tile numbers outside
 * [0, bytes / 2048) are clamped into it.  data 16-byte aligned; waves in
 * [1, 65535]; ntiles = 0 launches nothing.
 */
int sa_read_tiles_probe(const void* data, size_t bytes, const int32_t* tiles, int64_t ntiles,
                        int32_t waves, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* sa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SA_H_ */
