"""fp64 oracle of the single-token decode step over a paged / ring KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path must
never import this module.

Sources.  The SimpleLLM README (shadowgraph.io/naklecha/simple-llm): its
optimisation table has one row for the fused decode-attention kernel
(attention sinks, sliding window, GQA and the KV append in one kernel), one
row for the paged KV cache of full-attention layers and one row for the ring
buffer of sliding-window layers.  The setup page of the
"learn-llm-inference-from-scratch" tutorial (llminference.xinbetween.com/en/setup):
its file table lists chapters on the KV cache (S05), PagedAttention (S06) and
FlashAttention (S12) without their contents.  A discussion thread
(astro-solid-hn.netlify.app/stories/49693384) only remarks that GQA and
sliding-window attention change an implementation a lot.  No page prints a
formula, so the definitions here are the standard ones for the named
concepts; the readings taken where the pages are silent are:

* softmax scale 1/sqrt(D), applied to q.k (not to the sink);
* one sink logit per *query* head, compared unscaled with the scaled scores,
  entering the softmax denominator only (it has no value row);
* GQA with contiguous groups: query head h reads KV head h // (Hq/Hkv);
* ``seq_lens[b]`` counts the tokens *after* this step's append, so the new
  token sits at position L-1;
* a window W > 0 keeps the W most recent positions including the new one,
  stored in a ring of W slots (position p in slot p mod W); W <= 0 means a
  full-attention layer over the paged cache;
* cache layout (the library's documented layout, restated here on its own):
  K pool ``[num_blocks][Hkv][n][block_size][D/n]`` (each K row cut into n
  pieces of D/n dimensions, each piece slot-major: slot s, dimension d at
  ``[d // (D/n)][s][d % (D/n)]``; the library's n is 2, the pool's third
  axis gives it) and V pool ``[num_blocks][Hkv][block_size/c][D][c]`` (V
  transposed inside a block in chunks of c slots: slot s, dimension d at
  ``[s // c][d][s % c]``; the library's c is 8, the pool's last axis gives
  it);
  ``block_table[b][j]`` is the physical block holding slots
  ``[j*block_size, (j+1)*block_size)`` of sequence b.

Everything is computed in float64 from the exact widening of the bf16
inputs.  The code walks positions, not tiles: there is no blocking, no
online softmax and no split of the sum.
"""

from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# Value widening
# --------------------------------------------------------------------------

def bf16_bits_to_f64(x):
    """Exact widening of bfloat16 bit patterns (uint16) to float64.

    A bfloat16 is the upper half of an IEEE-754 binary32, so the value is the
    binary32 whose high 16 bits are the pattern and whose low 16 bits are 0.
    Arrays of any floating dtype are widened with ``astype``.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# Indexing: GQA group, attended positions, storage slot, block lookup
# --------------------------------------------------------------------------

def query_group(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h`` under GQA (SimpleLLM README, fused-kernel row;
    the discussion thread on GQA).  Reading: contiguous groups of Hq/Hkv query heads share
    one KV head."""
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    return h // (num_q_heads // num_kv_heads)


def attended_positions(L: int, window: int) -> range:
    """Positions a query at position L-1 attends to (SimpleLLM README, fused-kernel row:
    sliding window).  Full attention sees [0, L); a window W > 0 sees the W
    most recent positions including the current one, [max(0, L-W), L)."""
    if window <= 0:
        return range(0, L)
    return range(max(0, L - window), L)


def storage_slot(p, window: int):
    """Slot that holds position p (SimpleLLM README, paged-cache and ring-buffer rows).
    A full-attention layer stores position p in slot p; a sliding-window
    layer keeps a ring of W slots and stores position p in slot p mod W.
    ``p`` may be an int or an integer array."""
    return p if window <= 0 else p % window


def locate(block_table, b: int, slot, block_size: int):
    """(physical block, offset) of a slot of sequence b through its block
    table (SimpleLLM README, paged-cache row; tutorial setup page, S06 PagedAttention).  ``slot``
    may be an int or an integer array."""
    row = np.asarray(block_table)[b]
    return row[slot // block_size].astype(np.int64), slot % block_size


def _gather(k_cache, v_cache, block_table, b, g, positions, window):
    """K and V rows [n, D] (float64) of KV head g for the given positions."""
    p = np.asarray(positions, dtype=np.int64)
    blks, offs = locate(block_table, b, storage_slot(p, window), k_cache.shape[3])
    # the row's pieces, in order (advanced indices first: [n, pieces, D/pieces])
    D = k_cache.shape[2] * k_cache.shape[4]
    K = bf16_bits_to_f64(k_cache[blks, g, :, offs, :]).reshape(len(p), D)    # [n, D]
    c = v_cache.shape[-1]                                    # slots per V chunk
    V = bf16_bits_to_f64(v_cache[blks, g, offs // c, :, offs % c])   # [n, D]
    return K, V


# --------------------------------------------------------------------------
# Attention with a sink
# --------------------------------------------------------------------------

def _sink(sinks, h: int) -> float:
    """Sink logit of query head h; no sinks means a logit of -inf, i.e. no
    sink at all (SimpleLLM README, fused-kernel row, attention sinks)."""
    if sinks is None:
        return -math.inf
    return float(np.asarray(sinks, dtype=np.float64)[h])


def decode_attention(q, k_cache, v_cache, block_table, seq_lens, sinks, window):
    """Output of the decode-attention step, float64 ``[B][Hq][D]``.

    For sequence b and query head h with KV head g = h // (Hq/Hkv), the scores
    are s_p = (q[b,h] . K_p) / sqrt(D) over the attended positions p.  The
    sink logit sigma_h joins the softmax normaliser but has no value row:

        M   = max(max_p s_p, sigma_h)
        Z   = sum_p exp(s_p - M) + exp(sigma_h - M)
        out = sum_p exp(s_p - M) V_p / Z

    i.e. a softmax over [s_lo .. s_{L-1}, sigma_h] with the last column's
    weight dropped (SimpleLLM README, fused-kernel row; tutorial setup page, S05/S06 for the cached
    keys and values read through the block table).  With no positions and no
    sink the output is 0.

    ``q`` is bf16 bits (uint16) or float ``[B][Hq][D]``; caches are bf16 bits
    or float in the layouts of the module docstring; ``sinks`` is ``[Hq]`` or
    None.
    """
    q = bf16_bits_to_f64(q)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        positions = attended_positions(int(seq_lens[b]), window)
        for g in range(Hkv):
            K, V = _gather(k_cache, v_cache, block_table, b, g, positions, window)
            for h in range(Hq):
                if query_group(h, Hq, Hkv) != g:
                    continue
                s = (K @ q[b, h]) * scale                   # [n]
                sigma = _sink(sinks, h)
                M = max(s.max() if len(s) else -math.inf, sigma)
                if M == -math.inf:
                    continue                                 # nothing to attend
                w = np.exp(s - M)
                Z = w.sum() + math.exp(sigma - M)
                out[b, h] = (w @ V) / Z
    return out


def partial_attention(q, k_cache, v_cache, block_table, b, h, positions, window):
    """Softmax attention of (b, h) over a subset of positions, without sink.

    Returns ``(o, lse)`` with lse = log sum_p exp(s_p) and
    o = sum_p exp(s_p) V_p / exp(lse).  An empty subset gives (0, -inf).
    This is one split-K partition of the flash-decoding scheme that the
    combine merges (tutorial setup page, S12 FlashAttention names the tiled softmax).
    """
    q = bf16_bits_to_f64(q)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_cache.shape[1]
    g = query_group(h, Hq, Hkv)
    positions = list(positions)
    if not positions:
        return np.zeros(D), -math.inf
    K, V = _gather(k_cache, v_cache, block_table, b, g, positions, window)
    s = (K @ q[b, h]) / math.sqrt(D)
    m = s.max()
    w = np.exp(s - m)
    lse = m + math.log(w.sum())
    return (w @ V) / w.sum(), lse


def combine(part_o, part_lse, sinks):
    """Log-sum-exp merge of split partials with the sink, float64 [B][Hq][D].

    ``part_o`` is ``[B][Hq][S][D]`` (each partial already normalised by its
    own softmax sum), ``part_lse`` is ``[B][Hq][S]`` (natural log; -inf marks
    an empty partition).  With M = max(max_p lse_p, sigma_h):

        out = sum_p exp(lse_p - M) o_p / (sum_p exp(lse_p - M) + exp(sigma_h - M))

    which equals the one-shot definition of ``decode_attention`` for any
    partition of the attended positions.
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    B, Hq, S, D = part_o.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            sigma = _sink(sinks, h)
            M = max(part_lse[b, h].max() if S else -math.inf, sigma)
            if M == -math.inf:
                continue
            num = np.zeros(D)
            den = math.exp(sigma - M)
            for p in range(S):
                if part_lse[b, h, p] == -math.inf:
                    continue                                 # empty partition
                w = math.exp(part_lse[b, h, p] - M)
                num += w * part_o[b, h, p]
                den += w
            out[b, h] = num / den
    return out


# --------------------------------------------------------------------------
# KV append
# --------------------------------------------------------------------------

def kv_append(k_cache, v_cache, k_new, v_new, block_table, seq_lens, window):
    """Caches after writing the new token's K and V (SimpleLLM README, fused-kernel row:
    the KV append; paged-cache and ring-buffer rows for where it goes).

    The new token of sequence b is position L-1 (L = seq_lens[b]); it goes to
    slot storage_slot(L-1, window) through the block table, for every KV head.
    Sequences with L <= 0 append nothing, and neither does a sequence whose
    slot lies past its table row (slot >= entries x block_size: a length past
    the table's capacity, a caller error the library documents as writing
    nothing).  Returns modified copies; the copy is a bit copy, so any dtype
    (e.g. bf16 bits as uint16) works.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    pieces, bs = k.shape[2], k.shape[3]                      # K row pieces, block size
    Hkv = k.shape[1]
    c = v.shape[-1]                                          # slots per V chunk
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        slot = storage_slot(L - 1, window)
        if slot // bs >= np.asarray(block_table).shape[1]:
            continue                                         # past the table: no write
        blk, off = locate(block_table, b, slot, bs)
        blk, off = int(blk), int(off)
        for g in range(Hkv):
            k[blk, g, :, off, :] = np.reshape(k_new[b, g, :], (pieces, -1))
            v[blk, g, off // c, :, off % c] = v_new[b, g, :]
    return k, v
