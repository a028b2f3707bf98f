"""The decode step with several new tokens per sequence (a query tile of T >
1): TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources.  The tutorial's setup page lists, beside its KV-cache and
PagedAttention chapters, speculative decoding and chunked prefill; both read
the paged cache with more than one new token per sequence.  No page prints the
computation, so this is the plain causal reading:

* a call carries T new tokens for every sequence; ``seq_lens[b]`` = L counts
  them, so token t (0 <= t < T) sits at position L - T + t;
* token t attends every position up to and including its own (causal inside
  the new tokens, the whole cached history before them), with the same scale,
  GQA map and sink as the single-token step: its output is exactly the
  single-token decode output of a sequence of length L - T + t + 1;
* the append writes new token t at position L - T + t (positions below 0 or
  past the table's capacity are skipped, as the single-token append skips
  them);
* full-attention (paged) layers only: a ring of exactly W slots cannot hold
  the window of every token of a tile (the later tokens overwrite positions the
  earlier ones still see), so T > 1 with a window is outside this definition.

Layouts: q and out ``[B][T][Hq][D]``, k_new and v_new ``[B][T][Hkv][D]``.
"""

from __future__ import annotations

import numpy as np

from . import decode_step as _ds


def token_lengths(seq_lens, T: int) -> np.ndarray:
    """[B][T]: the length whose last position is token t's, L - (T - 1 - t)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    return L[:, None] - (T - 1 - np.arange(T))[None, :]


def decode_attention_multi(q, k_cache, v_cache, block_table, seq_lens, sinks, window=0):
    """fp64 output [B][T][Hq][D] of T causal query tokens per sequence."""
    q = np.asarray(q)
    B, T, Hq, D = q.shape
    if window > 0 and T > 1:
        raise ValueError("several query tokens per sequence need a full-attention layer")
    lens = token_lengths(seq_lens, T)
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            Lt = max(int(lens[b, t]), 0)
            out[b, t] = _ds.decode_attention(q[b:b + 1, t], k_cache, v_cache, block_table[b:b + 1],
                                             np.array([Lt]), sinks, window)[0]
    return out


def kv_append_multi(k_cache, v_cache, k_new, v_new, block_table, seq_lens, window=0):
    """Copies of the pools after writing new token t of sequence b at position
    L - T + t, for every t (in order)."""
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    T = k_new.shape[1]
    if window > 0 and T > 1:
        raise ValueError("several new tokens per sequence need a full-attention layer")
    lens = token_lengths(seq_lens, T)
    k, v = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    for t in range(T):
        k, v = _ds.kv_append(k, v, k_new[:, t], v_new[:, t], block_table,
                             np.maximum(lens[:, t], 0), window)
    return k, v
