"""Rotary position embedding of the new token's query and key, and the decode
step with it: TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources.  The SimpleLLM README (shadowgraph.io/naklecha/simple-llm) counts a
fused RoPE kernel, used whatever the batch size, among the decode-path kernels
of its optimisation table.  The setup page of the
"learn-llm-inference-from-scratch" tutorial warns, in its closing advice on
running a real model, that the RoPE layout is among the things most likely to
be got wrong.  Neither page prints the rotation, so this module states
the standard rotary embedding:

* the D dims of a head vector form D/2 pairs (x1, x2), and pair i is turned
  by the angle a_i(p) of the token's position p:
  (x1, x2) -> (x1 cos a - x2 sin a,  x2 cos a + x1 sin a);
* the two pairings in use are both offered, since the pages fix neither:
  "half"        pair i = (dim i, dim i + D/2)  for i < D/2,
  "interleaved" pair i = (dim 2i, dim 2i + 1);
* the angles are not on the pages either: the caller passes the tables
  cos_table[p][i] = cos a_i(p) and sin_table[p][i] = sin a_i(p) (float32,
  [positions][D/2]); a position past the table's last row uses that row;
* the token appended at this step sits at position L - 1 (``seq_lens`` counts
  it), and q and the new key are both rotated there; V is not rotated.

Precision reading.  The rotated vectors are rounded to bf16: the key because
the cache holds bf16, the query because the products take bf16 operands.
Where a rounding decides stored bits, the oracle takes the decision in the
kernel's precision: each product and each sum in float32, rounded on its own
(no fused multiply-add), then rounded to the nearest bf16 (ties to even).
That keeps the cache comparison bit-exact; the rest of the step is the fp64
definition of ``decode_step``.
"""

from __future__ import annotations

import numpy as np

from . import decode_step as _ds

HALF = "half"
INTERLEAVED = "interleaved"


def pair_dims(D: int, style: str):
    """(first, second) dim index of every pair i = 0..D/2-1."""
    i = np.arange(D // 2)
    if style == HALF:
        return i, i + D // 2
    if style == INTERLEAVED:
        return 2 * i, 2 * i + 1
    raise ValueError(f"unknown RoPE style {style!r}")


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; uint16 bits.

    A bfloat16 is the high half of a binary32, so rounding keeps the high 16
    bits and adds one unit of the kept part when the dropped half exceeds
    0x8000, or equals it with an odd kept part.  (No NaN or infinity occurs
    in these inputs.)
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> 16
    drop = u & 0xFFFF
    up = (drop > 0x8000) | ((drop == 0x8000) & (keep & 1 == 1))
    return (keep + up).astype(np.uint16)


def rotate_f32(x, cos_row, sin_row, style: str) -> np.ndarray:
    """The rotation of head vectors x[..., D] (float32) by per-pair cos/sin rows
    [..., D/2], each product and sum rounded to float32 on its own."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    d1, d2 = pair_dims(x.shape[-1], style)
    x1, x2 = x[..., d1], x[..., d2]
    y = np.empty_like(x)
    # numpy float32 arithmetic rounds every product and every sum on its own
    y[..., d1] = (x1 * c) - (x2 * s)
    y[..., d2] = (x2 * c) + (x1 * s)
    return y


def table_rows(table, positions) -> np.ndarray:
    """Rows of a [P][D/2] table at the given positions (past the end: last row)."""
    table = np.asarray(table, dtype=np.float32)
    p = np.minimum(np.asarray(positions), table.shape[0] - 1)
    return table[p]


def rope_bf16(x_bits, positions, cos_table, sin_table, style: str) -> np.ndarray:
    """bf16 bits of head vectors x (bf16 bits [..., D]) rotated at ``positions``
    (broadcast over x's leading axes except the last)."""
    x = _ds.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)).astype(np.float32)
    c = table_rows(cos_table, positions)
    s = table_rows(sin_table, positions)
    return f32_to_bf16_bits(rotate_f32(x, c, s, style))


def decode_step_rope(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, sinks, window,
                     cos_table, sin_table, style: str):
    """The decode step with RoPE: rotate each sequence's query heads and new key
    at its position L-1, append the rotated key and the (unrotated) value,
    then attend with the rotated query.

    Inputs as in ``decode_step.decode_attention`` / ``kv_append`` (bf16 bits),
    plus the cos/sin tables.  Returns (k_cache, v_cache, out): the caches after
    the append (copies) and the fp64 output.  A sequence with L = 0 appends
    nothing and its output is 0.
    """
    seq_lens = np.asarray(seq_lens)
    pos = np.maximum(seq_lens.astype(np.int64) - 1, 0)
    q_rot = rope_bf16(q, pos[:, None], cos_table, sin_table, style)
    k_rot = rope_bf16(k_new, pos[:, None], cos_table, sin_table, style)
    k2, v2 = _ds.kv_append(k_cache, v_cache, k_rot, v_new, block_table, seq_lens, window)
    out = _ds.decode_attention(q_rot, k2, v2, block_table, seq_lens, sinks, window)
    return k2, v2, out
