"""Pins of the multi-token oracle (oracle/multi_token.py), written apart from it:
a pure-Python brute force over a layout-free history with an explicit causal
mask, torch's fp64 scaled_dot_product_attention with a boolean mask and the
sink as an extra key, the single-token case, and the append written position
by position from the history.

Each pin takes the module so that the planted-mistake tests can hand it a
mutated one.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import pins
from oracle import decode_step


def _history(seed, B, T, Hq, Hkv, lens):
    """A layout-free history (pins.History) and T query tokens per sequence."""
    h = pins.make_history(seed, B, Hq, Hkv, 64, lens)
    g = torch.Generator().manual_seed(seed + 1)
    qs = pins.bf16_bits(torch.randn(B, T, Hq, 64, generator=g))
    return h, qs


def _brute(h, qs):
    """Pure Python: token t of sequence b sees positions p <= L - T + t."""
    B, T, Hq, D = qs.shape
    Hkv = h.K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        L = int(h.lens[b])
        for t in range(T):
            last = L - T + t
            for hh in range(Hq):
                g = hh // G
                qv = [pins.bits_to_float(x) for x in qs[b, t, hh]]
                row = []
                for p in range(h.K.shape[1]):
                    if p <= last:
                        kv = [pins.bits_to_float(x) for x in h.K[b, p, g]]
                        row.append(math.fsum(a * c for a, c in zip(qv, kv)) / math.sqrt(D))
                    else:
                        row.append(-math.inf)
                row.append(float(h.sinks[hh]))
                m = max(row)
                e = [math.exp(x - m) for x in row]
                Z = math.fsum(e)
                for d in range(D):
                    out[b, t, hh, d] = math.fsum(e[p] * pins.bits_to_float(h.V[b, p, g, d])
                                                 for p in range(len(row) - 1)) / Z
    return out


def _sdpa(h, qs):
    """torch fp64 SDPA: keys are the history plus one sink key (zero value);
    the boolean mask admits p <= L - T + t and the sink column."""
    B, T, Hq, D = qs.shape
    Hkv = h.K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        L = int(h.lens[b])
        q = torch.from_numpy(decode_step.bf16_bits_to_f64(qs[b])).permute(1, 0, 2)   # [Hq][T][D]
        K = torch.from_numpy(decode_step.bf16_bits_to_f64(h.K[b, :L])).permute(1, 0, 2)
        V = torch.from_numpy(decode_step.bf16_bits_to_f64(h.V[b, :L])).permute(1, 0, 2)
        K = K.repeat_interleave(G, 0)
        V = V.repeat_interleave(G, 0)
        scale = 1.0 / math.sqrt(D)
        # sink key: its score must equal sigma after scaling, its value is 0
        sink_k = torch.zeros(Hq, 1, D, dtype=torch.float64)
        sink_v = torch.zeros(Hq, 1, D, dtype=torch.float64)
        K = torch.cat([K, sink_k], 1)
        V = torch.cat([V, sink_v], 1)
        allowed = torch.zeros(T, L + 1, dtype=torch.bool)
        for t in range(T):
            allowed[t, :L - T + t + 1] = True
            allowed[t, L] = True
        bias = torch.zeros(Hq, T, L + 1, dtype=torch.float64)
        bias[:, :, L] = torch.from_numpy(h.sinks.astype(np.float64))[:, None]
        bias = bias.masked_fill(~allowed, -math.inf)
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=bias, scale=scale)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


def pin_brute_force(mt):
    for seed, lens, T in ((1, [5, 9], 3), (2, [4, 17], 4), (3, [2], 2)):
        h, qs = _history(seed, len(lens), T, 4, 2, lens)
        kp, vp, bt = pins.lay_out(h, 0, 4, seed=seed)
        got = mt.decode_attention_multi(qs, kp, vp, bt, h.lens, h.sinks, 0)
        assert np.abs(got - _brute(h, qs)).max() < 1e-12, (seed, lens, T)


def pin_sdpa(mt):
    for seed, lens, T, bs in ((4, [40, 33, 2], 2, 16), (5, [70], 5, 8), (6, [31, 16], 16, 16)):
        h, qs = _history(seed, len(lens), T, 8, 2, lens)
        kp, vp, bt = pins.lay_out(h, 0, bs, seed=seed)
        got = mt.decode_attention_multi(qs, kp, vp, bt, h.lens, h.sinks, 0)
        assert np.abs(got - _sdpa(h, qs)).max() < 1e-12, (seed, lens, T)


def pin_single_token(mt):
    h, qs = _history(7, 3, 1, 8, 2, [1, 16, 33])
    kp, vp, bt = pins.lay_out(h, 0, 16, seed=7)
    got = mt.decode_attention_multi(qs, kp, vp, bt, h.lens, h.sinks, 0)
    want = decode_step.decode_attention(qs[:, 0], kp, vp, bt, h.lens, h.sinks, 0)
    assert np.array_equal(got[:, 0], want)


def pin_append(mt):
    """The tile's T rows land at positions L-T..L-1: laying out the full history
    equals laying out its first L-T positions and appending the last T."""
    lens = [6, 20, 3]
    T = 3
    h, _ = _history(8, len(lens), T, 4, 2, lens)
    kp_full, vp_full, bt = pins.lay_out(h, 0, 4, seed=8)
    short = pins.History(h.q, h.K, h.V, h.lens - T, h.sinks)
    kp, vp, bt2 = pins.lay_out(short, 0, 4, seed=8, cap_lens=h.lens)
    assert np.array_equal(bt, bt2)
    rows = np.stack([h.K[b, L - T:L] for b, L in enumerate(lens)])
    vrows = np.stack([h.V[b, L - T:L] for b, L in enumerate(lens)])
    k2, v2 = mt.kv_append_multi(kp, vp, rows, vrows, bt, h.lens, 0)
    assert np.array_equal(k2, kp_full) and np.array_equal(v2, vp_full)


def pin_rejects_ring(mt):
    h, qs = _history(9, 1, 2, 4, 2, [10])
    kp, vp, bt = pins.lay_out(h, 8, 4, seed=9)
    try:
        mt.decode_attention_multi(qs, kp, vp, bt, h.lens, h.sinks, 8)
    except ValueError:
        return
    raise AssertionError("a ring layer with two query tokens was accepted")


ALL = [pin_brute_force, pin_sdpa, pin_single_token, pin_append, pin_rejects_ring]
