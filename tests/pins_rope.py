"""Pins of the RoPE oracle (oracle/rope.py) against facts it does not compute
itself: exact special angles, the complex-number form of the rotation, the
relative-position property of rotary embeddings, torch's bf16 rounding, and
closed forms of the decode step at the new token's position.

Each pin takes the module so that the planted-mistake tests can hand it a
mutated one.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import decode_step

STYLES = ("half", "interleaved")


def _bf16_bits(rng, shape, scale=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _widen(bits):
    return decode_step.bf16_bits_to_f64(bits)


def _split_pairs(x, style):
    """The pairs of the last axis, written with slices (not index arrays)."""
    D = x.shape[-1]
    if style == "half":
        return x[..., : D // 2], x[..., D // 2:]
    return x[..., 0::2], x[..., 1::2]


def _join_pairs(a, b, style):
    if style == "half":
        return np.concatenate([a, b], axis=-1)
    out = np.empty(a.shape[:-1] + (2 * a.shape[-1],), dtype=a.dtype)
    out[..., 0::2], out[..., 1::2] = a, b
    return out


def _angle_tables(P, D, base=10000.0):
    """Standard rotary angles a_i(p) = p * base^(-2i/D), as float32 tables."""
    inv = base ** (-np.arange(D // 2, dtype=np.float64) * 2.0 / D)
    ang = np.arange(P, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def pin_special_angles(rope):
    """Angle 0 keeps every bit; a quarter turn maps (x1, x2) to (-x2, x1)
    exactly (negation only flips a sign bit)."""
    rng = np.random.default_rng(11)
    x = _bf16_bits(rng, (3, 5, 64))
    ones, zeros = np.ones((4, 32), np.float32), np.zeros((4, 32), np.float32)
    for style in STYLES:
        assert np.array_equal(rope.rope_bf16(x, 2, ones, zeros, style), x)
        got = rope.rope_bf16(x, 1, zeros, ones, style)
        x1, x2 = _split_pairs(x, style)
        want = _join_pairs(x2 ^ np.uint16(0x8000), x1, style)
        assert np.array_equal(got, want), style


def pin_complex_form(rope):
    """Pair (x1, x2) as z = x1 + i x2 turned by e^{ia}: the complex product in
    complex128, rounded to bf16, agrees with the oracle to one bf16 step, and
    exactly for nearly every element."""
    rng = np.random.default_rng(12)
    x = _bf16_bits(rng, (4, 8, 64))
    a = rng.uniform(-np.pi, np.pi, (16, 32))
    c, s = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    pos = np.array([3, 0, 15, 7])[:, None]
    for style in STYLES:
        x1, x2 = _split_pairs(_widen(x), style)
        z = (x1 + 1j * x2) * (c[pos].astype(np.float64) + 1j * s[pos].astype(np.float64))
        y = _join_pairs(z.real, z.imag, style)
        want = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = rope.rope_bf16(x, pos, c, s, style)
        diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
        assert diff.max() <= 1, style
        assert (diff == 0).mean() > 0.97, style


def pin_relative_position(rope):
    """With the standard angle tables, <R_p q, R_k k> depends only on p - k
    (the property rotary embeddings exist for); this fails for any pairing
    that differs between the two rotations or any wrong sign."""
    rng = np.random.default_rng(13)
    D = 64
    cos_t, sin_t = _angle_tables(64, D)
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    for style in STYLES:
        def rot(v, p):
            return rope.rotate_f32(v, cos_t[p], sin_t[p], style).astype(np.float64)
        base = float(np.dot(rot(q, 20), rot(k, 7)))
        for p, kp in ((33, 20), (13, 0), (50, 37)):
            assert abs(float(np.dot(rot(q, p), rot(k, kp))) - base) < 1e-4 * (1 + abs(base))
        # and it does change with the distance
        assert abs(float(np.dot(rot(q, 21), rot(k, 7))) - base) > 1e-3


def pin_rounding(rope):
    """float32 -> bf16 rounding equals torch's (round to nearest, ties to even),
    ties included."""
    rng = np.random.default_rng(14)
    x = (rng.standard_normal(4096) * 10).astype(np.float32)
    ties = (np.arange(1, 257, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    for v in (x, ties, -ties):
        want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(rope.f32_to_bf16_bits(v), want)


def _tiny_layer(rng, lens, window=0, bs=16, hq=8, hkv=2):
    B = len(lens)
    cap = max(max(lens), window if window > 0 else 0, 1)
    mbs = -(-cap // bs)
    nb = B * mbs + 1
    k = _bf16_bits(rng, (nb, hkv, 2, bs, 32))          # K rows in two halves
    v = _bf16_bits(rng, (nb, hkv, bs // 8, 64, 8))     # V in chunks of 8 slots
    perm = rng.permutation(B * mbs).reshape(B, mbs).astype(np.int32)
    return dict(q=_bf16_bits(rng, (B, hq, 64)), k=k, v=v,
                kn=_bf16_bits(rng, (B, hkv, 64)), vn=_bf16_bits(rng, (B, hkv, 64)),
                bt=perm, lens=np.asarray(lens), sinks=rng.standard_normal(hq))


def pin_step_at_last_position(rope):
    """Tables that turn only row L-1 (a quarter turn) and leave every other row
    alone: the cache gains exactly the quarter-turned new key, V unturned, and
    the output equals plain attention with the quarter-turned query."""
    rng = np.random.default_rng(15)
    for style in STYLES:
        for window in (0, 8):
            lens = [5, 12]
            t = _tiny_layer(rng, lens, window)
            P = 16
            for b, L in enumerate(lens):
                cos_t = np.ones((P, 32), np.float32)
                sin_t = np.zeros((P, 32), np.float32)
                cos_t[L - 1], sin_t[L - 1] = 0.0, 1.0
                one = {key: (val[b:b + 1] if key in ("q", "kn", "vn", "bt", "lens") else val)
                       for key, val in t.items()}
                k2, v2, out = rope.decode_step_rope(one["q"], one["k"], one["v"], one["kn"],
                                                    one["vn"], one["bt"], one["lens"],
                                                    one["sinks"], window, cos_t, sin_t, style)
                def turn(bits):                 # (x1, x2) -> (-x2, x1)
                    x1, x2 = _split_pairs(bits, style)
                    return _join_pairs(x2 ^ np.uint16(0x8000), x1, style)
                ke, ve = decode_step.kv_append(one["k"], one["v"], turn(one["kn"]), one["vn"],
                                               one["bt"], one["lens"], window)
                assert np.array_equal(k2, ke) and np.array_equal(v2, ve), (style, window, b)
                want = decode_step.decode_attention(turn(one["q"]), ke, ve, one["bt"],
                                                    one["lens"], one["sinks"], window)
                assert np.allclose(out, want, rtol=0, atol=1e-12), (style, window, b)


def pin_zero_angle_step(rope):
    """All-zero angles: the step is exactly the plain append then attention."""
    rng = np.random.default_rng(16)
    t = _tiny_layer(rng, [1, 9, 30])
    ones, zeros = np.ones((40, 32), np.float32), np.zeros((40, 32), np.float32)
    for style in STYLES:
        k2, v2, out = rope.decode_step_rope(t["q"], t["k"], t["v"], t["kn"], t["vn"], t["bt"],
                                            t["lens"], t["sinks"], 0, ones, zeros, style)
        ke, ve = decode_step.kv_append(t["k"], t["v"], t["kn"], t["vn"], t["bt"], t["lens"], 0)
        assert np.array_equal(k2, ke) and np.array_equal(v2, ve)
        want = decode_step.decode_attention(t["q"], ke, ve, t["bt"], t["lens"], t["sinks"], 0)
        assert np.array_equal(out, want)


def pin_table_end(rope):
    """A position past the table's last row uses that row."""
    rng = np.random.default_rng(17)
    x = _bf16_bits(rng, (2, 64))
    a = rng.uniform(-3, 3, (6, 32))
    c, s = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    for style in STYLES:
        assert np.array_equal(rope.rope_bf16(x, 40, c, s, style),
                              rope.rope_bf16(x, 5, c, s, style))


def pin_float32_steps(rope):
    """The bf16 bits follow the stated precision: every product and sum in
    float32 on its own, then nearest-even bf16.  torch's float32 elementwise
    kernels and its bf16 conversion, applied step by step, give the same bits
    on a sample large enough that a single rounding of the exact value (or a
    fused multiply-add) would differ somewhere."""
    rng = np.random.default_rng(18)
    x = _bf16_bits(rng, (64, 16, 64), scale=3.0)
    a = rng.uniform(-np.pi, np.pi, (64, 32))
    c, s = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    pos = np.arange(64)[:, None]
    xt = torch.from_numpy(_widen(x).astype(np.float32))
    ct, st = torch.from_numpy(c[pos]), torch.from_numpy(s[pos])
    for style in STYLES:
        x1, x2 = _split_pairs(xt, style)
        y1 = torch.sub(torch.mul(x1, ct), torch.mul(x2, st))
        y2 = torch.add(torch.mul(x2, ct), torch.mul(x1, st))
        y = torch.cat([y1, y2], -1) if style == "half" else torch.stack([y1, y2], -1).flatten(-2)
        want = y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(rope.rope_bf16(x, pos, c, s, style), want), style


ALL = [pin_special_angles, pin_complex_form, pin_relative_position, pin_rounding,
       pin_step_at_last_position, pin_zero_angle_step, pin_table_end, pin_float32_steps]
