"""Pins of the RoPE oracle (CPU), and planted mistakes they must catch."""

import numpy as np
import pytest

from oracle import rope
import pins_rope


@pytest.mark.parametrize("pin", pins_rope.ALL, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(rope)


def _mutations():
    orig_rotate = rope.rotate_f32
    orig_pairs = rope.pair_dims
    orig_step = rope.decode_step_rope
    orig_rope = rope.rope_bf16

    def sign_flipped(x, c, s, style):           # turns the other way
        return orig_rotate(x, c, -np.asarray(s, np.float32), style)

    def pairing_swapped(D, style):              # half and interleaved exchanged
        return orig_pairs(D, "interleaved" if style == "half" else "half")

    def fused_rounding(x, c, s, style):         # products summed in float64, rounded once
        x = np.asarray(x, np.float64)
        d1, d2 = orig_pairs(x.shape[-1], style)
        c, s = np.asarray(c, np.float64), np.asarray(s, np.float64)
        y = np.empty_like(x)
        y[..., d1] = x[..., d1] * c - x[..., d2] * s
        y[..., d2] = x[..., d2] * c + x[..., d1] * s
        return y.astype(np.float32)

    def position_is_length(q, kc, vc, kn, vn, bt, lens, sinks, w, ct, st, style):
        return orig_step(q, kc, vc, kn, vn, bt, np.asarray(lens), sinks, w,
                         np.roll(ct, -1, axis=0), np.roll(st, -1, axis=0), style)

    def query_not_rotated(q, kc, vc, kn, vn, bt, lens, sinks, w, ct, st, style):
        k2, v2, _ = orig_step(q, kc, vc, kn, vn, bt, lens, sinks, w, ct, st, style)
        from oracle import decode_step
        return k2, v2, decode_step.decode_attention(q, k2, v2, bt, lens, sinks, w)

    def truncating_round(x, pos, ct, st, style):    # bf16 by truncation, not nearest
        x32 = rope.rotate_f32(rope._ds.bf16_bits_to_f64(np.asarray(x, np.uint16)).astype(np.float32),
                              rope.table_rows(ct, pos), rope.table_rows(st, pos), style)
        return (x32.view(np.uint32) >> 16).astype(np.uint16)

    return [("rotate_f32", sign_flipped), ("pair_dims", pairing_swapped),
            ("rotate_f32", fused_rounding), ("decode_step_rope", position_is_length),
            ("decode_step_rope", query_not_rotated), ("rope_bf16", truncating_round)]


@pytest.mark.parametrize("name,fn", _mutations(), ids=lambda x: getattr(x, "__name__", str(x)))
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(rope, name, fn)
    failed = []
    for pin in pins_rope.ALL:
        try:
            pin(rope)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake in {name}"
