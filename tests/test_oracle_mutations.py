"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each test swaps one piece of the oracle for a plausible wrong version and
checks that at least one pin fails; then the original is restored.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import decode_step
import pins

ALL_PINS = [pins.pin_brute_force, pins.pin_sdpa, pins.pin_closed_forms,
            pins.pin_invariants, pins.pin_combine, pins.pin_append,
            pins.pin_append_past_capacity]


def _some_pin_fails(monkeypatch_ctx):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(decode_step)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


def _mutations():
    orig_group = decode_step.query_group
    orig_slot = decode_step.storage_slot
    orig_sink = decode_step._sink
    orig_gather = decode_step._gather
    orig_positions = decode_step.attended_positions
    orig_locate = decode_step.locate
    orig_append = decode_step.kv_append

    def group_modulo(h, hq, hkv):                 # interleaved instead of contiguous groups
        return h % hkv

    def slot_off_by_one(p, w):                    # ring slot shifted by one
        return p if w <= 0 else (p + 1) % w

    def sink_dropped(sinks, h):                   # sink left out of the denominator
        return -math.inf

    def sink_doubled(sinks, h):                   # sink scaled like a score
        v = orig_sink(sinks, h)
        return v * 2.0

    def v_untransposed(k_cache, v_cache, block_table, b, g, positions, window):
        K, V = orig_gather(k_cache, v_cache, block_table, b, g, positions, window)
        return K, K.copy()                        # reads V from the K pool

    def window_excludes_current(L, w):            # window ends one position early
        return orig_positions(L, w) if w <= 0 else range(max(0, L - w - 1), L - 1)

    def offset_from_block_start(block_table, b, slot, bs):   # offset dropped
        blk, off = orig_locate(block_table, b, slot, bs)
        return blk, off * 0

    def append_clamped_to_capacity(k_cache, v_cache, k_new, v_new, block_table, seq_lens, w):
        # a slot past the table row written to the row's last slot instead of skipped
        cap = np.asarray(block_table).shape[1] * k_cache.shape[3]
        lens = [min(int(L), cap) if w <= 0 else int(L) for L in seq_lens]
        return orig_append(k_cache, v_cache, k_new, v_new, block_table, lens, w)

    return [
        ("query_group", group_modulo),
        ("storage_slot", slot_off_by_one),
        ("_sink", sink_dropped),
        ("_sink", sink_doubled),
        ("_gather", v_untransposed),
        ("attended_positions", window_excludes_current),
        ("locate", offset_from_block_start),
        ("kv_append", append_clamped_to_capacity),
    ]


@pytest.mark.parametrize("name,fn", _mutations(), ids=lambda x: getattr(x, "__name__", str(x)))
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(decode_step, name, fn)
    failed = _some_pin_fails(monkeypatch)
    assert failed, f"no pin caught the planted mistake in {name}"


def test_unmutated_oracle_passes_all_pins():
    assert _some_pin_fails(None) == []
