"""The oracle against routes that do not go through it (CPU only).

Brute force, torch fp64 SDPA, closed forms, invariants, split/combine and the
append are in ``pins.py``; the hand-derived example is in
``golden/hand_example.json``.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def test_brute_force():
    pins.pin_brute_force(oracle)


def test_sdpa_library_route():
    pins.pin_sdpa(oracle)


def test_closed_forms():
    pins.pin_closed_forms(oracle)


def test_invariants():
    pins.pin_invariants(oracle)


def test_combine_partition_invariance():
    pins.pin_combine(oracle)


def test_append_matches_history_layout():
    pins.pin_append(oracle)


def test_append_past_capacity_writes_nothing():
    pins.pin_append_past_capacity(oracle)


def _k_rows(a):
    """The fixture's K pool [blk][kvh][slot][d] in the documented piece layout
    [blk][kvh][n][bs][D/n] with n = 1 (a row in one piece): an axis of size 1
    is added."""
    return np.asarray(a)[:, :, None]


def _v_chunked(a):
    """The fixture's V pool [blk][kvh][d][slot] as the library's chunked layout
    [blk][kvh][bs/c][d][c]: at the fixture's block size (2, below the chunk of
    8) one chunk holds the whole block, so only an axis of size 1 is added."""
    return np.asarray(a)[:, :, None]


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("layer", ["full", "ring"])
def test_hand_example_attention(layer):
    g = _golden()
    c = g[layer]
    W = c.get("window", 0)
    q = np.array(g["q"], dtype=np.float64)
    out = oracle.decode_attention(q, _k_rows(np.array(c["k_pool_after"], dtype=np.float64)),
                                  _v_chunked(np.array(c["v_pool_after"], dtype=np.float64)),
                                  np.array(c["block_table"]), np.array(c["seq_lens"]),
                                  np.array(g["sinks"]), W)
    np.testing.assert_allclose(out, np.array(c["expected_out"]), rtol=0, atol=1e-12)
    if "expected_out_no_sinks" in c:
        out = oracle.decode_attention(q, _k_rows(np.array(c["k_pool_after"], dtype=np.float64)),
                                      _v_chunked(np.array(c["v_pool_after"], dtype=np.float64)),
                                      np.array(c["block_table"]), np.array(c["seq_lens"]),
                                      None, W)
        np.testing.assert_allclose(out, np.array(c["expected_out_no_sinks"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("layer", ["full", "ring"])
def test_hand_example_append(layer):
    g = _golden()
    c = g[layer]
    k, v = oracle.kv_append(_k_rows(c["k_pool_before"]), _v_chunked(c["v_pool_before"]),
                            np.array(c["k_new"]), np.array(c["v_new"]),
                            np.array(c["block_table"]), np.array(c["seq_lens"]),
                            c.get("window", 0))
    assert np.array_equal(k, _k_rows(c["k_pool_after"]))
    assert np.array_equal(v, _v_chunked(c["v_pool_after"]))


def test_bf16_widening_exact():
    # 1.0, -2.0, 0.15625, the largest finite bf16, the smallest subnormal, -0
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x7F7F, 0x0001, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 0.15625, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, -0.0]
    got = oracle.bf16_bits_to_f64(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[-1]) == -1.0


def test_empty_context_and_no_sink_gives_zero():
    q = np.ones((1, 2, 4))
    kp = np.ones((2, 1, 2, 2, 2))                   # [blk][kvh][half][slot][d % 2]
    vp = np.ones((2, 1, 1, 4, 2))                   # [blk][kvh][chunk][d][slot]
    out = oracle.decode_attention(q, kp, vp, np.array([[0]]), np.array([0]), None, 0)
    assert np.array_equal(out, np.zeros((1, 2, 4)))
    # a finite sink with no positions also gives 0 (the sink has no value row)
    out = oracle.decode_attention(q, kp, vp, np.array([[0]]), np.array([0]), np.zeros(2), 0)
    assert np.array_equal(out, np.zeros((1, 2, 4)))


def test_pool_layout_as_documented():
    """The oracle reads K at [blk][g][d // 32][s % bs][d % 32] and V at
    [blk][g][s % bs // 8][d][s % 8] (the layouts the C header documents),
    through the block table: a pool whose every element encodes its own
    (block, head, slot, dim) comes back row by row."""
    from oracle import decode_step
    NB, Hkv, bs, D = 5, 2, 16, 64
    k = np.zeros((NB, Hkv, 2, bs, D // 2))
    v = np.zeros((NB, Hkv, bs // 8, D, 8))
    for blk in range(NB):
        for g in range(Hkv):
            for s in range(bs):
                for d in range(D):
                    code = blk * 1e6 + g * 1e5 + s * 1e3 + d
                    k[blk, g, d // 32, s, d % 32] = code
                    v[blk, g, s // 8, d, s % 8] = -code
    table = np.array([[3, 0, 4]])
    positions = [0, 7, 8, 15, 16, 33, 47]
    for g in range(Hkv):
        K, V = decode_step._gather(k, v, table, 0, g, positions, 0)
        for i, p in enumerate(positions):
            blk, s = table[0, p // bs], p % bs
            want = blk * 1e6 + g * 1e5 + s * 1e3 + np.arange(D)
            assert np.array_equal(K[i], want) and np.array_equal(V[i], -want), (g, p)
