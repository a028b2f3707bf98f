"""Seeded random configurations against the oracle: batch, heads per group,
block size, window, ragged lengths (empty sequences included), spare table
capacity, split count and kernel variant are drawn per case; attention is
checked to the parity bar and the fused append's pools bit for bit.  The
cases are fixed by their seeds, so a failure names a reproducible shape."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, out_f64, sub_layer

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(10_000 + seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    bs = int(rng.choice([8, 16, 32, 64]))
    B = int(rng.integers(1, 41))
    window = int(rng.choice([0, 0, 0, int(rng.integers(1, 300))]))
    lmax = int(rng.choice([40, 700, 3000]))
    lens = rng.integers(0, lmax + 1, size=B)
    lens[rng.random(B) < 0.1] = 0
    cap = lens + rng.integers(0, 3 * bs, size=B)
    variant = int(rng.choice([0, 1, 2, 4, 5]))
    splits = int(rng.choice([0, 0, int(rng.integers(1, 20))]))
    return dict(hkv=hkv, G=G, bs=bs, B=B, window=window, lens=lens, cap=cap,
                variant=variant, splits=splits)


@pytest.mark.parametrize("seed", range(100))
def test_random_configuration(lib, seed):
    c = draw(seed)
    layer = synth.make_layer(batch=c["B"], q_heads=c["hkv"] * c["G"], kv_heads=c["hkv"],
                             head_dim=64, block_size=c["bs"], lens=c["lens"].tolist(),
                             capacity=c["cap"].tolist(), window=c["window"],
                             seed=20_000 + seed, device="cuda")
    W = c["window"]
    tag = f"seed {seed}: {c}"
    s = sub_layer(layer, range(layer.batch))
    ref = oracle.decode_attention(s["q"], s["k"], s["v"], s["bt"], s["lens"], s["sinks"], W)
    out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                               layer.seq_lens, layer.sinks, W, num_splits=c["splits"],
                               variant=c["variant"])
    torch.cuda.synchronize()
    assert_parity(out_f64(out), ref, tag)
    # the fused step: the append inside the attention launch
    k_ref, v_ref = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"], s["lens"], W)
    ref2 = oracle.decode_attention(s["q"], k_ref, v_ref, s["bt"], s["lens"], s["sinks"], W)
    out2 = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, layer.k_cache,
                                       layer.v_cache, layer.block_table, layer.seq_lens,
                                       layer.sinks, W, num_splits=c["splits"],
                                       variant=c["variant"])
    torch.cuda.synchronize()
    after = sub_layer(layer, range(layer.batch))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref), tag
    assert_parity(out_f64(out2), ref2, tag + " (fused)")


@pytest.mark.parametrize("seed", range(20))
def test_random_query_tile(lib, seed):
    """T causal query tokens per sequence (T*G <= 16), paged layers, the fused
    append of the tile's rows included."""
    import test_gpu_multi as tm
    rng = np.random.default_rng(30_000 + seed)
    T = int(rng.choice([2, 3, 4, 8, 16]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if T * g <= 16]))
    hkv = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([8, 16, 32, 64]))
    B = int(rng.integers(1, 25))
    lens = np.maximum(rng.integers(0, 2500, size=B), T)
    variant = int(rng.choice([0, 1, 2, 4, 5]))
    splits = int(rng.choice([0, 0, int(rng.integers(1, 12))]))
    tag = f"seed {seed}: T={T} G={G} hkv={hkv} bs={bs} B={B} v={variant} S={splits}"
    layer, q, kn, vn = tm.tile_layer(lens.tolist(), T, hkv * G, hkv, seed=40_000 + seed, bs=bs)
    s = sub_layer(layer, range(B))
    k_ref, v_ref = oracle.multi_token.kv_append_multi(s["k"], s["v"], bits(kn), bits(vn), s["bt"],
                                                      s["lens"], 0)
    ref = oracle.multi_token.decode_attention_multi(bits(q), k_ref, v_ref, s["bt"], s["lens"],
                                                    s["sinks"], 0)
    out = lib.decode_attention_append(q, kn, vn, layer.k_cache, layer.v_cache, layer.block_table,
                                      layer.seq_lens, layer.sinks, 0, num_splits=splits,
                                      variant=variant)
    torch.cuda.synchronize()
    after = sub_layer(layer, range(B))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref), tag
    assert_parity(out_f64(out), ref, tag)


@pytest.mark.parametrize("seed", range(20))
def test_random_rope_step(lib, seed):
    """The step with the rotary embedding fused in: either pairing, paged or
    ring, positions past the tables' end included."""
    import test_gpu_rope as tr
    rng = np.random.default_rng(50_000 + seed)
    style = str(rng.choice(["half", "interleaved"]))
    hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8, 16]))
    bs = int(rng.choice([8, 16, 32, 64]))
    B = int(rng.integers(1, 25))
    window = int(rng.choice([0, 0, int(rng.integers(1, 200))]))
    lens = rng.integers(1, 2000, size=B)
    P = int(rng.choice([64, 4096]))            # rows of the angle tables
    variant = int(rng.choice([0, 1, 2, 4, 5]))
    splits = int(rng.choice([0, 0, int(rng.integers(1, 12))]))
    tag = f"seed {seed}: {style} hkv={hkv} G={G} bs={bs} B={B} W={window} P={P} v={variant}"
    layer = synth.make_layer(batch=B, q_heads=hkv * G, kv_heads=hkv, head_dim=64, block_size=bs,
                             lens=lens.tolist(), window=window, seed=60_000 + seed,
                             device="cuda")
    cos_t, sin_t = tr.angle_tables(P)
    s, (k_ref, v_ref, out_ref) = tr.oracle_step(layer, cos_t, sin_t, style, compact=True)
    out = tr.run_rope(lib, layer, layer.k_cache, layer.v_cache, cos_t, sin_t, style, splits,
                      variant)
    after = sub_layer(layer, range(B))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref), tag
    assert_parity(out_f64(out), out_ref, tag)
