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
    variant = int(rng.choice([0, 1, 2, 4]))
    splits = int(rng.choice([0, 0, int(rng.integers(1, 20))]))
    return dict(hkv=hkv, G=G, bs=bs, B=B, window=window, lens=lens, cap=cap,
                variant=variant, splits=splits)


@pytest.mark.parametrize("seed", range(24))
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
