"""The seeded generators: deterministic, shaped as documented (CPU only)."""

import hashlib

import numpy as np
import torch

import synth


def _digest(layer):
    h = hashlib.sha256()
    for t in (layer.q, layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
              layer.block_table, layer.seq_lens, layer.sinks):
        h.update(synth.to_bits(t).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes_other_seed_differs():
    kw = dict(batch=3, q_heads=8, kv_heads=2, head_dim=64, block_size=16, lens=[5, 40, 17])
    a = synth.make_layer(seed=7, **kw)
    b = synth.make_layer(seed=7, **kw)
    c = synth.make_layer(seed=8, **kw)
    assert _digest(a) == _digest(b)
    assert _digest(a) != _digest(c)


def test_shapes_tables_and_poison():
    L = [1, 16, 17, 100]
    lay = synth.make_layer(batch=4, q_heads=8, kv_heads=2, head_dim=64, block_size=16,
                           lens=L, seed=3)
    assert lay.k_cache.shape == (lay.num_blocks, 2, 2, 16, 32)    # [NB][Hkv][2][bs][D/2]
    assert lay.v_cache.shape == (lay.num_blocks, 2, 2, 64, 8)      # [NB][Hkv][bs/8][D][8]
    assert lay.k_cache.dtype == torch.bfloat16 and lay.sinks.dtype == torch.float32
    assert lay.blocks_per_seq == [1, 1, 2, 7]
    bt = lay.block_table.numpy()
    owned = np.concatenate([bt[b, :n] for b, n in enumerate(lay.blocks_per_seq)])
    assert len(set(owned.tolist())) == len(owned)            # no block shared
    assert lay.poison_block not in set(owned.tolist())
    for b, n in enumerate(lay.blocks_per_seq):
        assert (bt[b, n:] == lay.poison_block).all()
    assert (lay.k_cache[lay.poison_block].float() == 64.0).all()


def test_ring_layer_blocks():
    lay = synth.make_layer(batch=2, q_heads=8, kv_heads=2, head_dim=64, block_size=16,
                           lens=[5, 500], window=128, seed=4)
    assert lay.blocks_per_seq == [8, 8]
    assert lay.window == 128


def test_identity_table_is_contiguous():
    lay = synth.make_layer(batch=2, q_heads=4, kv_heads=1, head_dim=64, block_size=16,
                           lens=[40, 20], seed=5, table="identity")
    assert lay.block_table[0, :3].tolist() == [0, 1, 2]
    assert lay.block_table[1, :2].tolist() == [3, 4]


def test_ragged_lengths_range():
    x = synth.ragged_lengths(1, 1000, 512, 8192)
    assert x.min() >= 512 and x.max() <= 8192
    assert (x == synth.ragged_lengths(1, 1000, 512, 8192)).all()
