"""KV append on the GPU: bit-exact against the oracle's append, nothing else
in either pool changes (paged and ring layers, several block sizes)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
@pytest.mark.parametrize("window", [0, 128, 100, 7])
def test_append_bit_exact(lib, bs, window):
    lens = [1, 2, bs - 1, bs, bs + 1, 3 * bs + 5, 129, 400]
    layer = synth.make_layer(batch=len(lens), q_heads=16, kv_heads=4, head_dim=64,
                             block_size=bs, lens=lens, window=window,
                             seed=100 + bs + window, device="cuda", guard_blocks=3)
    k0, v0 = bits(layer.k_cache), bits(layer.v_cache)
    lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
                  layer.block_table, layer.seq_lens, window)
    torch.cuda.synchronize()
    kr, vr = oracle.kv_append(k0, v0, bits(layer.k_new), bits(layer.v_new),
                              bits(layer.block_table), bits(layer.seq_lens), window)
    assert np.array_equal(bits(layer.k_cache), kr)
    assert np.array_equal(bits(layer.v_cache), vr)
    # and something did change (the append is not a no-op)
    assert not np.array_equal(kr, k0)


def test_append_skips_empty_sequences(lib):
    layer = synth.make_layer(batch=3, q_heads=8, kv_heads=2, head_dim=64, block_size=16,
                             lens=[5, 9, 17], seed=7, device="cuda")
    layer.seq_lens[1] = 0
    k0 = bits(layer.k_cache)
    lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
                  layer.block_table, layer.seq_lens, 0)
    torch.cuda.synchronize()
    kr, _ = oracle.kv_append(k0, bits(layer.v_cache), bits(layer.k_new), bits(layer.v_new),
                             bits(layer.block_table), bits(layer.seq_lens), 0)
    assert np.array_equal(bits(layer.k_cache), kr)


def test_append_then_attend_sees_new_token(lib):
    """A query equal to a large multiple of the new key attends to it alone."""
    layer = synth.make_layer(batch=2, q_heads=8, kv_heads=2, head_dim=64, block_size=16,
                             lens=[20, 33], seed=8, device="cuda", sinks=False)
    lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
                  layer.block_table, layer.seq_lens, 0)
    q = (layer.k_new.float().repeat_interleave(4, dim=1) * 8.0).to(torch.bfloat16)
    out = lib.decode_attention(q, layer.k_cache, layer.v_cache, layer.block_table,
                               layer.seq_lens, None, 0)
    torch.cuda.synchronize()
    want = layer.v_new.float().repeat_interleave(4, dim=1)
    assert torch.allclose(out.float(), want, atol=2e-2)
