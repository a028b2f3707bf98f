"""Several causal query tokens per sequence (a query tile) on the GPU.

Token t of a tile sits at position L-T+t and attends up to itself.  Against
the multi-token oracle: attention over an existing cache, the fused step that
appends the tile's T rows first (pools bit for bit), the standalone append,
the split partials with their merge, for every MFMA variant and split count,
and tiles that fill the 16 MFMA columns in three ways (2 tokens x 8 heads,
4 x 4, 16 x 1)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, out_f64, sub_layer

pytestmark = pytest.mark.gpu

MFMA_VARIANTS = [0, 1, 2, 4, 5]


def tile_layer(lens, T, q_heads, kv_heads, seed, bs=16, capacity=None):
    """A synthetic layer plus a tile of T query tokens and T new K/V rows per
    sequence (seq_lens = L counts the tile)."""
    layer = synth.make_layer(batch=len(lens), q_heads=q_heads, kv_heads=kv_heads, head_dim=64,
                             block_size=bs, lens=lens, capacity=capacity, seed=seed,
                             device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    B = len(lens)
    q = torch.randn(B, T, q_heads, 64, generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn(B, T, kv_heads, 64, generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn(B, T, kv_heads, 64, generator=g, device="cuda").to(torch.bfloat16)
    return layer, q, kn, vn


def host(layer):
    return dict(k=bits(layer.k_cache), v=bits(layer.v_cache), bt=bits(layer.block_table),
                lens=bits(layer.seq_lens), sinks=layer.sinks.cpu().numpy())


@pytest.mark.parametrize("T,hq,hkv", [(2, 32, 4), (4, 16, 4), (16, 4, 4)])
def test_tile_attention_over_the_cache(lib, T, hq, hkv):
    lens = [T, T + 1, 31, 32, 33, 700, 3001]
    layer, q, _, _ = tile_layer(lens, T, hq, hkv, seed=8000 + T)
    h = host(layer)
    ref = oracle.multi_token.decode_attention_multi(bits(q), h["k"], h["v"], h["bt"], h["lens"],
                                                    h["sinks"], 0)
    for v in MFMA_VARIANTS:
        for S in (0, 1, 3):
            out = lib.decode_attention(q, layer.k_cache, layer.v_cache, layer.block_table,
                                       layer.seq_lens, layer.sinks, 0, num_splits=S, variant=v)
            torch.cuda.synchronize()
            assert out.shape == q.shape
            assert_parity(out_f64(out), ref, f"T={T} G={hq // hkv} S={S} v={v}")


@pytest.mark.parametrize("T,hq,hkv", [(2, 16, 2), (4, 8, 2)])
@pytest.mark.parametrize("bs", [8, 16, 64])
def test_tile_fused_append(lib, T, hq, hkv, bs):
    """The tile's rows are appended at L-T..L-1 inside the launch (the rows may
    straddle blocks and wavefronts), then attended causally."""
    lens = [T, bs - 1, bs, bs + T - 1, 2 * bs + 1, 1000]
    lens = [max(L, T) for L in lens]
    layer, q, kn, vn = tile_layer(lens, T, hq, hkv, seed=8100 + bs + T, bs=bs)
    h = host(layer)
    k_ref, v_ref = oracle.multi_token.kv_append_multi(h["k"], h["v"], bits(kn), bits(vn), h["bt"],
                                                      h["lens"], 0)
    ref = oracle.multi_token.decode_attention_multi(bits(q), k_ref, v_ref, h["bt"], h["lens"],
                                                    h["sinks"], 0)
    for v in MFMA_VARIANTS:
        for S in (0, 1, 3):
            kc, vc = layer.k_cache.clone(), layer.v_cache.clone()
            out = lib.decode_attention_append(q, kn, vn, kc, vc, layer.block_table,
                                              layer.seq_lens, layer.sinks, 0, num_splits=S,
                                              variant=v)
            torch.cuda.synchronize()
            tag = f"T={T} bs={bs} S={S} v={v}"
            assert np.array_equal(bits(kc), k_ref), f"{tag}: K pool"
            assert np.array_equal(bits(vc), v_ref), f"{tag}: V pool"
            assert_parity(out_f64(out), ref, tag)
    # the standalone append writes the same rows
    kc, vc = layer.k_cache.clone(), layer.v_cache.clone()
    lib.kv_append(kn, vn, kc, vc, layer.block_table, layer.seq_lens, 0)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), k_ref) and np.array_equal(bits(vc), v_ref)


def test_tile_partials_and_merge(lib):
    T = 2
    layer, q, _, _ = tile_layer([5000, 17, 2], T, 16, 2, seed=8200)
    h = host(layer)
    ref = oracle.multi_token.decode_attention_multi(bits(q), h["k"], h["v"], h["bt"], h["lens"],
                                                    h["sinks"], 0)
    po, pl = lib.decode_partials(q, layer.k_cache, layer.v_cache, layer.block_table,
                                 layer.seq_lens, 0, num_splits=8)
    out = lib.combine(po, pl, layer.sinks)
    torch.cuda.synchronize()
    assert out.shape == q.shape
    assert_parity(out_f64(out), ref, "partials + merge")


def test_tile_ragged_batch64(lib):
    """Batch 64, ragged 513..8193, 2 tokens x 8 heads (the full 16 columns), the
    default launch with the append inside: every sequence, pools bit for bit."""
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 2
    layer, q, kn, vn = tile_layer(lens.tolist(), 2, 64, 8, seed=c["seed"] + 60)
    s = sub_layer(layer, range(64))
    k_ref, v_ref = oracle.multi_token.kv_append_multi(s["k"], s["v"], bits(kn), bits(vn), s["bt"],
                                                      s["lens"], 0)
    ref = oracle.multi_token.decode_attention_multi(bits(q), k_ref, v_ref, s["bt"], s["lens"],
                                                    s["sinks"], 0)
    out = lib.decode_attention_append(q, kn, vn, layer.k_cache, layer.v_cache, layer.block_table,
                                      layer.seq_lens, layer.sinks, 0)
    torch.cuda.synchronize()
    after = sub_layer(layer, range(64))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref)
    assert_parity(out_f64(out), ref, "ragged tile")
