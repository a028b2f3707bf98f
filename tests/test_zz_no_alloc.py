"""sa_decode_attention_append_noalloc (the fused decode step with the
library's own per-GPU scratch instead of a caller's workspace) against
sa_decode_attention_append on the same inputs, through the C ABI: outputs and
pools bit-identical, for two calls in a row with the second on a smaller
input (the scratch keeps the first call's contents), over every way a call
uses the scratch: the balanced kernel and its merge, a static split and its
combine, the fused last-partition combine and its counters, and a call that
needs no scratch at all."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def layer_pair(**kw):
    """Two identical copies of one layer's inputs (each path appends into its
    own pools)."""
    a = synth.make_layer(device="cuda", **kw)
    b = synth.make_layer(device="cuda", **kw)
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.v_cache, b.v_cache)
    return a, b


CASES = {
    # balanced kernel + merge: batch 64 ragged, then batch 16 shorter
    "balanced": (dict(batch=64, lens=synth.ragged_lengths(71, 64, 513, 8193)),
                 dict(batch=16, lens=synth.ragged_lengths(72, 16, 1, 3000))),
    # one partition per unit (the ring layer): no scratch used
    "ring": (dict(batch=64, lens=synth.ragged_lengths(73, 64, 1, 9000), window=128),
             dict(batch=8, lens=synth.ragged_lengths(74, 8, 1, 300), window=128)),
    # static split (two partitions per unit) and its combine launch
    "static": (dict(batch=64, lens=[2048] * 64), dict(batch=32, lens=[1500] * 32)),
    # batch 1, long: many segments per unit
    "batch1": (dict(batch=1, lens=[8192]), dict(batch=1, lens=[700])),
}


@pytest.mark.parametrize("variant", [0, 2, 5])
@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_equals_workspace_call(lib, case, variant):
    for i, kw in enumerate(CASES[case]):
        kw = dict(q_heads=64, kv_heads=8, head_dim=64, block_size=16, seed=5000 + 10 * i + variant,
                  **kw)
        a, b = layer_pair(**kw)
        want = lib.decode_attention_append(a.q, a.k_new, a.v_new, a.k_cache, a.v_cache,
                                           a.block_table, a.seq_lens, a.sinks, a.window,
                                           variant=variant)
        out = torch.full_like(b.q, float("nan"))
        lib.decode_attention_append_noalloc(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache,
                                            b.block_table, b.seq_lens, out, b.sinks, b.window,
                                            variant=variant)
        torch.cuda.synchronize()
        what = f"{case} call {i} variant {variant}"
        assert torch.equal(out, want), f"{what}: output differs"
        assert torch.equal(a.k_cache, b.k_cache), f"{what}: K pool differs"
        assert torch.equal(a.v_cache, b.v_cache), f"{what}: V pool differs"


def tile_pair(batch, lens, T, q_heads, seed):
    """Two identical copies of a layer with a query tile of T tokens (the
    tile's K/V rows appended inside the call)."""
    a, b = layer_pair(batch=batch, q_heads=q_heads, kv_heads=8, head_dim=64, block_size=16,
                      lens=lens, seed=seed)
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    q = torch.randn(batch, T, q_heads, 64, generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn(batch, T, 8, 64, generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn(batch, T, 8, 64, generator=g, device="cuda").to(torch.bfloat16)
    return a, b, q, kn, vn


@pytest.mark.parametrize("variant", [0, 2, 5])
def test_noalloc_query_tile_equals_workspace_call(lib, variant):
    """Query tiles through the no-allocation call: batch 64 ragged with 2
    tokens, then batch 8 with 4 tokens (32 query heads, so the tile still
    fills 16 columns); bit-identical to the workspace call."""
    calls = ((64, (synth.ragged_lengths(75, 64, 513, 8193) + 2).tolist(), 2, 64),
             (8, (synth.ragged_lengths(76, 8, 4, 3000) + 4).tolist(), 4, 32))
    for i, (B, lens, T, hq) in enumerate(calls):
        a, b, q, kn, vn = tile_pair(B, lens, T, hq, seed=5200 + 10 * i + variant)
        want = lib.decode_attention_append(q, kn, vn, a.k_cache, a.v_cache, a.block_table,
                                           a.seq_lens, a.sinks[:hq], 0, variant=variant)
        out = torch.full_like(q, float("nan"))
        lib.decode_attention_append_noalloc(q, kn, vn, b.k_cache, b.v_cache, b.block_table,
                                            b.seq_lens, out, b.sinks[:hq], 0, variant=variant)
        torch.cuda.synchronize()
        what = f"tile call {i} (T={T}) variant {variant}"
        assert torch.equal(out, want), f"{what}: output differs"
        assert torch.equal(a.k_cache, b.k_cache), f"{what}: K pool differs"
        assert torch.equal(a.v_cache, b.v_cache), f"{what}: V pool differs"
