"""Decode attention on the GPU against the fp64 oracle (max-abs <= 2e-2,
mean-abs <= 2e-3), through the C ABI.  Sizes span several partitions and a
ragged tail; the full-size workloads are checked in test_gpu_workloads.py."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, oracle_attention, out_f64, poison_tails, sub_layer

pytestmark = pytest.mark.gpu

VARIANTS = [0, 1, 2, 3, 4, 5]  # default, static two-pass, static fused, vector-ALU, balanced
# (merge launch), balanced with the last wavefront of a unit merging it


def attend(lib, layer, num_splits=0, variant=0, sinks="layer"):
    s = layer.sinks if sinks == "layer" else sinks
    out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                               layer.seq_lens, s, layer.window, num_splits=num_splits,
                               variant=variant)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("L", [38, 37])
@pytest.mark.parametrize("variant", VARIANTS)
def test_tiny_config_with_append(lib, L, variant):
    """batch 1, 4 query heads / 1 KV head, D 64, bs 16, shuffled table, sinks,
    one new token appended (L = 38 reads 37 cached + 1 new; 37 also run)."""
    cfg = dict(synth.CONFIGS["tiny"], lens=[L])
    layer = synth.make_layer(device="cuda", **cfg)
    ref = oracle_attention(layer, after_append=True)
    lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
                  layer.block_table, layer.seq_lens, 0)
    assert_parity(out_f64(attend(lib, layer, variant=variant)), ref, f"tiny L={L}")


@pytest.mark.parametrize("scale", [0.125, 1.0])
def test_gptoss_layer_8k(lib, scale):
    cfg = dict(synth.CONFIGS["gptoss_layer_8k"], scale=scale)
    layer = synth.make_layer(device="cuda", **cfg)
    ref = oracle_attention(layer)
    for v in VARIANTS:
        assert_parity(out_f64(attend(lib, layer, variant=v)), ref, f"8k scale={scale} v={v}")


@pytest.mark.parametrize("S", [1, 2, 7, 32, 256])
def test_split_sweep(lib, S):
    layer = synth.make_layer(batch=3, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[8192, 3001, 77], seed=300 + S, device="cuda")
    ref = oracle_attention(layer)
    for v in VARIANTS:
        got = out_f64(attend(lib, layer, num_splits=S, variant=v))
        assert_parity(got, ref, f"S={S} variant={v}")


@pytest.mark.parametrize("W", [128, 100])
def test_window_edges(lib, W):
    lens = [1, W - 1, W, W + 1, 2 * W + 3, 5000]
    layer = synth.make_layer(batch=len(lens), q_heads=64, kv_heads=8, head_dim=64,
                             block_size=16, lens=lens, window=W, seed=400 + W, device="cuda")
    ref = oracle_attention(layer, after_append=True)
    lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
                  layer.block_table, layer.seq_lens, W)
    for v in VARIANTS:
        for S in (0, 1, 3):
            assert_parity(out_f64(attend(lib, layer, num_splits=S, variant=v)), ref,
                          f"W={W} S={S} v={v}")


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_block_sizes(lib, bs):
    lens = [1, 31, 32, 33, 1000, 2049]
    layer = synth.make_layer(batch=len(lens), q_heads=32, kv_heads=4, head_dim=64,
                             block_size=bs, lens=lens, seed=500 + bs, device="cuda")
    ref = oracle_attention(layer)
    for S in (0, 1, 5):
        assert_parity(out_f64(attend(lib, layer, num_splits=S)), ref, f"bs={bs} S={S}")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_group_sizes(lib, G):
    layer = synth.make_layer(batch=2, q_heads=4 * G, kv_heads=4, head_dim=64, block_size=16,
                             lens=[700, 129], seed=600 + G, device="cuda")
    ref = oracle_attention(layer)
    assert_parity(out_f64(attend(lib, layer)), ref, f"G={G}")


def test_no_sinks_is_plain_softmax(lib):
    layer = synth.make_layer(batch=4, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[1, 17, 300, 2000], seed=700, device="cuda", sinks=False)
    ref = oracle_attention(layer)
    got = out_f64(attend(lib, layer))
    assert_parity(got, ref, "no sinks")
    # L = 1 without a sink returns v0 exactly (bf16 of it)
    v0 = bits(layer.v_cache)[int(layer.block_table[0, 0]), :, 0, :, 0]   # slot 0: [Hkv][D]
    v0 = oracle.bf16_bits_to_f64(v0)
    assert np.array_equal(got[0], np.repeat(v0, 8, axis=0))
    # sinks of -inf equal no sinks, bit for bit
    neg = torch.full((64,), -math.inf, device="cuda")
    assert torch.equal(attend(lib, layer, sinks=neg), attend(lib, layer, sinks=None))


def test_large_sinks_and_scores(lib):
    """Sinks far above and below the scores, and large-magnitude queries."""
    layer = synth.make_layer(batch=3, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=[50, 900, 4000], seed=710, device="cuda")
    # scores with a spread of ~N(0, 9) (q times 4, exact in bf16); V stays
    # N(0,1) so the output magnitude is the one the tolerance is stated for
    layer.q.mul_(4.0)
    layer.sinks = torch.tensor([60.0, -60.0, 0.0, 5.0] * 4, device="cuda")
    ref = oracle_attention(layer)
    for v in VARIANTS:
        assert_parity(out_f64(attend(lib, layer, variant=v)), ref, f"large v={v}")


def test_paged_equals_contiguous_bitwise(lib):
    """The same cache contents through a shuffled and an identity table give
    bit-identical outputs at a fixed split count."""
    layer = synth.make_layer(batch=4, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[40, 999, 4096, 123], seed=800, device="cuda")
    bt = layer.block_table.cpu()
    order = []
    for b, n in enumerate(layer.blocks_per_seq):
        order.extend(bt[b, :n].tolist())
    order.append(layer.poison_block)
    idx = torch.as_tensor(order, device="cuda")
    k2 = layer.k_cache.index_select(0, idx).contiguous()
    v2 = layer.v_cache.index_select(0, idx).contiguous()
    bt2 = torch.full_like(layer.block_table, len(order) - 1)
    start = 0
    for b, n in enumerate(layer.blocks_per_seq):
        bt2[b, :n] = torch.arange(start, start + n, dtype=torch.int32)
        start += n
    for v in VARIANTS:
        for S in (0, 4):
            a = attend(lib, layer, num_splits=S, variant=v)
            c = lib.decode_attention(layer.q, k2, v2, bt2, layer.seq_lens, layer.sinks, 0,
                                     num_splits=S, variant=v)
            torch.cuda.synchronize()
            assert torch.equal(a, c), f"paged != contiguous (S={S}, v={v})"


def test_deterministic(lib):
    layer = synth.make_layer(batch=8, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=synth.ragged_lengths(9, 8, 100, 6000).tolist(), seed=900,
                             device="cuda")
    for v in VARIANTS:
        a = attend(lib, layer, variant=v)
        b = attend(lib, layer, variant=v)
        assert torch.equal(a, b), f"variant {v} not deterministic"


def test_stale_nan_tails_never_leak(lib):
    """NaN in every slot past each sequence's end (inside its own blocks) and
    the poison block behind unused table entries never reach the output."""
    for W in (0, 128):
        layer = synth.make_layer(batch=5, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                                 lens=[1, 15, 33, 100, 1001], window=W, seed=950 + W,
                                 device="cuda")
        ref = oracle_attention(layer)
        poison_tails(layer)
        for v in VARIANTS:
            for S in (0, 1, 3):
                assert_parity(out_f64(attend(lib, layer, num_splits=S, variant=v)), ref,
                              f"NaN tails W={W} S={S} v={v}")


def test_empty_context_gives_zero(lib):
    layer = synth.make_layer(batch=3, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=[5, 64, 300], seed=990, device="cuda")
    layer.seq_lens[1] = 0
    for v in VARIANTS:
        for S in (0, 1, 4):
            out = attend(lib, layer, num_splits=S, variant=v)
            assert torch.count_nonzero(out[1]) == 0
    ref = oracle_attention(layer)
    assert_parity(out_f64(attend(lib, layer)), ref, "with an empty sequence")


def test_partials_and_combine_entry_points(lib):
    layer = synth.make_layer(batch=3, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[10, 3000, 8192], seed=1000, device="cuda")
    po, pl = lib.decode_partials(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                                 layer.seq_lens, 0, num_splits=16)
    torch.cuda.synchronize()
    S = po.shape[2]
    assert S >= 8
    # every non-empty partial against the oracle's partial over the same slots;
    # the partition length is the capacity split S ways, rounded up to 32 slots
    cap = layer.max_blocks_per_seq * layer.block_size
    P = math.ceil(math.ceil(cap / S) / 32) * 32
    assert math.ceil(cap / P) == S
    sl = synth.to_bits
    q, k, v, bt = sl(layer.q), sl(layer.k_cache), sl(layer.v_cache), sl(layer.block_table)
    lse = pl.cpu().numpy()
    o = po.cpu().numpy()
    for b, L in enumerate(layer.seq_lens.cpu().tolist()):
        for h in (0, 7, 8, 63):
            for j in range(S):
                lo, hi = j * P, min(L, (j + 1) * P)
                if lo >= L:
                    assert lse[b, h, j] == -np.inf
                    continue
                ro, rl = oracle.partial_attention(q, k, v, bt, b, h, range(lo, hi), 0)
                assert abs(lse[b, h, j] - rl) < 1e-3 * max(1.0, abs(rl))
                assert np.abs(o[b, h, j] - ro).max() < 1e-2
    out = lib.combine(po, pl, layer.sinks)
    torch.cuda.synchronize()
    assert_parity(out_f64(out), oracle_attention(layer), "partials + combine")


@pytest.mark.parametrize("S", [2, 8, 9])         # one-wavefront merge up to 8, then 4 waves
def test_combine_alone(lib, S):
    """sa_combine on random partials, some empty (-inf), against the oracle."""
    g = torch.Generator().manual_seed(5)
    B, Hq, D = 3, 8, 64
    po = torch.randn(B, Hq, S, D, generator=g)
    pl = torch.randn(B, Hq, S, generator=g) * 4
    e = min(3, S - 1)
    pl[0, :, e] = -math.inf
    pl[1, 2, :] = -math.inf            # a head with nothing: only the sink
    pl[2, 5, :] = -math.inf
    po[0, :, e] = float("nan")        # an empty partition's o never reaches out
    po[2, 5, :] = float("nan")
    sinks = torch.randn(Hq, generator=g)
    ref = oracle.combine(po.numpy(), pl.numpy(), sinks.numpy())
    out = lib.combine(po.cuda(), pl.cuda(), sinks.cuda())
    torch.cuda.synchronize()
    assert_parity(out_f64(out), ref, "combine")
    out = lib.combine(po.cuda(), pl.cuda(), None)
    torch.cuda.synchronize()
    assert_parity(out_f64(out), oracle.combine(po.numpy(), pl.numpy(), None), "combine no sink")
    assert torch.count_nonzero(out[1, 2]) == 0


def test_workspace_reused_across_calls(lib):
    """One zeroed workspace serves many fused calls of different shapes."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for i, lens in enumerate(([5000, 17, 8000], [1, 2, 3], [4097, 4096, 9000])):
        layer = synth.make_layer(batch=3, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                                 lens=lens, seed=1100 + i, device="cuda")
        ref = oracle_attention(layer)
        for S in (0, 5, 16):
            out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                                       layer.seq_lens, layer.sinks, 0, workspace=ws,
                                       num_splits=S, variant=2)
            torch.cuda.synchronize()
            assert_parity(out_f64(out), ref, f"reuse {i} S={S}")


@pytest.mark.parametrize("W", [0, 128])
@pytest.mark.parametrize("B,lo,hi", [(5, 0, 3000), (37, 0, 700), (200, 1, 2500), (1, 9000, 9000)])
def test_balanced_kernel_edge_cases(lib, W, B, lo, hi):
    """The equal-work kernel over ragged batches with empty sequences, more
    than 64 sequences (several scan chunks), and a single long sequence whose
    units spread over many wavefronts."""
    lens = synth.ragged_lengths(1234 + B, B, lo, hi).tolist()
    layer = synth.make_layer(batch=B, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=lens, window=W, seed=2000 + B + W, device="cuda",
                             capacity=[max(1, L) for L in lens])
    ref = oracle_attention(layer)
    for v in (0, 4, 5):
        a = attend(lib, layer, variant=v)
        assert_parity(out_f64(a), ref, f"balanced B={B} W={W} v={v}")
        assert torch.equal(a, attend(lib, layer, variant=v)), "not deterministic"


@pytest.mark.parametrize("lens", [[0, 0, 700, 0, 33, 0], [0, 0, 0], [900, 0, 0], [0, 5000],
                                  [0] * 70 + [129]])
def test_empty_sequences_zeroed_over_stale_state(lib, lens):
    """Empty sequences before the first one with a step, between two, after
    the last, and a batch with nothing at all: zeros land over an output
    prefilled with NaN, with a workspace that a call on other lengths has
    left dirty (the merge must read only what this call recorded)."""
    B = len(lens)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    cap = [max(3000, L) for L in lens]
    dirty = synth.make_layer(batch=B, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=[3000] * B, capacity=cap, seed=1300 + B, device="cuda")
    layer = synth.make_layer(batch=B, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=lens, capacity=cap, seed=1400 + B, device="cuda")
    ref = oracle_attention(layer)
    for v in (0, 4, 5):
        lib.decode_attention(dirty.q, dirty.k_cache, dirty.v_cache, dirty.block_table,
                             dirty.seq_lens, dirty.sinks, 0, workspace=ws, variant=v)
        out = torch.full_like(layer.q, float("nan"))
        lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                             layer.seq_lens, layer.sinks, 0, out=out, workspace=ws, variant=v)
        torch.cuda.synchronize()
        assert_parity(out_f64(out), ref, f"lens={lens} v={v}")


@pytest.mark.parametrize("lens", [[1800, 0], [0, 1800], [0, 0]])
def test_empty_sequences_with_more_than_64_kv_heads(lib, lens):
    """128 KV heads of one query head each: an empty sequence must leave a
    "done" record for every one of its units, not only for the first 64, when
    the workspace was dirtied by a call in which those units were spread over
    several wavefronts (a stale record would merge that call's partials over
    the zeros)."""
    B, H = 2, 128
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    dirty = synth.make_layer(batch=B, q_heads=H, kv_heads=H, head_dim=64, block_size=16,
                             lens=[2000] * B, capacity=[2048] * B, seed=1310, device="cuda")
    layer = synth.make_layer(batch=B, q_heads=H, kv_heads=H, head_dim=64, block_size=16,
                             lens=lens, capacity=[2048] * B, seed=1410 + sum(lens) // 7,
                             device="cuda")
    ref = oracle_attention(layer)
    for v in (0, 4, 5):
        lib.decode_attention(dirty.q, dirty.k_cache, dirty.v_cache, dirty.block_table,
                             dirty.seq_lens, dirty.sinks, 0, workspace=ws, variant=v)
        out = torch.full_like(layer.q, float("nan"))
        lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                             layer.seq_lens, layer.sinks, 0, out=out, workspace=ws, variant=v)
        torch.cuda.synchronize()
        got = out_f64(out)
        assert_parity(got, ref, f"lens={lens} v={v}")
        for b, L in enumerate(lens):
            if L == 0:
                assert not got[b].any(), f"sequence {b} is empty: all zeros (v={v})"


@pytest.mark.parametrize("W", [0, 128])
def test_short_sequences_under_a_large_capacity(lib, W):
    """Tables sized for long contexts (8192 slots) holding short ones: the
    launch plans for far more steps than there are, so most wavefronts have
    nothing to do and a unit's steps must still be merged from exactly the
    wavefronts that hold them (also after a call that dirtied the workspace)."""
    B = 64
    lens = synth.ragged_lengths(1500 + W, B, 1, 300)
    cap = [8192] * B
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    dirty = synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[8192] * B, capacity=cap, window=W, seed=1600 + W,
                             device="cuda")
    layer = synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=lens, capacity=cap, window=W, seed=1700 + W, device="cuda")
    ref = oracle_attention(layer)
    for v in (0, 4, 5):
        lib.decode_attention(dirty.q, dirty.k_cache, dirty.v_cache, dirty.block_table,
                             dirty.seq_lens, dirty.sinks, W, workspace=ws, variant=v)
        out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                                   layer.seq_lens, layer.sinks, W, workspace=ws, variant=v)
        torch.cuda.synchronize()
        assert_parity(out_f64(out), ref, f"short under capacity W={W} v={v}")


@pytest.mark.parametrize("W", [0, 128])
def test_pools_past_4gib(lib, W):
    """64-bit addressing: a layer's blocks moved to the top of pools of about
    4.3 GB each, so every block the table names starts past byte 2^32 of its
    pool.  Attention (every engine), the fused append and the standalone
    append must give what the oracle gives for the same blocks in a small
    pool."""
    layer = synth.make_layer(batch=4, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[3000, 17, 1000, 520], window=W, seed=9100 + W,
                             device="cuda")
    nb = layer.k_cache.shape[0]
    block_bytes = layer.k_cache[0].numel() * layer.k_cache.element_size()
    off = (1 << 32) // block_bytes + 1000
    assert off * block_bytes > (1 << 32)
    big_k = torch.empty((off + nb,) + tuple(layer.k_cache.shape[1:]), dtype=layer.k_cache.dtype,
                        device="cuda")
    big_v = torch.empty((off + nb,) + tuple(layer.v_cache.shape[1:]), dtype=layer.v_cache.dtype,
                        device="cuda")
    big_k[off:] = layer.k_cache
    big_v[off:] = layer.v_cache
    big = dataclasses.replace(layer, k_cache=big_k, v_cache=big_v,
                              block_table=layer.block_table + off,
                              poison_block=layer.poison_block + off)
    ref = oracle_attention(layer)
    for v in VARIANTS:
        assert_parity(out_f64(attend(lib, big, variant=v)), ref, f"W={W} variant={v}")
    # the appends write past 4 GiB too: compare the moved blocks bit for bit
    s = sub_layer(layer, range(layer.batch))
    k_ref, v_ref = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"], s["lens"], W)
    ref_after = oracle.decode_attention(s["q"], k_ref, v_ref, s["bt"], s["lens"], s["sinks"], W)
    for v in (0, 1, 2, 4):
        kc, vc = big_k.clone(), big_v.clone()
        run = dataclasses.replace(big, k_cache=kc, v_cache=vc)
        out = lib.decode_attention_append(run.q, run.k_new, run.v_new, kc, vc, run.block_table,
                                          run.seq_lens, run.sinks, W, variant=v)
        torch.cuda.synchronize()
        after = sub_layer(run, range(layer.batch))
        assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref), \
            f"W={W} variant={v}: pools after the fused append"
        assert_parity(out_f64(out), ref_after, f"W={W} fused variant={v}")
        del kc, vc, run
    lib.kv_append(big.k_new, big.v_new, big_k, big_v, big.block_table, big.seq_lens, W)
    torch.cuda.synchronize()
    after = sub_layer(big, range(layer.batch))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref)


@pytest.mark.parametrize("B", [2048, 2049])
def test_batch_at_the_balanced_limit(lib, B):
    """2048 sequences is the most the balanced kernel takes (its per-sequence
    lengths and step prefix sit in LDS); one more and every call goes to the
    static split.  Attention and the fused append, every sequence checked."""
    lens = np.random.default_rng(B).integers(1, 300, size=B)
    layer = synth.make_layer(batch=B, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=lens, seed=9200 + B, device="cuda")
    ref = oracle_attention(layer)
    for v in (0, 4, 5):
        assert_parity(out_f64(attend(lib, layer, variant=v)), ref, f"B={B} variant={v}")
    s = sub_layer(layer, range(B))
    k_ref, v_ref = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"], s["lens"], 0)
    ref_after = oracle.decode_attention(s["q"], k_ref, v_ref, s["bt"], s["lens"], s["sinks"], 0)
    out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, layer.k_cache,
                                      layer.v_cache, layer.block_table, layer.seq_lens,
                                      layer.sinks, 0)
    torch.cuda.synchronize()
    after = sub_layer(layer, range(B))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref)
    assert_parity(out_f64(out), ref_after, f"B={B} fused")


def test_context_parallel_shards_merge(lib):
    """Context parallelism as it would run over several GPUs, emulated on one:
    each sequence's blocks are cut into R contiguous shards; every shard's
    partials come from sa_decode_partials over its own slice of the block
    table (its slots counted from 0: full attention does not depend on where
    a slot sits), and one sa_combine over all shards' partials, which is what
    the exchange would deliver, gives the whole attention.  Shape: one GPU's
    tensor-parallel share of the long-context layer (8 query heads, 1 KV
    head); a short sequence leaves whole shards empty."""
    R, bs = 4, 16
    layer = synth.make_layer(batch=3, q_heads=8, kv_heads=1, head_dim=64, block_size=bs,
                             lens=[20000, 7777, 33], seed=9300, device="cuda")
    ref = oracle_attention(layer)
    mbs = layer.block_table.shape[1]
    per = math.ceil(mbs / R)
    pos, pls = [], []
    for r in range(R):
        lo, hi = r * per, min(mbs, (r + 1) * per)
        table = layer.block_table[:, lo:hi].contiguous()
        lens = (layer.seq_lens - lo * bs).clamp(min=0, max=(hi - lo) * bs).to(torch.int32)
        po, pl = lib.decode_partials(layer.q, layer.k_cache, layer.v_cache, table, lens, 0)
        pos.append(po)
        pls.append(pl)
    torch.cuda.synchronize()
    out = lib.combine(torch.cat(pos, dim=2).contiguous(), torch.cat(pls, dim=2).contiguous(),
                      layer.sinks)
    torch.cuda.synchronize()
    assert_parity(out_f64(out), ref, f"{R} context shards merged")


def test_an_earlier_hip_error_does_not_fail_a_call(lib):
    """A call reports the status of its own launches only: an error an earlier,
    unrelated HIP call left on the thread (an invalid device ordinal here) does
    not turn a good call into SA_ERR_HIP."""
    import ctypes
    layer = synth.make_layer(batch=3, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=[100, 2000, 7], seed=9400, device="cuda")
    ref = oracle_attention(layer)
    out = torch.empty_like(layer.q)
    ws = lib.new_workspace(layer.q, layer.k_cache, layer.v_cache, layer.block_table, 0)
    d = lib.dims_for(layer.q, layer.k_cache, layer.v_cache, layer.block_table, 0,
                     lib.VARIANT_DEFAULT)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    torch.cuda.synchronize()
    # the HIP runtime this process has loaded (the one libsa calls)
    with open("/proc/self/maps") as f:
        paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    if len(paths) != 1:
        pytest.skip(f"{len(paths)} HIP runtimes loaded: {paths}")
    hip = ctypes.CDLL(paths[0])
    assert hip.hipSetDevice(ctypes.c_int(9999)) != 0          # leaves an error behind
    st = lib.load().sa_decode_attention(p(layer.q), p(layer.k_cache), p(layer.v_cache),
                                        p(layer.block_table), p(layer.seq_lens), p(layer.sinks),
                                        0, p(out), ctypes.byref(d),
                                        None if ws is None else p(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    hip.hipGetLastError()                                       # clear it again
    assert st == 0, lib.status_string(st)
    torch.cuda.synchronize()
    assert_parity(out_f64(out), ref, "after an earlier HIP error")


def test_context_past_the_table_is_cut_to_its_capacity(lib):
    """seq_lens beyond the table's capacity (max_blocks_per_seq * bs): attention
    covers the first capacity slots, as for a sequence of that length, and the
    append, whose slot lies past the table, writes nothing."""
    bs = 16
    layer = synth.make_layer(batch=3, q_heads=16, kv_heads=2, head_dim=64, block_size=bs,
                             lens=[20 * bs, 40, 7], seed=9500, device="cuda")
    cap = layer.block_table.shape[1] * bs                      # 320 slots per row
    over = torch.tensor([cap + 77, 40, 7], dtype=torch.int32, device="cuda")
    clamped = dataclasses.replace(layer, seq_lens=torch.minimum(
        over, torch.tensor(cap, dtype=torch.int32, device="cuda")))
    ref = oracle_attention(clamped)
    for v in VARIANTS:
        out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                                   over, layer.sinks, 0, variant=v)
        torch.cuda.synchronize()
        assert_parity(out_f64(out), ref, f"past capacity, variant {v}")
    # fused: sequence 0's new slot (position cap+76) is past the table: the
    # oracle's append writes nothing there either; the others append as usual
    s = sub_layer(clamped, range(3))
    lens_host = over.cpu().numpy()
    k_ref, v_ref = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"],
                                    lens_host, 0)
    out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, layer.k_cache,
                                      layer.v_cache, layer.block_table, over, layer.sinks, 0)
    torch.cuda.synchronize()
    after = sub_layer(clamped, range(3))
    assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref)
    ref2 = oracle.decode_attention(s["q"], k_ref, v_ref, s["bt"], np.minimum(lens_host, cap),
                                   s["sinks"], 0)
    assert_parity(out_f64(out), ref2, "past capacity, fused")


def test_table_entries_outside_the_pool(lib):
    """Block-table entries outside [0, num_blocks) are a caller error that never
    leads to a wild access: reads clamp the entry into the pool, and an append
    whose slot's entry is outside it writes nothing (inside the attention launch
    as in sa_kv_append)."""
    bs = 16
    layer = synth.make_layer(batch=3, q_heads=16, kv_heads=2, head_dim=64, block_size=bs,
                             lens=[300, 200, 90], seed=9600, device="cuda")
    NB = layer.k_cache.shape[0]
    bad = layer.block_table.clone()
    bad[0, 5] = -5                                   # a read of sequence 0, mid-context
    bad[1, (200 - 1) // bs] = NB + 100               # sequence 1's new token's block
    clipped = dataclasses.replace(layer, block_table=bad.clamp(0, NB - 1))
    # reads: as through the clamped table
    ref = oracle_attention(clipped)
    for v in VARIANTS:
        out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, bad, layer.seq_lens,
                                   layer.sinks, 0, variant=v)
        torch.cuda.synchronize()
        assert_parity(out_f64(out), ref, f"entries outside the pool, variant {v}")
    # appends: sequence 1's is skipped, the others land
    k0 = bits(layer.k_cache)
    v0 = bits(layer.v_cache)
    lens = layer.seq_lens.cpu().numpy().copy()
    skip1 = lens.copy()
    skip1[1] = 0
    cb = bits(clipped.block_table)
    k_ref, v_ref = oracle.kv_append(k0, v0, bits(layer.k_new), bits(layer.v_new), cb, skip1, 0)
    ref2 = oracle.decode_attention(bits(layer.q), k_ref, v_ref, cb, lens,
                                   layer.sinks.cpu().numpy(), 0)
    for v in (0, 1, 2, 4):
        kc, vc = layer.k_cache.clone(), layer.v_cache.clone()
        out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, kc, vc, bad,
                                          layer.seq_lens, layer.sinks, 0, variant=v)
        torch.cuda.synchronize()
        assert np.array_equal(bits(kc), k_ref) and np.array_equal(bits(vc), v_ref), f"v={v}"
        assert_parity(out_f64(out), ref2, f"fused, entries outside the pool, variant {v}")
    kc, vc = layer.k_cache.clone(), layer.v_cache.clone()
    lib.kv_append(layer.k_new, layer.v_new, kc, vc, bad, layer.seq_lens, 0)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), k_ref) and np.array_equal(bits(vc), v_ref)


def _set_keys(layer, b, rows):
    """Write K rows [n][Hkv][D] for positions 0..n-1 of sequence b into the
    pool (test-side layout arithmetic: position p in block table[b][p // bs] at
    slot p % bs; a K row as two halves of 32 dims)."""
    bs = layer.block_size
    p = torch.arange(rows.shape[0], device=rows.device)
    blks = layer.block_table[b].to(torch.long)[p // bs]
    n, hkv, d = rows.shape
    layer.k_cache[blks, :, :, p % bs, :] = rows.reshape(n, hkv, 2, d // 2).to(torch.bfloat16)


def test_running_max_rises_jumps_and_falls(lib):
    """Score profiles that move the online softmax's running max in every way:
    a steady climb far past 2^8 (many rescales), one late jump to a single
    position that then dominates the output (and a lower peak after it), a
    staircase of rises each below 2^8 (probabilities up to that size between
    rescales), and a steady fall.  In each KV group the first query head gets the profile
    exactly (keys along its query), the others a random fraction of it."""
    lens = [3000, 3000, 2000, 700]
    layer = synth.make_layer(batch=4, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=lens, seed=720, device="cuda")
    G = 8
    for b, L in enumerate(lens):
        p = torch.arange(L, device="cuda", dtype=torch.float32)
        s = [60.0 * p / L,                                     # climb
             torch.where(p == 2500, 40.0, torch.where(p == 2900, 35.0, 0.0)),  # late jump
             4.0 * torch.floor(p / 200),                       # staircase below 2^8
             30.0 - 60.0 * p / L][b]                           # fall
        rows = torch.empty(L, 2, 64, device="cuda")
        for g in range(2):
            q0 = layer.q[b, g * G].float()
            rows[:, g] = s[:, None] * 8.0 * q0[None, :] / float(q0 @ q0)
        _set_keys(layer, b, rows)
    ref = oracle_attention(layer)
    for v in VARIANTS:
        for S in (0, 3):
            assert_parity(out_f64(attend(lib, layer, num_splits=S, variant=v)), ref,
                          f"running max v={v} S={S}")
