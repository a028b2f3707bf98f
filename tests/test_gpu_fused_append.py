"""The fused decode step (KV append inside the attention launch) on the GPU.

For every MFMA variant and split count, on paged and ring layers: the pools
after the call are bit-identical to the oracle's append, the output is within
tolerance of the oracle's attention over the appended cache, and it is
bit-identical to the separate append followed by the attention call (the
fused kernel feeds the same bits to the same arithmetic)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, oracle_attention, out_f64, sub_layer

pytestmark = pytest.mark.gpu

MFMA_VARIANTS = [0, 1, 2, 4, 5]   # default, static two-pass, static fused combine,
# balanced (merge launch), balanced with the last wavefront of a unit merging it


def fresh_caches(layer):
    return layer.k_cache.clone(), layer.v_cache.clone()


def fused(lib, layer, k_cache, v_cache, num_splits=0, variant=0, ws=None, lens=None):
    out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, k_cache, v_cache,
                                      layer.block_table,
                                      layer.seq_lens if lens is None else lens,
                                      layer.sinks, layer.window, workspace=ws,
                                      num_splits=num_splits, variant=variant)
    torch.cuda.synchronize()
    return out


def separate(lib, layer, k_cache, v_cache, num_splits=0, variant=0):
    lib.kv_append(layer.k_new, layer.v_new, k_cache, v_cache, layer.block_table,
                  layer.seq_lens, layer.window)
    out = lib.decode_attention(layer.q, k_cache, v_cache, layer.block_table, layer.seq_lens,
                               layer.sinks, layer.window, num_splits=num_splits,
                               variant=variant)
    torch.cuda.synchronize()
    return out


def check_layer(lib, layer, splits=(0, 1, 3), variants=MFMA_VARIANTS, what=""):
    k0, v0 = bits(layer.k_cache), bits(layer.v_cache)
    kr, vr = oracle.kv_append(k0, v0, bits(layer.k_new), bits(layer.v_new),
                              bits(layer.block_table), bits(layer.seq_lens), layer.window)
    ref = oracle_attention(layer, after_append=True)
    for v in variants:
        for S in splits:
            kc, vc = fresh_caches(layer)
            got = fused(lib, layer, kc, vc, S, v)
            tag = f"{what} S={S} v={v}"
            assert np.array_equal(bits(kc), kr), f"{tag}: K pool differs from the oracle append"
            assert np.array_equal(bits(vc), vr), f"{tag}: V pool differs from the oracle append"
            assert_parity(out_f64(got), ref, tag)
            ks, vs = fresh_caches(layer)
            want = separate(lib, layer, ks, vs, S, v)
            assert torch.equal(got, want), f"{tag}: fused != append + attention"


@pytest.mark.parametrize("L", [38, 37, 1, 16, 17])
def test_tiny_fused(lib, L):
    cfg = dict(synth.CONFIGS["tiny"], lens=[L])
    check_layer(lib, synth.make_layer(device="cuda", **cfg), what=f"tiny L={L}")


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
@pytest.mark.parametrize("window", [0, 128, 100])
def test_block_sizes_and_windows(lib, bs, window):
    """New slots at block starts, block ends and the ring's wrap point; runs
    long enough for the table slice to span several runs (bs 8: 64 blocks =
    512 slots per run)."""
    lens = [1, bs - 1, bs, bs + 1, 31, 32, 33, 127, 128, 129, 200, 1500]
    layer = synth.make_layer(batch=len(lens), q_heads=32, kv_heads=4, head_dim=64,
                             block_size=bs, lens=lens, window=window,
                             seed=5000 + bs + window, device="cuda")
    check_layer(lib, layer, what=f"bs={bs} W={window}")


@pytest.mark.parametrize("W", [128, 100])
def test_ring_wrap_points(lib, W):
    """Every residue of the ring slot near the wrap, and lengths many windows
    past it, so the new token overwrites the oldest one."""
    lens = [W - 1, W, W + 1, 2 * W - 1, 2 * W, 2 * W + 1, 5 * W + 37, 9000]
    layer = synth.make_layer(batch=len(lens), q_heads=64, kv_heads=8, head_dim=64,
                             block_size=16, lens=lens, window=W, seed=5100 + W, device="cuda")
    check_layer(lib, layer, splits=(0, 1, 2, 7), what=f"ring W={W}")


def test_empty_sequences_append_nothing(lib):
    layer = synth.make_layer(batch=4, q_heads=8, kv_heads=2, head_dim=64, block_size=16,
                             lens=[5, 9, 17, 40], seed=5200, device="cuda")
    layer.seq_lens[1] = 0
    layer.seq_lens[3] = 0
    check_layer(lib, layer, what="empty sequences")


def test_split_sweep_long(lib):
    layer = synth.make_layer(batch=3, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                             lens=[8192, 3001, 77], seed=5300, device="cuda")
    check_layer(lib, layer, splits=(0, 2, 32, 256), what="long")


def test_vector_alu_variant_is_refused(lib):
    layer = synth.make_layer(device="cuda", **synth.CONFIGS["tiny"])
    kc, vc = fresh_caches(layer)
    with pytest.raises(lib.SAError):
        fused(lib, layer, kc, vc, variant=lib.VARIANT_VALU)
    torch.cuda.synchronize()
    assert torch.equal(kc, layer.k_cache) and torch.equal(vc, layer.v_cache)


def test_batch64_ragged_fused(lib):
    """Batch 64, ragged 513..8193 after the append, a paged full layer and a
    ring-128 layer, the default launch: every sequence checked, pools bit for
    bit."""
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
    for w in (0, 128):
        layer = synth.make_layer(batch=c["batch"], q_heads=c["q_heads"], kv_heads=c["kv_heads"],
                                 head_dim=c["head_dim"], block_size=c["block_size"], lens=lens,
                                 window=w, seed=c["seed"] + 30 + w, device="cuda")
        s = sub_layer(layer, range(layer.batch))
        kr, vr = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"], s["lens"], w)
        ref = oracle_attention(layer, after_append=True)
        out = fused(lib, layer, layer.k_cache, layer.v_cache)
        after = sub_layer(layer, range(layer.batch))
        assert np.array_equal(after["k"], kr) and np.array_equal(after["v"], vr)
        assert_parity(out_f64(out), ref, f"ragged fused W={w}")


def test_fused_decode_loop_sampled(lib):
    """Consecutive decode steps through the fused call (4 layers alternating
    ring-128 / full, batch 64, 6 steps), sampled sequences replayed by the
    oracle at every step, cache bytes compared after the last step."""
    c = synth.CONFIGS["decode_loop"]
    B, layers, steps, W = c["batch"], 4, 6, c["window"]
    L0 = synth.ragged_lengths(c["seed"] + 1, B, *c["len_range"])
    model = [synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                              lens=L0 + 1, capacity=L0 + steps, window=W if li % 2 == 0 else 0,
                              seed=c["seed"] * 100 + 50 + li, device="cuda")
             for li in range(layers)]
    seqs = [0, 31, 63]
    host = [sub_layer(m, seqs) for m in model]
    seq_lens = model[0].seq_lens.clone()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(c["seed"] + 1)
    sel = torch.as_tensor(seqs, device="cuda")
    for t in range(steps):
        for li, m in enumerate(model):
            q = torch.randn(m.q.shape, generator=g, device="cuda").to(torch.bfloat16)
            kn = torch.randn(m.k_new.shape, generator=g, device="cuda").to(torch.bfloat16)
            vn = torch.randn(m.v_new.shape, generator=g, device="cuda").to(torch.bfloat16)
            out = lib.decode_attention_append(q, kn, vn, m.k_cache, m.v_cache, m.block_table,
                                              seq_lens, m.sinks, m.window, workspace=ws)
            torch.cuda.synchronize()
            hs = host[li]
            lens = seq_lens.cpu().numpy()[seqs]
            hs["k"], hs["v"] = oracle.kv_append(hs["k"], hs["v"], bits(kn.index_select(0, sel)),
                                                bits(vn.index_select(0, sel)), hs["bt"], lens,
                                                m.window)
            ref = oracle.decode_attention(bits(q.index_select(0, sel)), hs["k"], hs["v"],
                                          hs["bt"], lens, hs["sinks"], m.window)
            assert_parity(out_f64(out)[seqs], ref, f"fused loop step {t} layer {li}")
        seq_lens += 1
    for li, m in enumerate(model):
        now = sub_layer(m, seqs)
        assert np.array_equal(now["k"], host[li]["k"]) and np.array_equal(now["v"], host[li]["v"])


@pytest.mark.parametrize("variant", [0, 1, 2])
@pytest.mark.parametrize("W", [0, 500])
@pytest.mark.parametrize("part", [0, 128, 256])
def test_burst_partitions_with_the_append(lib, W, part, variant):
    """Calls small enough for burst partitions (every step loaded at once): of
    4 steps (128 slots, the plan's choice here: part 0) and of 8 (256 slots,
    forced through the split count); the new token at a partition's first,
    last and next-to-last slot, short last partitions, a ring wider than one
    partition; pools bit for bit and the output against the oracle, plain and
    fused; the default launch, the static two-pass split and the static split
    whose last partition merges (variants 0, 1, 2)."""
    lens = [1, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1000]
    layer = synth.make_layer(batch=len(lens), q_heads=64, kv_heads=8, head_dim=64,
                             block_size=16, lens=lens, window=W, seed=9900 + W, device="cuda")
    n_max = min(W, 1008) if W > 0 else 1008              # 63 blocks of capacity
    forced = -(-n_max // part) if part else 0
    S = lib.num_splits(layer.q, layer.k_cache, layer.v_cache, layer.block_table, W,
                       num_splits=forced, variant=variant)
    assert S == -(-n_max // (part or 128)), "partitions of the intended length"
    assert len(lens) * 8 * S <= 1024, "a grid the burst kernels take"
    s = sub_layer(layer, range(layer.batch))
    kr, vr = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"], s["lens"], W)
    ref = oracle.decode_attention(s["q"], kr, vr, s["bt"], s["lens"], s["sinks"], W)
    kc, vc = layer.k_cache.clone(), layer.v_cache.clone()
    out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, kc, vc,
                                      layer.block_table, layer.seq_lens, layer.sinks, W,
                                      num_splits=forced, variant=variant)
    torch.cuda.synchronize()
    after = sub_layer(dataclasses.replace(layer, k_cache=kc, v_cache=vc), range(layer.batch))
    assert np.array_equal(after["k"], kr) and np.array_equal(after["v"], vr)
    assert_parity(out_f64(out), ref, f"burst W={W} part={part} v={variant} fused")
    lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache, layer.block_table,
                  layer.seq_lens, W)
    plain = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                                 layer.seq_lens, layer.sinks, W, num_splits=forced,
                                 variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(plain, out), "fused and append-then-attend differ"
