"""The measured workloads at full size, in the launch configuration the bench
times (default split table, default variant), checked against the oracle on
every sequence where that takes seconds and on sampled sequences otherwise,
plus closed-form probes that hold at any size."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, oracle_attention, out_f64, sub_layer

pytestmark = pytest.mark.gpu


def attend(lib, layer, ws=None):
    out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                               layer.seq_lens, layer.sinks, layer.window, workspace=ws)
    torch.cuda.synchronize()
    return out


def ragged_layers(device="cuda"):
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
    common = dict(batch=c["batch"], q_heads=c["q_heads"], kv_heads=c["kv_heads"],
                  head_dim=c["head_dim"], block_size=c["block_size"], lens=lens, device=device)
    full = synth.make_layer(window=0, seed=c["seed"] + 10, **common)
    ring = synth.make_layer(window=128, seed=c["seed"] + 20, **common)
    return full, ring


def test_batch64_ragged_full_and_ring_with_append(lib):
    """Batch 64, ragged 513..8193 after the append, a paged full layer and a
    sliding-window-128 ring layer: every sequence checked."""
    full, ring = ragged_layers()
    for layer in (full, ring):
        ref = oracle_attention(layer, after_append=True)
        s = sub_layer(layer, range(layer.batch))
        kr, vr = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"],
                                  s["lens"], layer.window)
        lib.kv_append(layer.k_new, layer.v_new, layer.k_cache, layer.v_cache,
                      layer.block_table, layer.seq_lens, layer.window)
        after = sub_layer(layer, range(layer.batch))
        assert np.array_equal(after["k"], kr) and np.array_equal(after["v"], vr)
        assert_parity(out_f64(attend(lib, layer)), ref, f"ragged window={layer.window}")


def test_batch64_uniform_8k_every_sequence(lib):
    """Batch 64 x 8192 (the bandwidth headline), attention alone and the fused
    step (append inside the launch), every sequence against the oracle."""
    layer = synth.make_layer(device="cuda", **synth.CONFIGS["batch64_8k"])
    ref = oracle_attention(layer)
    assert_parity(out_f64(attend(lib, layer)), ref, "batch64 8k")
    s = sub_layer(layer, range(layer.batch))
    kr, vr = oracle.kv_append(s["k"], s["v"], s["k_new"], s["v_new"], s["bt"], s["lens"], 0)
    ref_f = oracle.decode_attention(s["q"], kr, vr, s["bt"], s["lens"], s["sinks"], 0)
    out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, layer.k_cache,
                                      layer.v_cache, layer.block_table, layer.seq_lens,
                                      layer.sinks, 0)
    torch.cuda.synchronize()
    after = sub_layer(layer, range(layer.batch))
    assert np.array_equal(after["k"], kr) and np.array_equal(after["v"], vr)
    assert_parity(out_f64(out), ref_f, "batch64 8k, append inside")


@pytest.mark.parametrize("name", ["long_131k_b1", "long_131k_b8", "long_131k_b8_tp_share"])
def test_long_context_every_sequence(lib, name):
    layer = synth.make_layer(device="cuda", **synth.CONFIGS[name])
    S = lib.num_splits(layer.q, layer.k_cache, layer.v_cache, layer.block_table, 0)
    assert 32 <= S <= 256
    got = out_f64(attend(lib, layer))
    assert_parity(got, oracle_attention(layer), f"{name} (S={S})")


def test_long_context_closed_form_q_zero(lib):
    """q = 0 at 131072: every weight is equal, so
    out = mean(V) * n / (n + e^sigma) exactly in the definition."""
    cfg = dict(synth.CONFIGS["long_131k_b1"], seed=77)
    layer = synth.make_layer(device="cuda", **cfg)
    layer.q.zero_()
    got = out_f64(attend(lib, layer))
    n = 131072
    # mean over positions of V, per KV head: V pool is [blk][g][bs/8][D][8]
    bt = layer.block_table[0, :layer.blocks_per_seq[0]].long()
    vsum = layer.v_cache.index_select(0, bt).double().sum(dim=(0, 2, 4))   # [Hkv][D]
    mean_v = (vsum / n).cpu().numpy()
    sig = layer.sinks.double().cpu().numpy()
    want = np.stack([mean_v[h // 8] * n / (n + math.exp(sig[h])) for h in range(64)])
    assert_parity(got[0], want, "q=0 closed form at 131k")


def test_decode_loop_sampled(lib):
    """The decode loop: layers alternating ring-128 / full, batch 64, initial
    lengths 1024..32768, consecutive steps each appending one token per
    sequence.  Run here with 4 layers x 6 steps (the bench runs all 24 x 50);
    sampled sequences are replayed by the oracle at every step, and their
    cache bytes are compared bit for bit after the last step."""
    c = synth.CONFIGS["decode_loop"]
    B, layers, steps, W = c["batch"], 4, 6, c["window"]
    L0 = synth.ragged_lengths(c["seed"], B, *c["len_range"])
    cap = L0 + steps
    model = []
    for li in range(layers):
        w = W if li % 2 == 0 else 0
        model.append(synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64,
                                      block_size=16, lens=L0 + 1, capacity=cap, window=w,
                                      seed=c["seed"] * 100 + li, device="cuda"))
    seqs = [0, 31, 63]
    host = [sub_layer(m, seqs) for m in model]          # oracle's own copies
    seq_lens = model[0].seq_lens.clone()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(c["seed"])
    for t in range(steps):
        for li, m in enumerate(model):
            q = torch.randn(m.q.shape, generator=g, device="cuda").to(torch.bfloat16)
            kn = torch.randn(m.k_new.shape, generator=g, device="cuda").to(torch.bfloat16)
            vn = torch.randn(m.v_new.shape, generator=g, device="cuda").to(torch.bfloat16)
            lib.kv_append(kn, vn, m.k_cache, m.v_cache, m.block_table, seq_lens, m.window)
            out = lib.decode_attention(q, m.k_cache, m.v_cache, m.block_table, seq_lens,
                                       m.sinks, m.window, workspace=ws)
            torch.cuda.synchronize()
            hs = host[li]
            sel = torch.as_tensor(seqs, device="cuda")
            lens = seq_lens.cpu().numpy()[seqs]
            hs["k"], hs["v"] = oracle.kv_append(hs["k"], hs["v"], bits(kn.index_select(0, sel)),
                                                bits(vn.index_select(0, sel)), hs["bt"], lens,
                                                m.window)
            ref = oracle.decode_attention(bits(q.index_select(0, sel)), hs["k"], hs["v"],
                                          hs["bt"], lens, hs["sinks"], m.window)
            assert_parity(out_f64(out)[seqs], ref, f"loop step {t} layer {li}")
        seq_lens += 1
    for li, m in enumerate(model):
        now = sub_layer(m, seqs)
        assert np.array_equal(now["k"], host[li]["k"]) and np.array_equal(now["v"], host[li]["v"])


@pytest.mark.parametrize("variant", [0, 5])
@pytest.mark.parametrize("shape", ["batch64_8k", "batch64_ragged"])
def test_full_size_calls_repeat_bit_for_bit(lib, shape, variant):
    """Races in the merge across wavefronts (units split over wavefronts, the
    merge launch or the last-arriving wavefront's merge) would show as runs
    that differ: five calls at full size through one reused workspace, each
    bit-identical to the first, the attention alone and with the append."""
    layer = (synth.make_layer(device="cuda", **synth.CONFIGS["batch64_8k"])
             if shape == "batch64_8k" else ragged_layers()[0])
    ws = lib.new_workspace(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                           layer.window, variant=variant)
    first = None
    for i in range(5):
        out = lib.decode_attention(layer.q, layer.k_cache, layer.v_cache, layer.block_table,
                                   layer.seq_lens, layer.sinks, layer.window, workspace=ws,
                                   variant=variant)
        torch.cuda.synchronize()
        if first is None:
            first = out.clone()
        assert torch.equal(out, first), f"{shape} v={variant}: run {i} differs from run 0"
    # the fused step: its append is idempotent here (the same rows into the
    # same slots), so every run sees the same pools
    fused0 = None
    for i in range(3):
        out = lib.decode_attention_append(layer.q, layer.k_new, layer.v_new, layer.k_cache,
                                          layer.v_cache, layer.block_table, layer.seq_lens,
                                          layer.sinks, layer.window, workspace=ws,
                                          variant=variant)
        torch.cuda.synchronize()
        if fused0 is None:
            fused0 = out.clone()
            k1, v1 = layer.k_cache.clone(), layer.v_cache.clone()
        assert torch.equal(out, fused0), f"{shape} v={variant}: fused run {i} differs"
        assert torch.equal(layer.k_cache, k1) and torch.equal(layer.v_cache, v1)
