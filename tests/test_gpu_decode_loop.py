"""The decode loop at full size: 24 layers alternating a sliding-window-128
ring and a paged full-attention layer, batch 64, 64 query / 8 KV heads,
initial ragged lengths 1024..32768, 50 consecutive steps each appending one
token per sequence in every layer (the fused step: append inside the
attention launch), with fresh seeded q / k_new / v_new at every step.

The same loop runs twice side by side: eagerly, and replayed from a HIP graph
of one step captured once (the per-step inputs are gathered by a device step
counter and ``seq_lens += 1`` runs inside the graph, so nothing on the host
changes between replays).  Every replay's outputs and pools must equal the
eager step's bit for bit, with the eager work between replays.  Both are
checked against the oracle, which replays every step's append on its own
copies of the pools:

* the ring layers, every sequence, at steps 0, 1, 24 and 49;
* the full layers, four fixed sequences (the shortest, the longest and two
  more), at steps 0, 1, 24 and 49, and every sequence of the last full layer
  at step 49;
* after the last step, the pool bytes of those sequences in every layer, and
  of every sequence in the last full layer and the ring layers, bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, out_f64, sub_layer

pytestmark = pytest.mark.gpu

CHECK_STEPS = (0, 1, 24, 49)


def oracle_append(host, kn, vn, lens, window, bs):
    """The oracle's append of one step on host pool copies: the blocks this
    step can write (each sequence's block of slot L-1) go through
    oracle.kv_append under a table that maps exactly those entries, and are
    put back (the oracle returns copies; copying whole multi-GB pools every
    step would take minutes)."""
    bt = host["bt"]
    B = len(lens)
    slots = (lens - 1) if window <= 0 else (lens - 1) % window
    col = slots // bs
    touched = bt[np.arange(B), col].astype(np.int64)
    sub_bt = np.zeros_like(bt)
    sub_bt[np.arange(B), col] = np.arange(B)
    k2, v2 = oracle.kv_append(host["k"][touched], host["v"][touched], kn, vn, sub_bt, lens,
                              window)
    host["k"][touched] = k2
    host["v"][touched] = v2


def build(B, layers, steps, L0, W, dev):
    model = []
    for li in range(layers):
        w = W if li % 2 == 0 else 0
        model.append(synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64,
                                      block_size=16, lens=L0 + 1, capacity=L0 + steps,
                                      window=w, seed=synth.CONFIGS["decode_loop"]["seed"] * 100
                                      + li, device=dev))
    return model


@pytest.mark.timeout(600)         # about a minute of it is the fp64 oracle on the host
def test_decode_loop_full_size_eager_and_graph(lib):
    c = synth.CONFIGS["decode_loop"]
    B, layers, steps, W = c["batch"], c["layers"], c["steps"], c["window"]
    dev = torch.device("cuda")
    L0 = synth.ragged_lengths(c["seed"], B, *c["len_range"])
    eager = build(B, layers, steps, L0, W, dev)
    graph = build(B, layers, steps, L0, W, dev)
    full_ids = [li for li in range(layers) if eager[li].window == 0]
    last_full = full_ids[-1]
    seqs = sorted({int(np.argmin(L0)), int(np.argmax(L0)), 21, 42})
    # the oracle's own copies, taken before the first step
    host = {}
    for li, m in enumerate(eager):
        every = m.window > 0 or li == last_full
        host[li] = sub_layer(m, range(B) if every else seqs)
        host[li]["rows"] = list(range(B)) if every else seqs

    # seeded inputs of every step, resident on the device: [steps][B][...]
    gen = torch.Generator(device=dev).manual_seed(c["seed"] + 5)
    pools = []
    for m in eager:
        qs = torch.randn((steps,) + tuple(m.q.shape), generator=gen, device=dev).bfloat16()
        ks = torch.randn((steps,) + tuple(m.k_new.shape), generator=gen, device=dev).bfloat16()
        vs = torch.randn((steps,) + tuple(m.v_new.shape), generator=gen, device=dev).bfloat16()
        pools.append((qs, ks, vs))
    ws_bytes = max(lib.workspace_bytes(m.q, m.k_cache, m.v_cache, m.block_table, m.window)
                   for m in eager)

    def runner(model):
        lens = model[0].seq_lens.clone()
        step_idx = torch.zeros(1, dtype=torch.int64, device=dev)
        bufs = [(torch.empty((1,) + tuple(m.q.shape), dtype=torch.bfloat16, device=dev),
                 torch.empty((1,) + tuple(m.k_new.shape), dtype=torch.bfloat16, device=dev),
                 torch.empty((1,) + tuple(m.v_new.shape), dtype=torch.bfloat16, device=dev))
                for m in model]
        outs = [torch.empty_like(m.q) for m in model]
        ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

        def step():
            for m, (qs, ks, vs), (qb, kb, vb), o in zip(model, pools, bufs, outs):
                torch.index_select(qs, 0, step_idx, out=qb)
                torch.index_select(ks, 0, step_idx, out=kb)
                torch.index_select(vs, 0, step_idx, out=vb)
                lib.decode_attention_append(qb[0], kb[0], vb[0], m.k_cache, m.v_cache,
                                            m.block_table, lens, m.sinks, m.window, out=o,
                                            workspace=ws)
            lens.add_(1)
            step_idx.add_(1)
        return step, lens, step_idx, outs

    e_step, e_lens, _, e_outs = runner(eager)
    g_step, g_lens, g_idx, g_outs = runner(graph)
    g_start = g_lens.clone()
    graph_obj = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_obj):
        g_step()
    torch.cuda.synchronize()
    g_lens.copy_(g_start)                    # capture records the step, it does not run it
    g_idx.zero_()
    torch.cuda.synchronize()

    got = {}                                 # (step, layer) -> host output of the graph run
    for t in range(steps):
        e_step()
        torch.cuda.synchronize()
        graph_obj.replay()
        torch.cuda.synchronize()
        assert torch.equal(e_lens, g_lens), f"step {t}: lengths"
        for li in range(layers):
            assert torch.equal(e_outs[li], g_outs[li]), f"step {t} layer {li}: graph != eager"
        if t in CHECK_STEPS:
            for li in range(layers):
                got[(t, li)] = out_f64(g_outs[li])
        # unrelated eager work between replays
        torch.randn(1 << 20, device=dev).sum().item()
    for li in range(layers):
        assert torch.equal(eager[li].k_cache, graph[li].k_cache), f"layer {li}: K pools"
        assert torch.equal(eager[li].v_cache, graph[li].v_cache), f"layer {li}: V pools"
    del graph, g_outs, graph_obj
    torch.cuda.empty_cache()

    # the oracle: every step's append on its copies, attention at the checkpoints
    lens0 = L0 + 1
    for li in range(layers):
        h = host[li]
        rows = h["rows"]
        sel = torch.as_tensor(rows, device=dev)
        qs, ks, vs = pools[li]
        window = eager[li].window
        for t in range(steps):
            lens = lens0[rows] + t
            oracle_append(h, bits(ks[t].index_select(0, sel)), bits(vs[t].index_select(0, sel)),
                          lens, window, 16)
            if t not in CHECK_STEPS:
                continue
            # which of this copy's rows to check: all of them, except in the
            # last full layer before the last step (the sampled sequences)
            idx = list(range(len(rows)))
            if window == 0 and len(rows) == B and t != CHECK_STEPS[-1]:
                idx = seqs
            q_t = bits(qs[t].index_select(0, torch.as_tensor([rows[i] for i in idx], device=dev)))
            ref = oracle.decode_attention(q_t, h["k"], h["v"], h["bt"][idx], lens[idx],
                                          h["sinks"], window)
            assert_parity(got[(t, li)][[rows[i] for i in idx]], ref,
                          f"decode loop step {t} layer {li}")
        now = sub_layer(eager[li], rows)
        assert np.array_equal(now["k"], h["k"]), f"layer {li}: K pool after the last step"
        assert np.array_equal(now["v"], h["v"]), f"layer {li}: V pool after the last step"
