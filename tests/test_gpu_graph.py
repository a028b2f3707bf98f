"""The decode step captured in a HIP graph: replays match eager execution.

Each replay is checked against the eager result of the same step, with eager
work and synchronisations between replays (a graph node that misbehaves only
on later replays would show up here)."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def build_model(layers, B, seed, steps):
    lens0 = synth.ragged_lengths(seed, B, 100, 3000)
    model = [synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                              lens=lens0 + 1, capacity=lens0 + steps + 1,
                              window=128 if li % 2 == 0 else 0, seed=seed * 10 + li,
                              device="cuda") for li in range(layers)]
    return model, model[0].seq_lens.clone()


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_equals_eager(lib, fused):
    steps, layers, B = 4, 4, 8
    eager, lens_e = build_model(layers, B, 77, steps)
    graph_m, lens_g = build_model(layers, B, 77, steps)
    ws_e = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    ws_g = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    outs_e = [torch.empty_like(m.q) for m in eager]
    outs_g = [torch.empty_like(m.q) for m in graph_m]

    def step(model, lens, outs, ws):
        for m, o in zip(model, outs):
            if fused:
                lib.decode_attention_append(m.q, m.k_new, m.v_new, m.k_cache, m.v_cache,
                                            m.block_table, lens, m.sinks, m.window, out=o,
                                            workspace=ws)
                continue
            lib.kv_append(m.k_new, m.v_new, m.k_cache, m.v_cache, m.block_table, lens, m.window)
            lib.decode_attention(m.q, m.k_cache, m.v_cache, m.block_table, lens, m.sinks,
                                 m.window, out=o, workspace=ws)
        lens.add_(1)

    g = torch.cuda.CUDAGraph()
    start = lens_g.clone()
    with torch.cuda.graph(g):
        step(graph_m, lens_g, outs_g, ws_g)
    torch.cuda.synchronize()
    lens_g.copy_(start)                       # capture does not execute the step
    for t in range(steps):
        step(eager, lens_e, outs_e, ws_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lens_e, lens_g)
        for li in range(layers):
            assert torch.equal(outs_e[li], outs_g[li]), f"step {t} layer {li}"
            assert torch.equal(eager[li].k_cache, graph_m[li].k_cache), f"K cache step {t}"
            assert torch.equal(eager[li].v_cache, graph_m[li].v_cache), f"V cache step {t}"
        # unrelated eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()
