"""The decode step with the rotary embedding fused in, on the GPU.

For both pairings, every MFMA variant and several split counts, on paged and
ring layers: the pools after the call hold exactly the oracle's rotated keys
(bit for bit: both sides round the rotation in float32 step by step), the
output is within tolerance of the oracle, and it is bit-identical to the plain
fused step run on inputs the oracle rotated on the host (so the kernel's query
rotation produced the same bits too)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import assert_parity, bits, out_f64, sub_layer

pytestmark = pytest.mark.gpu

STYLES = {"half": 0, "interleaved": 1}
MFMA_VARIANTS = [0, 1, 2, 4, 5]


def angle_tables(P, D=64, base=10000.0, device="cuda"):
    inv = base ** (-np.arange(D // 2, dtype=np.float64) * 2.0 / D)
    ang = np.arange(P, dtype=np.float64)[:, None] * inv[None, :]
    c = torch.from_numpy(np.cos(ang).astype(np.float32)).to(device)
    s = torch.from_numpy(np.sin(ang).astype(np.float32)).to(device)
    return c, s


def from_bits(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def host_layer(layer):
    """Host copies (bf16 bits) of a whole layer, pools as they are on the device."""
    return dict(q=bits(layer.q), k=bits(layer.k_cache), v=bits(layer.v_cache),
                k_new=bits(layer.k_new), v_new=bits(layer.v_new), bt=bits(layer.block_table),
                lens=bits(layer.seq_lens),
                sinks=None if layer.sinks is None else layer.sinks.cpu().numpy())


def oracle_step(layer, cos_t, sin_t, style, compact=False):
    """The oracle's step on host copies: the whole pools, or (compact) only
    the blocks the sequences own, as sub_layer lays them out."""
    s = sub_layer(layer, range(layer.batch)) if compact else host_layer(layer)
    return s, oracle.rope.decode_step_rope(s["q"], s["k"], s["v"], s["k_new"], s["v_new"], s["bt"],
                                           s["lens"], s["sinks"], layer.window,
                                           cos_t.cpu().numpy(), sin_t.cpu().numpy(), style)


def run_rope(lib, layer, kc, vc, cos_t, sin_t, style, num_splits=0, variant=0):
    out = lib.decode_attention_append_rope(layer.q, layer.k_new, layer.v_new, kc, vc,
                                           layer.block_table, layer.seq_lens, cos_t, sin_t,
                                           style=STYLES[style], sinks=layer.sinks,
                                           window=layer.window, num_splits=num_splits,
                                           variant=variant)
    torch.cuda.synchronize()
    return out


def check(lib, layer, cos_t, sin_t, style, splits=(0, 1, 3), variants=MFMA_VARIANTS, what=""):
    s, (k_ref, v_ref, out_ref) = oracle_step(layer, cos_t, sin_t, style)
    # host-rotated inputs for the plain fused step
    pos = np.maximum(s["lens"].astype(np.int64) - 1, 0)[:, None]
    q_rot = from_bits(oracle.rope.rope_bf16(s["q"], pos, cos_t.cpu().numpy(),
                                            sin_t.cpu().numpy(), style))
    k_rot = from_bits(oracle.rope.rope_bf16(s["k_new"], pos, cos_t.cpu().numpy(),
                                            sin_t.cpu().numpy(), style))
    for v in variants:
        for S in splits:
            tag = f"{what} {style} S={S} v={v}"
            kc, vc = layer.k_cache.clone(), layer.v_cache.clone()
            got = run_rope(lib, layer, kc, vc, cos_t, sin_t, style, S, v)
            assert np.array_equal(bits(kc), k_ref), f"{tag}: K pool differs from the oracle"
            assert np.array_equal(bits(vc), v_ref), f"{tag}: V pool differs from the oracle"
            assert_parity(out_f64(got), out_ref, tag)
            kc2, vc2 = layer.k_cache.clone(), layer.v_cache.clone()
            plain = lib.decode_attention_append(q_rot, k_rot, layer.v_new, kc2, vc2,
                                                layer.block_table, layer.seq_lens, layer.sinks,
                                                layer.window, num_splits=S, variant=v)
            torch.cuda.synchronize()
            assert torch.equal(got, plain), f"{tag}: differs from the step on host-rotated inputs"


@pytest.mark.parametrize("style", list(STYLES))
@pytest.mark.parametrize("window", [0, 128, 100])
def test_rope_step(lib, style, window):
    lens = [1, 2, 15, 16, 17, 38, 129, 700, 3001]
    layer = synth.make_layer(batch=len(lens), q_heads=32, kv_heads=4, head_dim=64,
                             block_size=16, lens=lens, window=window, seed=7000 + window,
                             device="cuda")
    cos_t, sin_t = angle_tables(4096)
    check(lib, layer, cos_t, sin_t, style, what=f"W={window}")


@pytest.mark.parametrize("style", list(STYLES))
@pytest.mark.parametrize("bs", [8, 32, 64])
def test_rope_block_sizes(lib, style, bs):
    lens = [5, bs, bs + 1, 300]
    layer = synth.make_layer(batch=len(lens), q_heads=16, kv_heads=2, head_dim=64,
                             block_size=bs, lens=lens, seed=7100 + bs, device="cuda")
    cos_t, sin_t = angle_tables(512, base=500000.0)
    check(lib, layer, cos_t, sin_t, style, splits=(0, 2), what=f"bs={bs}")


@pytest.mark.parametrize("style", list(STYLES))
def test_rope_positions_past_the_table(lib, style):
    """Positions past the tables' last row use that row (both sides)."""
    lens = [40, 100, 7]
    layer = synth.make_layer(batch=3, q_heads=16, kv_heads=2, head_dim=64, block_size=16,
                             lens=lens, seed=7200, device="cuda")
    cos_t, sin_t = angle_tables(32)
    check(lib, layer, cos_t, sin_t, style, splits=(0,), variants=[0, 4, 5], what="table end")


def test_rope_ragged_batch64(lib):
    """Batch 64, ragged 513..8193, the default launch: every sequence, pools bit for bit."""
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
    for style, w in (("half", 0), ("interleaved", 128)):
        layer = synth.make_layer(batch=64, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                                 lens=lens, window=w, seed=c["seed"] + 40 + w, device="cuda")
        cos_t, sin_t = angle_tables(8200)
        s, (k_ref, v_ref, out_ref) = oracle_step(layer, cos_t, sin_t, style, compact=True)
        out = run_rope(lib, layer, layer.k_cache, layer.v_cache, cos_t, sin_t, style)
        after = sub_layer(layer, range(64))
        assert np.array_equal(after["k"], k_ref) and np.array_equal(after["v"], v_ref)
        assert_parity(out_f64(out), out_ref, f"ragged rope {style} W={w}")
