"""Helpers shared by the GPU tests: run the HIP path, run the oracle on the
same bits, compare to the stated tolerance.

Tolerance for attention outputs (bf16 inputs, fp32 accumulation, bf16
output) against the fp64 oracle: max-abs <= 2e-2 and mean-abs <= 2e-3 over
all compared elements.  Appends and block-table indexing are bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def bits(t):
    return synth.to_bits(t)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, \
        f"{what}: max-abs {mx:.3e} (<= {MAX_ABS}), mean-abs {mean:.3e} (<= {MEAN_ABS})"
    return mx, mean


def sub_layer(layer: synth.Layer, seqs):
    """Host copies of the inputs of a subset of sequences, with the pool cut
    down to the blocks those sequences own (table entries remapped; unused
    entries point at a copy of the poison block).  Lets the oracle check
    sampled sequences of a workload too large to copy whole."""
    seqs = list(seqs)
    bt = layer.block_table.cpu().numpy()
    owned = [bt[b, :layer.blocks_per_seq[b]] for b in seqs]
    ids = np.concatenate(owned + [np.array([layer.poison_block])]).astype(np.int64)
    idx = torch.as_tensor(ids, device=layer.k_cache.device)
    k = bits(layer.k_cache.index_select(0, idx))
    v = bits(layer.v_cache.index_select(0, idx))
    new_bt = np.full((len(seqs), bt.shape[1]), len(ids) - 1, dtype=np.int32)
    start = 0
    for i, o in enumerate(owned):
        new_bt[i, :len(o)] = np.arange(start, start + len(o))
        start += len(o)
    sel = torch.as_tensor(seqs, device=layer.q.device)
    return dict(q=bits(layer.q.index_select(0, sel)), k=k, v=v, bt=new_bt,
                lens=layer.seq_lens.cpu().numpy()[seqs],
                sinks=None if layer.sinks is None else layer.sinks.cpu().numpy(),
                k_new=bits(layer.k_new.index_select(0, sel)),
                v_new=bits(layer.v_new.index_select(0, sel)))


def oracle_attention(layer: synth.Layer, seqs=None, after_append=False):
    """fp64 oracle output for the given sequences (all by default).  With
    ``after_append`` the oracle first applies its own append of k_new/v_new to
    its copy of the pool."""
    seqs = range(layer.batch) if seqs is None else seqs
    s = sub_layer(layer, seqs)
    k, v = s["k"], s["v"]
    if after_append:
        k, v = oracle.kv_append(k, v, s["k_new"], s["v_new"], s["bt"], s["lens"], layer.window)
    return oracle.decode_attention(s["q"], k, v, s["bt"], s["lens"], s["sinks"], layer.window)


def poison_tails(layer: synth.Layer, value_bits: int = 0x7FC0):
    """Fill every slot past each sequence's attended range, inside the blocks
    it owns, with ``value_bits`` (default: a bf16 NaN).  Test-side layout
    arithmetic: slot s of sequence b is block_table[b][s // bs], offset s % bs."""
    bs = layer.block_size
    bt = layer.block_table.cpu()
    lens = layer.seq_lens.cpu()
    kv = layer.k_cache.view(torch.int16)
    vv = layer.v_cache.view(torch.int16)
    val = np.int16(np.uint16(value_bits).view(np.int16))
    blks, offs = [], []
    for b in range(layer.batch):
        n = int(lens[b]) if layer.window <= 0 else min(int(lens[b]), layer.window)
        for slot in range(n, layer.blocks_per_seq[b] * bs):
            blks.append(int(bt[b, slot // bs]))
            offs.append(slot % bs)
    if not blks:
        return
    bi = torch.as_tensor(blks, device=kv.device)
    oi = torch.as_tensor(offs, device=kv.device)
    kv[bi, :, :, oi, :] = int(val)
    vv[bi, :, oi // 8, :, oi % 8] = int(val)
