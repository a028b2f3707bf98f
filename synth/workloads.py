"""Seeded synthetic decode-step workloads.

What is drawn (no attention arithmetic happens here):

* ``q``       bf16 ``[B][Hq][D]``, N(0,1) times ``scale``;
* ``k_new``, ``v_new``  bf16 ``[B][Hkv][D]``, N(0,1) times ``scale``;
* ``sinks``   fp32 ``[Hq]``, N(0,1) (or ``None``);
* the KV pools, bf16, every element N(0,1) times ``scale``:
  ``k_cache [NB][Hkv][2][bs][D/2]`` and ``v_cache [NB][Hkv][bs/8][D][8]``
  (the library's layouts: each K row in two halves of D/2 dimensions, each
  half slot-major; V transposed inside a block in chunks of 8 slots);
* ``block_table`` int32 ``[B][MBS]``: each sequence owns ``ceil(cap/bs)``
  distinct physical blocks (``cap`` = its capacity in tokens for a paged
  layer, the window for a ring layer), drawn from a seeded permutation of the
  pool (or assigned in order for the ``identity`` control); unused entries
  name one poison block filled with a large finite value, so an over-read
  shows up as a wrong value, never as a fault;
* ``seq_lens`` int32 ``[B]``, given by the caller (lengths after the append).

Small tensors and pools under ``_DEVICE_POOL_ELEMS`` elements are drawn with
a CPU ``torch.Generator`` and copied to ``device``, so a seed gives the same
bits on every machine; larger pools are drawn by a generator on ``device``
(deterministic for a seed and a device type).  Values are fp32 draws rounded
to bf16 (round to nearest even) by ``Tensor.to``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Pools with more elements than this are drawn on the target device.
_DEVICE_POOL_ELEMS = 1 << 27
# Elements drawn per chunk (bounds the fp32 temporary).
_CHUNK_ELEMS = 1 << 26


@dataclasses.dataclass
class Layer:
    """One attention layer's inputs for one decode step."""
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    sinks: Optional[torch.Tensor]
    window: int
    block_size: int
    poison_block: int
    blocks_per_seq: list

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def q_heads(self):
        return self.q.shape[1]

    @property
    def kv_heads(self):
        return self.k_cache.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def max_blocks_per_seq(self):
        return self.block_table.shape[1]

    def to(self, device):
        kw = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for k, v in kw.items():
            if isinstance(v, torch.Tensor):
                kw[k] = v.to(device)
        return Layer(**kw)


def _seeds(seed: int, n: int):
    return [int(s) for s in np.random.SeedSequence(seed).generate_state(n)]


def _normal_bf16(shape, seed, scale, device):
    g = torch.Generator(device=device).manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for start in range(0, flat.numel(), _CHUNK_ELEMS):
        n = min(_CHUNK_ELEMS, flat.numel() - start)
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device)
        if scale != 1.0:
            x.mul_(scale)
        flat[start:start + n] = x.to(torch.bfloat16)
    return out


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """``batch`` integers uniform in [lo, hi] (both ends included)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=batch).astype(np.int64)


def make_layer(*, batch, q_heads, kv_heads, head_dim=64, block_size=16, lens,
               window=0, capacity=None, max_blocks_per_seq=None, seed,
               device="cpu", scale=1.0, sinks=True, table="shuffled",
               guard_blocks=2, poison=64.0) -> Layer:
    """Draw one layer's inputs.

    ``lens`` are the sequence lengths after this step's append.  ``capacity``
    (tokens per sequence, default ``lens``) sizes each paged sequence's
    blocks, e.g. to leave room for later steps of a decode loop; a ring layer
    (``window > 0``) always owns ``ceil(window/block_size)`` blocks.
    """
    lens = np.asarray(lens, dtype=np.int64).reshape(-1)
    assert lens.shape[0] == batch
    cap = lens if capacity is None else np.asarray(capacity, dtype=np.int64).reshape(-1)
    if window > 0:
        nblk = [math.ceil(window / block_size)] * batch
    else:
        nblk = [max(1, math.ceil(int(c) / block_size)) for c in cap]
    mbs = max(nblk) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    assert mbs >= max(nblk)
    used = int(sum(nblk))
    nb = used + 1 + guard_blocks
    s = _seeds(seed, 8)

    # block table: a seeded permutation (or the identity) of the pool
    if table == "shuffled":
        perm = torch.randperm(nb, generator=torch.Generator().manual_seed(s[0]))
    elif table == "identity":
        perm = torch.arange(nb)
    else:
        raise ValueError(table)
    poison_block = int(perm[used])
    bt = torch.full((batch, mbs), poison_block, dtype=torch.int32)
    start = 0
    for b in range(batch):
        bt[b, :nblk[b]] = perm[start:start + nblk[b]].to(torch.int32)
        start += nblk[b]

    # pools
    elems = nb * kv_heads * block_size * head_dim
    dev = torch.device(device)
    pool_dev = dev if (dev.type != "cpu" and elems > _DEVICE_POOL_ELEMS) else torch.device("cpu")
    # K rows in two halves, each half slot-major; V in chunks of 8 slots
    k_cache = _normal_bf16((nb, kv_heads, 2, block_size, head_dim // 2), s[1], scale, pool_dev)
    v_cache = _normal_bf16((nb, kv_heads, block_size // 8, head_dim, 8), s[2], scale, pool_dev)
    k_cache[poison_block].fill_(poison)
    v_cache[poison_block].fill_(-poison)

    q = _normal_bf16((batch, q_heads, head_dim), s[3], scale, "cpu")
    k_new = _normal_bf16((batch, kv_heads, head_dim), s[4], scale, "cpu")
    v_new = _normal_bf16((batch, kv_heads, head_dim), s[5], scale, "cpu")
    snk = None
    if sinks:
        snk = torch.randn(q_heads, generator=torch.Generator().manual_seed(s[6]),
                          dtype=torch.float32)
    layer = Layer(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                  block_table=bt, seq_lens=torch.as_tensor(lens, dtype=torch.int32),
                  sinks=snk, window=int(window), block_size=block_size,
                  poison_block=poison_block, blocks_per_seq=nblk)
    return layer.to(dev)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as its uint16 bit patterns (other dtypes are
    copied as they are)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy().copy()
    return t.numpy().copy()


# The workloads the decode step is measured and checked on.  Lengths are the
# context after this step's append unless stated.
CONFIGS = {
    # batch 1, 4 query heads / 1 KV head, D 64, 37 cached tokens + 1 appended
    "tiny": dict(batch=1, q_heads=4, kv_heads=1, head_dim=64, block_size=16,
                 lens=[38], window=0, seed=1001),
    # one gpt-oss-shaped layer: batch 1, 64/8 heads, context 8192, inputs
    # scaled by 1/sqrt(64)
    "gptoss_layer_8k": dict(batch=1, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                            lens=[8192], window=0, seed=1002, scale=0.125),
    # batch 64, ragged context 512..8192 (+1 appended), paged full layer and a
    # sliding-window-128 ring layer
    "batch64_ragged": dict(batch=64, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                           len_range=(512, 8192), windows=(0, 128), seed=1003),
    # long context: batch 1 and 8 at 131072
    "long_131k_b1": dict(batch=1, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                         lens=[131072], window=0, seed=1004),
    "long_131k_b8": dict(batch=8, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                         lens=[131072] * 8, window=0, seed=1005),
    # one GPU's share of long_131k_b8 with the KV heads split over 8 GPUs
    # (tensor parallelism): 8 query heads / 1 KV head per GPU
    "long_131k_b8_tp_share": dict(batch=8, q_heads=8, kv_heads=1, head_dim=64, block_size=16,
                                  lens=[131072] * 8, window=0, seed=1008),
    # decode loop: 24 layers alternating ring-128 / full, batch 64, initial
    # ragged lengths 1024..32768, 50 steps of one appended token per sequence
    "decode_loop": dict(batch=64, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                        len_range=(1024, 32768), layers=24, steps=50, window=128,
                        seed=1006),
    # uniform batch 64 x 8192, the bandwidth headline point
    "batch64_8k": dict(batch=64, q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                       lens=[8192] * 64, window=0, seed=1007),
}
