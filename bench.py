#!/usr/bin/env python3
"""Benchmark of the decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batch64_8k]
                    [--configs all|none] [--graph]

A step is one pass of the whole hot path over one batch.  For the default
workload (batch64_8k, the metric's "batch 64, 8k ctx") it is one call that
appends each sequence's new K/V row and attends over the paged cache: 64
sequences of 8192 tokens (the new one included), 64 query / 8 KV heads, D 64,
block size 16, a shuffled block table, learned sinks, split-K partitions and
their merge.  ``--workload batch64_ragged`` times the two-layer step instead
(a paged full layer and a sliding-window-128 ring layer, ragged contexts
512..8192 plus the appended token).  Inputs are seeded synthetic bf16 N(0,1)
values, resident in HBM before timing starts.

Reported (one JSON line):
  value        the step's algorithmic bytes / its time (GB/s).  An attention
               call moves 2048 B per attended token (K and V rows of 8 KV heads
               x 64 dims x bf16) plus 16 KiB per sequence (its bf16 query and
               output rows); an append moves 4 KiB per sequence (read and write
               of K and V rows).
  roofline     the dominant call (the full-layer attention), timed with HIP
               events on the stream it runs on, back to back: the whole call,
               and its decode kernel alone from the profiler's device trace.
  cpu_baseline the fp64 oracle on this host's cores (a pool of worker
               processes), on the same step.
  batch64_ragged_step  the two-layer ragged step, timed the same way.  The
               ring layer's pools (18 MB) would stay in the 256 MB Infinity
               Cache from one step to the next; it rotates over enough input
               sets that every step reads it from HBM, as a model with many
               layers would.
  configs      every synthetic configuration: GPU us per call, GB/s and
               fraction of peak, next to the oracle's seconds on the same
               inputs.  Calls whose inputs fit the 256 MB Infinity Cache rotate
               several input sets so every call reads HBM.
"""

from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import math
import os
import statistics
import sys
import tempfile
import time

_ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, _ROOT)

PEAK_HBM = 8.0e12            # MI355X HBM3E, bytes/s
MALL_BYTES = 256 << 20       # Infinity Cache
ROUNDS = 5                   # further timing rounds per call, for the spread
METRIC = "decode-attn µs/call + achieved HBM GB/s (% of peak), batch 64, 8k ctx"
# sources of the dominant call's kernels; the committed counter summary is
# valid only for the exact sources it was taken on
KERNEL_SRCS = [os.path.join(_ROOT, "paged_gqa_decode_step_amd", "csrc", f)
               for f in ("decode_stream.hip", "mfma_attend.h", "sa_internal.h", "plan.h")]
# the bench's step workloads: name -> context lengths (after the append)
HEADLINE = "batch64_8k"
STEP_WORKLOADS = {"batch64_8k": "8192 for every sequence",
                  "batch64_ragged": "1 + U{512..8192} per sequence"}
APPEND_WORKLOADS = ("batch64_8k", "batch64_ragged")


def attn_bytes(lens, window, q_heads=64, kv_heads=8, head_dim=64):
    n = [min(int(L), window) if window > 0 else int(L) for L in lens]
    return sum(n) * kv_heads * head_dim * 2 * 2 + len(lens) * q_heads * head_dim * 2 * 2


def append_bytes(batch, kv_heads=8, head_dim=64):
    return batch * kv_heads * head_dim * 2 * 2 * 2


def source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(workload):
    return os.path.join(_ROOT, "profiles", f"decode_attention_{workload}_traffic.json")


def load_traffic(workload):
    """Per-launch HBM bytes of the workload's dominant call from the committed
    counter summary, or None if there is none or the kernel sources changed
    since."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_digest():
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def ragged_layers(device, seed_offset=0, windows=(0, 128)):
    import synth
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
    common = dict(batch=c["batch"], q_heads=c["q_heads"], kv_heads=c["kv_heads"],
                  head_dim=c["head_dim"], block_size=c["block_size"], lens=lens, device=device)
    seed = {0: c["seed"] + 10, 128: c["seed"] + 20}
    return [synth.make_layer(window=w, seed=seed[w] + seed_offset, **common) for w in windows]


def make_workload(name, device, seed_offset=0):
    import synth
    if name == "batch64_ragged":
        return ragged_layers(device, seed_offset)
    if name in ("tiny", "batch64_8k", "gptoss_layer_8k", "long_131k_b1", "long_131k_b8",
                "long_131k_b8_tp_share"):
        c = dict(synth.CONFIGS[name])
        c["seed"] += seed_offset
        return [synth.make_layer(device=device, **c)]
    raise SystemExit(f"unknown workload {name}")


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

class Timer:
    """HIP-event timing on one stream.  ``settle`` runs the measured call until
    it has kept the GPU busy for SETTLE_S seconds: after host-side work the
    GPU's clocks drop and take that long to return, and a short warmup would
    time the ramp instead of the steady state."""
    SETTLE_S = 0.1

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def settle(self, fn, min_reps):
        done, elapsed_us = 0, 0.0
        while done < min_reps or elapsed_us < self.SETTLE_S * 1e6:
            n = max(min_reps, 8)
            elapsed_us += self.mean_us(fn, n) * n
            done += n

    def mean_us(self, fn, reps):
        """Mean microseconds of fn over reps back-to-back runs on the stream,
        bracketed by two HIP events (none in between, so no event gap)."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for i in range(reps):
            fn(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def per_call_us(self, fn, reps):
        """Microseconds of each of reps back-to-back runs, one HIP event after
        every run.  Each event marker adds a small gap of its own, so these
        sit slightly above the mean of ``mean_us``; they give the spread."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(reps):
            fn(i)
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]


def spread(times_us):
    """Median, 10th and 90th percentile of per-call times."""
    q = statistics.quantiles(times_us, n=10, method="inclusive")
    return dict(calls=len(times_us), us_median=round(statistics.median(times_us), 2),
                us_p10=round(q[0], 2), us_p90=round(q[-1], 2))


@contextlib.contextmanager
def one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        yield
        return
    with threadpool_limits(limits=1):
        yield


def host_inputs(layer, seqs=None):
    """Host copies (bf16 bits) of a layer's inputs; with ``seqs`` only those
    sequences, their pool blocks and a remapped table."""
    import numpy as np
    import synth
    import torch
    if seqs is None:
        return dict(q=synth.to_bits(layer.q), k=synth.to_bits(layer.k_cache),
                    v=synth.to_bits(layer.v_cache), bt=synth.to_bits(layer.block_table),
                    lens=synth.to_bits(layer.seq_lens), kn=synth.to_bits(layer.k_new),
                    vn=synth.to_bits(layer.v_new),
                    sinks=None if layer.sinks is None else layer.sinks.cpu().numpy(),
                    w=layer.window)
    bt = layer.block_table.cpu().numpy()
    owned = [bt[b, :layer.blocks_per_seq[b]] for b in seqs]
    ids = np.concatenate(owned + [np.array([layer.poison_block])]).astype(np.int64)
    idx = torch.as_tensor(ids, device=layer.k_cache.device)
    new_bt = np.full((len(seqs), bt.shape[1]), len(ids) - 1, dtype=np.int32)
    start = 0
    for i, o in enumerate(owned):
        new_bt[i, :len(o)] = np.arange(start, start + len(o))
        start += len(o)
    sel = torch.as_tensor(list(seqs), device=layer.q.device)
    return dict(q=synth.to_bits(layer.q.index_select(0, sel)),
                k=synth.to_bits(layer.k_cache.index_select(0, idx)),
                v=synth.to_bits(layer.v_cache.index_select(0, idx)), bt=new_bt,
                lens=layer.seq_lens.cpu().numpy()[list(seqs)],
                kn=synth.to_bits(layer.k_new.index_select(0, sel)),
                vn=synth.to_bits(layer.v_new.index_select(0, sel)),
                sinks=None if layer.sinks is None else layer.sinks.cpu().numpy(),
                w=layer.window)


# ---------------------------------------------------------------------------
# the fp64 oracle on this host's cores (reported baseline, never the GPU path)
# ---------------------------------------------------------------------------

_ARRAYS = ("q", "k", "v", "bt", "lens", "kn", "vn", "sinks")


def _oracle_warm(_):
    """Worker start-up: import NumPy and the oracle before anything is timed."""
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    return os.getpid()


def _oracle_task(task):
    """One worker's share of an oracle call: the fp64 oracle's append (when
    asked) and attention for some sequences and KV heads of a call whose host
    inputs sit in .npy files (memory-mapped, not copied).  The share's pool
    blocks and query heads are cut out first (data movement only: the oracle
    reads the same rows through a remapped table)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    path, seqs, g0, g1, append, window = task
    a = {n: np.load(os.path.join(path, n + ".npy"), mmap_mode="r")
         for n in _ARRAYS if os.path.exists(os.path.join(path, n + ".npy"))}
    bs = a["k"].shape[3]
    Hq, Hkv = a["q"].shape[1], a["k"].shape[1]
    G = Hq // Hkv
    with threadpool_limits(limits=1):
        lens = np.asarray(a["lens"])[seqs]
        bt = np.asarray(a["bt"])[seqs]
        # table entries covering each sequence's attended slots (the new
        # token's slot among them)
        att = [min(int(L), window) if window > 0 else int(L) for L in lens]
        need = [min(max(1, -(-n // bs)), bt.shape[1]) for n in att]
        ids = np.concatenate([bt[i, :n] for i, n in enumerate(need)]).astype(np.int64)
        sub_bt = np.zeros_like(bt)
        start = 0
        for i, n in enumerate(need):
            sub_bt[i, :n] = np.arange(start, start + n)
            start += n
        k = np.asarray(a["k"][ids, g0:g1])
        v = np.asarray(a["v"][ids, g0:g1])
        q = np.asarray(a["q"])[seqs, g0 * G:g1 * G]
        sinks = None if "sinks" not in a else np.asarray(a["sinks"])[g0 * G:g1 * G]
        if append:
            kn = np.asarray(a["kn"])[seqs, g0:g1]
            vn = np.asarray(a["vn"])[seqs, g0:g1]
            k, v = oracle.kv_append(k, v, kn, vn, sub_bt, lens, window)
        out = oracle.decode_attention(q, k, v, sub_bt, lens, sinks, window)
    return out


class HostOracle:
    """The fp64 oracle timed on this host's cores: a pool of spawned worker
    processes (NumPy and the oracle only; BLAS held to one thread in each),
    every call's sequences (or, for fewer sequences than workers, its
    (sequence, KV head) pairs) shared out among them.  The inputs are staged
    once as .npy files that the workers memory-map; the timed region is the
    pool's whole run over the call."""

    def __init__(self, workers=None):
        import concurrent.futures as cf
        import multiprocessing as mp
        avail = len(os.sched_getaffinity(0))
        # at most 16: the CPU share of one GPU on the boxes this runs on
        self.workers = max(1, min(16, avail) if workers is None else workers)
        self.dir = tempfile.TemporaryDirectory(prefix="sa_oracle_")
        self.pool = cf.ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"))
        self.pids = set(self.pool.map(_oracle_warm, range(4 * self.workers)))
        self.n = 0

    def stage(self, host):
        """Write one call's host inputs (bench's host_inputs dict); returns a
        handle for ``seconds``."""
        import numpy as np
        path = os.path.join(self.dir.name, f"call{self.n}")
        self.n += 1
        os.makedirs(path)
        for n in _ARRAYS:
            if host.get(n) is not None:
                np.save(os.path.join(path, n + ".npy"), np.ascontiguousarray(host[n]))
        return dict(path=path, B=len(host["lens"]), Hkv=host["k"].shape[1], window=host["w"])

    def tasks(self, staged, append):
        out = []
        for c in staged:
            B, Hkv = c["B"], c["Hkv"]
            if B >= self.workers:
                per = -(-B // self.workers)
                for s0 in range(0, B, per):
                    out.append((c["path"], list(range(s0, min(B, s0 + per))), 0, Hkv, append,
                                c["window"]))
            else:
                for b in range(B):
                    for g in range(Hkv):
                        out.append((c["path"], [b], g, g + 1, append, c["window"]))
        return out

    def seconds(self, staged, reps=1, append=False):
        """Median wall seconds of the oracle over the staged calls, run by the
        whole pool."""
        tasks = self.tasks(staged, append)
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            list(self.pool.map(_oracle_task, tasks))
            times.append(time.perf_counter() - t0)
        return statistics.median(times)

    def describe(self):
        import numpy as np
        return (f"NumPy {np.__version__} fp64 oracle, {self.workers} worker processes "
                f"(BLAS 1 thread each) on {len(os.sched_getaffinity(0))} available cores")

    def close(self):
        self.pool.shutdown()
        self.dir.cleanup()


def entry(name, what, us, nbytes, cpu_s=None, cpu_note=None, **extra):
    e = dict(config=name, call=what, us=round(us, 2), bytes=int(nbytes),
             gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
             frac_of_peak=round(nbytes / (us * 1e-6) / PEAK_HBM, 4))
    if cpu_s is not None:
        e["oracle_s"] = round(cpu_s, 4)
        e["oracle_gbps"] = round(nbytes / cpu_s / 1e9, 4)
        e["oracle_sample"] = cpu_note
        e["gpu_speedup_vs_oracle"] = round(cpu_s / (us * 1e-6), 1)
    e.update(extra)
    return e


# ---------------------------------------------------------------------------
# per-configuration measurements
# ---------------------------------------------------------------------------

def attention_config(sa, torch, timer, dev, name, steps, warmup, variant,
                     with_oracle=True, oracle_seqs=None, label=None):
    """One attention call per launch, rotating input sets past the Infinity
    Cache.  Calls too short for Python to keep the GPU fed (under 40 us) are
    timed by replaying a HIP graph of many launches.  Returns the entry and,
    for the oracle timed later, host copies of one input set (or of the given
    sequences)."""
    first = make_workload(name, dev)[0]
    one = attn_bytes(first.seq_lens.cpu().tolist(), first.window, first.q_heads,
                     first.kv_heads, first.head_dim)
    pool = first.k_cache.numel() * 4
    nsets = 1 if pool > 2 * MALL_BYTES else min(64, -(-(3 * MALL_BYTES) // max(pool, 1)))
    sets = [first] + [make_workload(name, dev, seed_offset=101 * i)[0] for i in range(1, nsets)]
    ws = sa.new_workspace(first.q, first.k_cache, first.v_cache, first.block_table,
                          first.window, variant=variant)
    outs = [torch.empty_like(L.q) for L in sets]

    def call(i):
        L = sets[i % len(sets)]
        sa.decode_attention(L.q, L.k_cache, L.v_cache, L.block_table, L.seq_lens, L.sinks,
                            L.window, out=outs[i % len(sets)], workspace=ws, variant=variant)
    timer.settle(call, warmup)
    us = timer.mean_us(call, steps)
    timing = "eager, back to back"
    per_call = None
    if us < 40.0:
        per_graph = max(len(sets), 32)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                call(i)
        reps = max(2, steps // 10)
        timer.settle(lambda _: g.replay(), reps)
        us = timer.mean_us(lambda _: g.replay(), reps) / per_graph
        timing = f"HIP graph of {per_graph} launches, replayed {reps} times"
        del g
    else:
        per_call = spread(timer.per_call_us(call, steps))
    kernels = kernel_times_us(torch, call, steps)
    host = note = None
    if with_oracle:
        B = first.batch
        seqs = oracle_seqs if oracle_seqs is not None else list(range(B))
        host = (host_inputs(first, seqs if len(seqs) < B else None), B / len(seqs), 3)
        note = (f"{len(seqs)} of {B} sequences, scaled x{B / len(seqs):g}" if len(seqs) < B
                else "every sequence")
    e = entry(label or name, "attention", us, one, input_sets=len(sets), timing=timing,
              **({} if per_call is None else {"per_call_events": per_call}),
              splits=sa.num_splits(first.q, first.k_cache, first.v_cache, first.block_table,
                                   first.window, variant=variant), kernels_us=kernels)
    if note:
        e["oracle_sample"] = note
    del sets, outs, ws
    torch.cuda.empty_cache()
    return e, host


def read_ceiling(sa, torch, timer, dev, nbytes=4 << 30):
    """The practical HBM read ceilings: the library's plain streaming-read
    probe over a 4 GiB buffer (far past the Infinity Cache), and its
    scattered-tile probe (the decode kernels' pattern: 2 KiB tiles at random
    places, 1024 wavefronts, 8 KiB steps, three in flight; 1 GiB a call from
    four disjoint sets of tiles in rotation)."""
    import numpy as np
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    x.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    f = lambda _=0: sa.read_bandwidth_probe(x, sink)                      # noqa: E731
    timer.settle(f, 5)
    us = timer.mean_us(f, 20)
    stream = dict(kernel="sa_read_bandwidth_probe (16-byte non-temporal streaming read)",
                  bytes=nbytes, us=round(us, 1), gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
                  frac_of_peak=round(nbytes / (us * 1e-6) / PEAK_HBM, 4))
    ntotal = nbytes // 2048
    perm = np.random.default_rng(7).permutation(ntotal).astype(np.int32)
    nsets = 4
    per = ntotal // nsets
    sets = [torch.from_numpy(perm[i * per:(i + 1) * per].copy()).to(dev) for i in range(nsets)]
    g = lambda i=0: sa.read_tiles_probe(x, sets[i % nsets], sink, waves=1024)   # noqa: E731
    timer.settle(g, 8)
    tus = timer.mean_us(g, 20)
    tb = per * 2048
    tiles = dict(kernel="sa_read_tiles_probe (2 KiB tiles at random places, the decode "
                        "kernels' read pattern with no arithmetic, 1024 wavefronts)",
                 bytes=tb, us=round(tus, 1), gbps=round(tb / (tus * 1e-6) / 1e9, 1),
                 frac_of_peak=round(tb / (tus * 1e-6) / PEAK_HBM, 4))
    del x, sets
    torch.cuda.empty_cache()
    return dict(stream, scattered_tiles=tiles)


BALANCED_WAVES = 1024       # the balanced kernel's width on calls of >= 8192 32-slot steps
TILE_BYTES = 2048           # one (block, KV head) K or V tile: 16 slots x 64 dims x bf16
FLOOR_TILES = 1 << 21       # 2 KiB tiles in the floor probe's 4 GiB buffer


def layer_lens(name):
    """(lens, window, kv_heads) of each attention layer of a named workload,
    from its recipe (no device memory)."""
    import synth
    c = synth.CONFIGS[name]
    if name == "batch64_ragged":
        lens = (synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1).tolist()
        return [(lens, w, c["kv_heads"]) for w in c["windows"]]
    return [(list(c["lens"]), c["window"], c["kv_heads"])]


def floor_tiles(rng, lens, window, kv_heads, balanced, splits, base=0, bs=16):
    """The K/V tiles one attention call reads, as tile numbers in the floor
    probe's buffer, in the order its wavefronts take them; the wavefront count;
    and the tiles its pools span.  As in the cache, the call has a K pool and a
    V pool of its own size (here side by side from tile ``base``), each
    [block][KV head] tiles, so the KV heads of a block sit side by side, and
    the sequences own the pool's blocks in a shuffled order.  Each wavefront's
    stretch alternates a block's K and V tile.  Balanced split: the (sequence,
    KV head) units in order, each unit's blocks in order, cut evenly over the
    kernel's wavefronts.  Static split: partition-major, as the static
    kernel's grid is (partition, sequence, KV head), one wavefront per
    non-empty partition."""
    import numpy as np
    nb = [-(-(min(L, window) if window > 0 else L) // bs) for L in lens]
    pool = sum(nb) * kv_heads                    # tiles in each of the two pools
    if base + 2 * pool > FLOOR_TILES:
        raise ValueError("the call's pools exceed the floor buffer")
    perm = rng.permutation(sum(nb))
    starts = np.cumsum([0] + nb)
    seq_blocks = [perm[starts[b]:starts[b + 1]] for b in range(len(lens))]

    def stretch(blocks, g):
        k = base + blocks.astype(np.int64) * kv_heads + g
        return np.stack([k, k + pool], axis=1).reshape(-1)
    parts = []
    if balanced:
        for blocks in seq_blocks:
            for g in range(kv_heads):
                parts.append(stretch(blocks, g))
        waves = BALANCED_WAVES
    else:
        per = -(-max(nb) // splits)
        for sp in range(splits):
            for blocks in seq_blocks:
                sel = blocks[sp * per:(sp + 1) * per]
                if len(sel):
                    parts += [stretch(sel, g) for g in range(kv_heads)]
        waves = len(parts)
    return np.concatenate(parts).astype(np.int32), waves, 2 * pool


def read_floors(sa, torch, timer, dev, specs, steps, warmup):
    """Each call's own read floor: sa_read_tiles_probe reading exactly the
    call's K/V tiles (floor_tiles: the cache's layout, the kernel's wavefront
    count and order) with no arithmetic, in one launch, timed as the calls are
    (input sets rotated past the Infinity Cache, graphs under 40 us).
    specs: {key: (lens, window, kv_heads, balanced, splits)}."""
    import numpy as np
    x = torch.empty(FLOOR_TILES * TILE_BYTES, dtype=torch.uint8, device=dev)
    x.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    rng = np.random.default_rng(11)
    out = {}
    for key, (lens, window, kvh, balanced, splits) in specs.items():
        try:
            first, waves, span = floor_tiles(rng, lens, window, kvh, balanced, splits)
        except ValueError as exc:            # an annex: the bench line goes on without it
            print(f"# read floor of {key} skipped: {exc}", flush=True)
            continue
        nbytes = int(first.size) * TILE_BYTES
        nsets = 1 if nbytes > 2 * MALL_BYTES else min(64, -(-(3 * MALL_BYTES) // nbytes))
        nsets = min(nsets, FLOOR_TILES // span)    # each set's pools in a place of their own
        if nsets < 1:
            print(f"# read floor of {key} skipped: its pools exceed the floor buffer", flush=True)
            continue
        sets = [torch.from_numpy(first).to(dev)] + [
            torch.from_numpy(floor_tiles(rng, lens, window, kvh, balanced, splits,
                                         base=i * span)[0]).to(dev)
            for i in range(1, nsets)]

        def f(i=0, sets=sets, waves=waves):
            sa.read_tiles_probe(x, sets[i % len(sets)], sink, waves=waves)
        e = time_calls(torch, timer, [(f"read floor of {key}", nbytes, f, nsets)], steps,
                       warmup)[0]
        out[key] = dict(us=e["us_mean"], bytes=nbytes, wavefronts=waves, input_sets=nsets,
                        split="balanced" if balanced else f"static, {splits} a unit",
                        timing=e["timing"])
        del sets
    del x
    torch.cuda.empty_cache()
    return out


def floor_fields(floor, call_us, kernel_us=None):
    """A call's read floor beside its own times: the floor's duration over the
    call's (and over its decode kernel's alone)."""
    r = dict(floor, what="sa_read_tiles_probe over the call's own K/V tiles, no arithmetic",
             call_frac=round(floor["us"] / call_us, 4))
    if kernel_us:
        r["kernel_frac"] = round(floor["us"] / kernel_us, 4)
    return r


def rope_step_config(sa, torch, timer, dev, steps, warmup, variant, with_oracle=True):
    """The batch-64 ragged step (paged full layer + ring-128 layer, append
    inside) with the rotary embedding of q and k_new fused in, beside the same
    step without it on the same inputs."""
    import numpy as np
    layers = make_workload("batch64_ragged", dev)
    P = max(int(L.seq_lens.max()) for L in layers) + 1
    inv = 10000.0 ** (-np.arange(32, dtype=np.float64) * 2.0 / 64)
    ang = np.arange(P, dtype=np.float64)[:, None] * inv[None, :]
    cos_t = torch.from_numpy(np.cos(ang).astype(np.float32)).to(dev)
    sin_t = torch.from_numpy(np.sin(ang).astype(np.float32)).to(dev)
    outs = [torch.empty_like(L.q) for L in layers]
    wss = [sa.new_workspace(L.q, L.k_cache, L.v_cache, L.block_table, L.window, variant=variant)
           for L in layers]

    def step_rope(_=0):
        for L, o, ws in zip(layers, outs, wss):
            sa.decode_attention_append_rope(L.q, L.k_new, L.v_new, L.k_cache, L.v_cache,
                                            L.block_table, L.seq_lens, cos_t, sin_t,
                                            style=sa.ROPE_HALF, sinks=L.sinks, window=L.window,
                                            out=o, workspace=ws, variant=variant)

    def step_plain(_=0):
        for L, o, ws in zip(layers, outs, wss):
            sa.decode_attention_append(L.q, L.k_new, L.v_new, L.k_cache, L.v_cache, L.block_table,
                                       L.seq_lens, L.sinks, L.window, out=o, workspace=ws,
                                       variant=variant)
    nbytes = sum(attn_bytes(L.seq_lens.cpu().tolist(), L.window) + append_bytes(L.batch)
                 for L in layers)
    timer.settle(step_plain, warmup)
    us_plain = timer.mean_us(step_plain, steps)
    timer.settle(step_rope, warmup)
    us_rope = timer.mean_us(step_rope, steps)
    e = entry("batch64_ragged + RoPE", "step (both layers: RoPE, append and attention in one "
              "launch each, half-split pairing)", us_rope, nbytes,
              us_without_rope=round(us_plain, 2),
              rope_overhead=round(us_rope / us_plain - 1.0, 4))
    if with_oracle:
        import oracle
        hs = [host_inputs(L) for L in layers]
        c_np, s_np = cos_t.cpu().numpy(), sin_t.cpu().numpy()
        with one_blas_thread():
            t0 = time.perf_counter()
            for L, h in zip(layers, hs):
                oracle.rope.decode_step_rope(h["q"], h["k"], h["v"], h["kn"], h["vn"], h["bt"],
                                             h["lens"], h["sinks"], h["w"], c_np, s_np, "half")
            cpu_s = time.perf_counter() - t0
        e.update(oracle_s=round(cpu_s, 4), oracle_gbps=round(nbytes / cpu_s / 1e9, 4),
                 oracle_sample="the whole step, once; NumPy fp64 (rotation in float32), 1 thread",
                 gpu_speedup_vs_oracle=round(cpu_s / (us_rope * 1e-6), 1))
    del layers, outs, wss
    torch.cuda.empty_cache()
    return e


def tile_step_config(sa, torch, timer, dev, steps, warmup, variant, T=2, with_oracle=True):
    """Speculative verify / chunked prefill on the batch-64 ragged paged layer:
    T causal query tokens per sequence (T x 8 heads fill the 16 MFMA columns),
    their K/V appended inside the launch, beside the one-token call on the same
    cache."""
    import synth
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + T
    L = synth.make_layer(batch=c["batch"], q_heads=64, kv_heads=8, head_dim=64, block_size=16,
                         lens=lens, seed=c["seed"] + 70, device=dev)
    g = torch.Generator(device=dev).manual_seed(c["seed"] + 71)
    B = c["batch"]
    q = torch.randn(B, T, 64, 64, generator=g, device=dev).to(torch.bfloat16)
    kn = torch.randn(B, T, 8, 64, generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn(B, T, 8, 64, generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    out1 = torch.empty_like(L.q)
    ws = sa.new_workspace(q, L.k_cache, L.v_cache, L.block_table, 0, variant=variant)
    ws1 = sa.new_workspace(L.q, L.k_cache, L.v_cache, L.block_table, 0, variant=variant)

    def tile(_=0):
        sa.decode_attention_append(q, kn, vn, L.k_cache, L.v_cache, L.block_table, L.seq_lens,
                                   L.sinks, 0, out=out, workspace=ws, variant=variant)

    def one(_=0):
        sa.decode_attention_append(L.q, L.k_new, L.v_new, L.k_cache, L.v_cache, L.block_table,
                                   L.seq_lens, L.sinks, 0, out=out1, workspace=ws1,
                                   variant=variant)
    nbytes = (attn_bytes(lens.tolist(), 0) + B * 64 * 64 * 2 * 2 * (T - 1) +
              append_bytes(B) * T)
    timer.settle(one, warmup)
    us_one = timer.mean_us(one, steps)
    timer.settle(tile, warmup)
    us = timer.mean_us(tile, steps)
    e = entry(f"batch64_ragged, {T}-token query tile",
              f"one call: append of {T} rows per sequence and causal attention of {T} query "
              "tokens (paged full layer)", us, nbytes, us_one_token=round(us_one, 2),
              tokens_per_s=round(B * T / (us * 1e-6), 1))
    if with_oracle:
        import oracle
        h = host_inputs(L)
        qb, knb, vnb = synth.to_bits(q), synth.to_bits(kn), synth.to_bits(vn)
        with one_blas_thread():
            t0 = time.perf_counter()
            k2, v2 = oracle.multi_token.kv_append_multi(h["k"], h["v"], knb, vnb, h["bt"],
                                                         h["lens"], 0)
            oracle.multi_token.decode_attention_multi(qb, k2, v2, h["bt"], h["lens"], h["sinks"],
                                                      0)
            cpu_s = time.perf_counter() - t0
        e.update(oracle_s=round(cpu_s, 4), oracle_gbps=round(nbytes / cpu_s / 1e9, 4),
                 oracle_sample="the whole call, once; NumPy fp64, 1 thread",
                 gpu_speedup_vs_oracle=round(cpu_s / (us * 1e-6), 1))
    del L, q, kn, vn, out, out1, ws, ws1
    torch.cuda.empty_cache()
    return e


def add_oracle(e, host, ho):
    """Time the oracle (on the host's cores) on the saved host inputs and add
    it to the entry."""
    h, scale, reps = host
    staged = [ho.stage(h)]
    ho.seconds(staged)                        # first touch of the staged inputs, untimed
    cpu_s = ho.seconds(staged, reps) * scale
    e["oracle_s"] = round(cpu_s, 4)
    e["oracle_gbps"] = round(e["bytes"] / cpu_s / 1e9, 4)
    e["oracle_sample"] += f"; median of {reps}; {ho.describe()}"
    e["gpu_speedup_vs_oracle"] = round(cpu_s / (e["us"] * 1e-6), 1)


def decode_loop_config(sa, torch, timer, dev, stream, variant, layers=24, steps=50,
                       graph=False, oracle_seqs=(0, 21, 42, 63), ho=None, fused=True):
    """The decode loop: 24 layers alternating ring-128 / paged full attention,
    batch 64, initial lengths 1024..32768, 50 steps each appending one token
    per sequence in every layer.  Timed as whole steps (all layers), eagerly
    or replayed from a HIP graph of one step."""
    import synth
    c = synth.CONFIGS["decode_loop"]
    B, W = c["batch"], c["window"]
    L0 = synth.ragged_lengths(c["seed"], B, *c["len_range"])
    model = []
    for li in range(layers):
        w = W if li % 2 == 0 else 0
        model.append(synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64,
                                      block_size=16, lens=L0 + 1, capacity=L0 + steps,
                                      window=w, seed=c["seed"] * 100 + li, device=dev))
    lens = model[0].seq_lens.clone()
    start_lens = lens.clone()
    ws_bytes = max(sa.workspace_bytes(m.q, m.k_cache, m.v_cache, m.block_table, m.window,
                                      variant=variant) for m in model)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(m.q) for m in model]

    def step(_=0):
        # launches go to torch's current stream: the timed stream when eager,
        # the capture stream while a HIP graph is being recorded
        for m, o in zip(model, outs):
            if fused:
                sa.decode_attention_append(m.q, m.k_new, m.v_new, m.k_cache, m.v_cache,
                                           m.block_table, lens, m.sinks, m.window, out=o,
                                           workspace=ws, variant=variant)
                continue
            sa.kv_append(m.k_new, m.v_new, m.k_cache, m.v_cache, m.block_table, lens, m.window)
            sa.decode_attention(m.q, m.k_cache, m.v_cache, m.block_table, lens, m.sinks,
                                m.window, out=o, workspace=ws, variant=variant)
        lens.add_(1)

    # bytes of the timed steps (lengths grow by one each step)
    total = 0
    for t in range(steps):
        cur = (L0 + 1 + t).tolist()
        for m in model:
            total += attn_bytes(cur, m.window) + append_bytes(B)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    lens.copy_(start_lens)
    runner = step
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        lens.copy_(start_lens)
        runner = lambda _=0: g.replay()                                   # noqa: E731
    timer.settle(runner, 4)                  # (its appends only rewrite slots of these steps)
    lens.copy_(start_lens)
    us_step = timer.mean_us(runner, steps)
    cpu_step = note = None
    if ho is not None:
        lens.copy_(start_lens)
        for m in model:
            m.seq_lens.copy_(lens)
        staged = [ho.stage(host_inputs(m, list(oracle_seqs))) for m in model]
        ho.seconds(staged, append=True)       # first touch, untimed
        cpu_step = ho.seconds(staged, 1, append=True) * B / len(oracle_seqs)
        note = (f"{len(oracle_seqs)} of {B} sequences, all {layers} layers (append + "
                f"attention), one step, scaled x{B / len(oracle_seqs):g}; {ho.describe()}")
    e = entry("decode_loop", f"step ({layers} layers: append + attention each, "
              f"{'one launch' if fused else 'separate append launch'})", us_step,
              total / steps, cpu_step, note, steps=steps, layers=layers,
              loop_ms=round(us_step * steps / 1e3, 3), hip_graph=graph, fused_append=fused)
    del model, outs, ws
    torch.cuda.empty_cache()
    return e


# ---------------------------------------------------------------------------

SWEEP_POINTS = ([(B, 8192) for B in (1, 2, 4, 8, 16, 32, 64, 128, 256)] +
                [(64, L) for L in (512, 1024, 2048, 4096, 16384, 32768)])


def sweep(sa, torch, timer, dev, steps, warmup):
    """The fused step (append inside the attention launch) of a paged full
    layer, 64 query / 8 KV heads, D 64, bs 16, uniform context L (after the
    append), over SWEEP_POINTS.  Inputs that would fit the Infinity Cache
    rotate over enough sets that every call reads HBM."""
    import synth
    for B, L in SWEEP_POINTS:
        mk = lambda i: synth.make_layer(batch=B, q_heads=64, kv_heads=8, head_dim=64,    # noqa: E731
                                        block_size=16, lens=[L] * B, seed=3000 + 101 * i,
                                        device=dev)
        first = mk(0)
        pool = first.k_cache.numel() * 4
        nsets = 1 if pool > 2 * MALL_BYTES else min(64, -(-(3 * MALL_BYTES) // max(pool, 1)))
        sets = [first] + [mk(i) for i in range(1, nsets)]
        outs = [torch.empty_like(x.q) for x in sets]
        ws = sa.new_workspace(first.q, first.k_cache, first.v_cache, first.block_table, 0)

        def call(i):
            x = sets[i % len(sets)]
            sa.decode_attention_append(x.q, x.k_new, x.v_new, x.k_cache, x.v_cache,
                                       x.block_table, x.seq_lens, x.sinks, 0,
                                       out=outs[i % len(sets)], workspace=ws)
        timer.settle(call, warmup)
        us = timer.mean_us(call, steps)
        timing = "eager, back to back"
        if us < 40.0:
            g = torch.cuda.CUDAGraph()
            per_graph = max(len(sets), 32)
            with torch.cuda.graph(g):
                for i in range(per_graph):
                    call(i)
            reps = max(2, steps // 10)
            timer.settle(lambda _: g.replay(), reps)
            us = timer.mean_us(lambda _: g.replay(), reps) / per_graph
            timing = f"HIP graph of {per_graph} launches"
            del g
        nbytes = attn_bytes([L] * B, 0) + append_bytes(B)
        print(json.dumps(dict(batch=B, context=L, us=round(us, 2), bytes=nbytes,
                              gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
                              frac_of_peak=round(nbytes / (us * 1e-6) / PEAK_HBM, 4),
                              splits=sa.num_splits(first.q, first.k_cache, first.v_cache,
                                                   first.block_table, 0),
                              input_sets=len(sets), timing=timing)), flush=True)
        del sets, outs, ws, first
        torch.cuda.empty_cache()


def step_calls(sa, torch, dev, workload, variant, separate_append=False):
    """One step of a workload as its calls in order: (name, algorithmic bytes,
    launcher(i), input sets).  A layer whose pools would stay in the 256 MB
    Infinity Cache from one step to the next (the ring layer) rotates over
    input sets, so that every step reads it from HBM as a model's many layers
    would; call i of a layer uses set i mod (its sets).  Returns the layers,
    the calls and each layer's split count."""
    layers = make_workload(workload, dev)
    rotations = []
    for L in layers:
        pool = L.k_cache.numel() * 4
        n = 1 if pool > 2 * MALL_BYTES else min(64, -(-(3 * MALL_BYTES) // max(pool, 1)))
        rot = [L]
        if n > 1 and workload == "batch64_ragged":
            rot += [ragged_layers(dev, seed_offset=101 * i, windows=(L.window,))[0]
                    for i in range(1, n)]
        rotations.append(rot)
    outs = [torch.empty_like(L.q) for L in layers]
    wss = [sa.new_workspace(L.q, L.k_cache, L.v_cache, L.block_table, L.window,
                            variant=variant) for L in layers]
    splits = [sa.num_splits(L.q, L.k_cache, L.v_cache, L.block_table, L.window,
                            variant=variant) for L in layers]
    with_append = workload in APPEND_WORKLOADS
    fused = with_append and not separate_append
    calls = []
    for L0, rot, o, ws in zip(layers, rotations, outs, wss):
        lens = L0.seq_lens.cpu().tolist()
        nb = attn_bytes(lens, L0.window, L0.q_heads, L0.kv_heads, L0.head_dim)
        if fused:
            # the append inside the attention launch (rewriting the same slot
            # with the same row on every repeat)
            calls.append((f"append+attention(w={L0.window})", nb + append_bytes(L0.batch),
                          lambda i=0, rot=rot, o=o, ws=ws: (lambda L: sa.decode_attention_append(
                              L.q, L.k_new, L.v_new, L.k_cache, L.v_cache, L.block_table,
                              L.seq_lens, L.sinks, L.window, out=o, workspace=ws,
                              variant=variant))(rot[i % len(rot)]), len(rot)))
            continue
        if with_append:
            calls.append((f"append(w={L0.window})", append_bytes(L0.batch),
                          lambda i=0, rot=rot: (lambda L: sa.kv_append(
                              L.k_new, L.v_new, L.k_cache, L.v_cache, L.block_table,
                              L.seq_lens, L.window))(rot[i % len(rot)]), len(rot)))
        calls.append((f"attention(w={L0.window})", nb,
                      lambda i=0, rot=rot, o=o, ws=ws: (lambda L: sa.decode_attention(
                          L.q, L.k_cache, L.v_cache, L.block_table, L.seq_lens, L.sinks,
                          L.window, out=o, workspace=ws, variant=variant))(rot[i % len(rot)]),
                      len(rot)))
    return layers, calls, splits, fused


def time_calls(torch, timer, calls, steps, warmup):
    """Each call alone, K times back to back between two HIP events on its
    stream (calls under 40 us from a HIP graph of 32 launches instead), with
    the spread over further rounds and single-call percentiles."""
    per_call = []
    for nm, b, f, nsets in calls:
        timer.settle(f, warmup)
        us = timer.mean_us(f, steps)
        timing = "eager, back to back"
        if us < 40.0:                        # host-bound from Python: replay a graph
            per_graph = 32
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(per_graph):
                    f(i)
            reps = max(2, steps // 10)
            timer.settle(lambda _: g.replay(), reps)
            us = timer.mean_us(lambda _: g.replay(), reps) / per_graph
            timing = f"HIP graph of {per_graph} launches, replayed {reps} times"
            del g
        e = dict(call=nm, us_mean=round(us, 2), bytes=b, gbps=round(b / (us * 1e-6) / 1e9, 1),
                 frac_of_peak=round(b / (us * 1e-6) / PEAK_HBM, 4), timing=timing,
                 input_sets=nsets)
        if timing.startswith("eager"):
            # spread: the same mean over ROUNDS further rounds of back-to-back calls
            rs = sorted(timer.mean_us(f, steps) for _ in range(ROUNDS))
            e["rounds"] = dict(rounds=ROUNDS, calls_per_round=steps,
                               us_median=round(statistics.median(rs), 2),
                               us_min=round(rs[0], 2), us_max=round(rs[-1], 2))
            e["per_call_events"] = spread(timer.per_call_us(f, steps))
        if nsets > 1:
            e["note"] = (f"{nsets} input sets in rotation (in the step too), so no call finds "
                         "its inputs in the 256 MB Infinity Cache")
        per_call.append(e)
        print(f"# {nm}: {us:.2f} us, {b / (us * 1e-6) / 1e9:.1f} GB/s", flush=True)
    return per_call


KERNEL_NAMES = ("decode_stream_kernel", "combine_stream_kernel", "decode_mfma_kernel",
                "combine_kernel", "kv_append_kernel")


def kernel_times_us(torch, fn, reps):
    """Mean device duration (us) of each of the library's kernels that fn
    launches, over reps back-to-back calls, from the PyTorch profiler's device
    trace (each kernel's own start and end on the GPU); None if the profiler
    gives no device events here."""
    try:
        from torch.profiler import ProfilerActivity, profile
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(reps):
                fn(i)
            torch.cuda.synchronize()
        sums, counts = {}, {}
        for ev in prof.events():
            name = getattr(ev, "name", "") or ""
            k = next((n for n in KERNEL_NAMES if n in name), None)
            dt = getattr(ev, "device_time", None)
            if dt is None:
                dt = getattr(ev, "cuda_time", 0.0)
            if k is None or not dt:
                continue
            sums[k] = sums.get(k, 0.0) + float(dt)
            counts[k] = counts.get(k, 0) + 1
        if not sums:
            return None
        return {k: round(sums[k] / counts[k], 2) for k in sums}
    except Exception as exc:                  # noqa: BLE001 - report, do not fail the bench
        print(f"# kernel timing from the profiler unavailable: {exc!r}", flush=True)
        return None


def roofline_of(call, kernels, traffic, split_kernel):
    """The dominant call's roofline: its algorithmic bytes over its mean
    event-timed duration (the whole call: decode kernel and, when split, the
    merge launch), and over the decode kernel's own mean duration from the
    profiler's device trace."""
    b, us = call["bytes"], call["us_mean"]
    achieved = b / (us * 1e-6) / 1e9
    r = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
             frac=round(achieved * 1e9 / PEAK_HBM, 4), traffic=traffic,
             algorithmic_bytes_per_launch=b, avg_launch_us=us,
             timed="the whole call (every launch it makes), HIP events on its stream")
    if kernels:
        k = kernels.get(split_kernel) or kernels.get("decode_mfma_kernel")
        if k:
            ka = b / (k * 1e-6) / 1e9
            r["kernel"] = dict(name=split_kernel if split_kernel in kernels
                               else "decode_mfma_kernel", us=k, achieved=round(ka, 1),
                               frac=round(ka * 1e9 / PEAK_HBM, 4),
                               timed="mean device duration from the profiler's trace")
        r["kernels_us"] = kernels
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(STEP_WORKLOADS))
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-reps", type=int, default=3)
    ap.add_argument("--configs", choices=("all", "none"), default="all",
                    help="also report every synthetic configuration (default: all)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with its own launch before each attention call instead of "
                         "inside it")
    ap.add_argument("--graph", action="store_true",
                    help="replay the decode loop's step from a HIP graph")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the fused step of a paged full layer over a grid of batch "
                         "sizes and context lengths (one JSON line per point) and exit")
    ap.add_argument("--only", default="", metavar="CONFIG[,CONFIG...]",
                    help="only time these attention configurations (tiny, gptoss_layer_8k, "
                         "long_131k_b1, long_131k_b8, long_131k_b8_tp_share, batch64_8k), one "
                         "JSON line each, and exit (for profiling them)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES, three times, and exit: the "
                         "reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode step is built and measured on a "
              "single MI355X only (no multi-GPU path in this library).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        x = torch.ones(args.copy_calibration // 2, dtype=torch.bfloat16, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(f"# copied {args.copy_calibration} bytes 3 times", flush=True)
        return
    import paged_gqa_decode_step_amd as sa
    sa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    if args.sweep:
        sweep(sa, torch, timer, dev, args.steps, args.warmup)
        return
    if args.only:
        for nm in args.only.split(","):
            e, _ = attention_config(sa, torch, timer, dev, nm, steps=args.steps,
                                    warmup=args.warmup, variant=args.variant, with_oracle=False)
            print(json.dumps(e), flush=True)
        return

    def measure(workload):
        """Step time, per-call times and the dominant call's roofline of one
        workload's step; also its host inputs for the oracle."""
        layers, calls, splits, fused = step_calls(sa, torch, dev, workload, args.variant,
                                                  args.separate_append)

        def step(i=0):
            for _, _, f, _ in calls:
                f(i)
        print(f"# workload {workload}: splits {splits}, warmup {args.warmup}", flush=True)
        timer.settle(step, args.warmup)
        # the timed region: exactly K steps, events at its two ends only
        ms = timer.mean_us(step, args.steps) / 1e3
        nbytes = sum(b for _, b, _, _ in calls)
        per_call = time_calls(torch, timer, calls, args.steps, args.warmup)
        # dominant call: the full-layer attention (the first layer's)
        dom = next(i for i, c in enumerate(calls) if "attention" in c[0])
        kernels = kernel_times_us(torch, calls[dom][2], args.steps)
        split_kernel = ("decode_stream_kernel" if splits[0] > 1 and args.variant in (0, 4, 5)
                        else "decode_mfma_kernel")
        traffic = load_traffic(workload) if args.variant == 0 else None
        roof = roofline_of(per_call[dom], kernels, traffic, split_kernel)
        roof["call"] = calls[dom][0]
        hosts = None if args.no_cpu_baseline else [host_inputs(L) for L in layers]
        info = dict(splits=splits, fused=fused, batch=layers[0].batch,
                    with_append=workload in APPEND_WORKLOADS)
        del calls, layers
        torch.cuda.empty_cache()
        return ms, nbytes, per_call, roof, hosts, info

    ms_per_step, step_bytes, per_call, roofline, main_hosts, info = measure(args.workload)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ceiling = read_ceiling(sa, torch, timer, dev)
    roofline["frac_of_read_ceiling"] = round(roofline["achieved"] / ceiling["gbps"], 4)
    roofline["frac_of_tile_ceiling"] = round(
        roofline["achieved"] / ceiling["scattered_tiles"]["gbps"], 4)
    print(f"# read ceiling: {ceiling['gbps']} GB/s ({ceiling['frac_of_peak']:.1%} of peak); "
          f"scattered tiles {ceiling['scattered_tiles']['gbps']} GB/s", flush=True)

    configs = []
    hosts = []
    ragged = None
    oc = not args.no_cpu_baseline
    if args.configs == "all":
        if args.workload != "batch64_ragged":
            r_ms, r_bytes, r_calls, r_roof, r_hosts, r_info = measure("batch64_ragged")
            ragged = dict(workload="batch64_ragged", call="step: a paged full layer and a "
                          "sliding-window-128 ring layer, append inside each attention launch",
                          ms_per_step=round(r_ms, 4), bytes=r_bytes,
                          value=round(r_bytes / (r_ms * 1e-3) / 1e9, 1), unit="GB/s",
                          frac_of_peak=round(r_bytes / (r_ms * 1e-3) / PEAK_HBM, 4),
                          splits=r_info["splits"], us_per_call=r_calls, roofline=r_roof)
            print(f"# batch64_ragged step: {r_ms * 1e3:.2f} us, {ragged['value']} GB/s",
                  flush=True)
        for nm in ("batch64_8k", "tiny", "gptoss_layer_8k", "long_131k_b1", "long_131k_b8",
                   "long_131k_b8_tp_share"):
            e, h = attention_config(sa, torch, timer, dev, nm, steps=args.steps,
                                    warmup=args.warmup, variant=args.variant, with_oracle=oc,
                                    label="batch64_8k, attention alone" if nm == "batch64_8k"
                                    else None)
            configs.append(e)
            hosts.append(h)
            print(f"# {e['config']}: {e['us']} us, {e['gbps']} GB/s", flush=True)
        rs = rope_step_config(sa, torch, timer, dev, args.steps, args.warmup, args.variant,
                              with_oracle=oc)
        configs.append(rs)
        hosts.append(None)
        print(f"# RoPE step: {rs['us']} us ({rs['us_without_rope']} without), {rs['gbps']} GB/s",
              flush=True)
        ts = tile_step_config(sa, torch, timer, dev, args.steps, args.warmup, args.variant,
                              with_oracle=oc)
        configs.append(ts)
        hosts.append(None)
        print(f"# 2-token tile: {ts['us']} us ({ts['us_one_token']} for one token), "
              f"{ts['gbps']} GB/s", flush=True)

    # each dominant call's read floor: its own tiles read with no arithmetic
    specs = {}

    def add_spec(key, name, layer, splits, kernels):
        lens, w, kvh = layer_lens(name)[layer]
        if splits == 1:
            balanced = False                 # one partition a unit: the static kernel
        elif kernels:
            balanced = "decode_stream_kernel" in kernels
        else:
            return
        n = max(min(L, w) if w > 0 else L for L in lens)
        if balanced and len(lens) * kvh * -(-n // 32) < 8 * BALANCED_WAVES:
            return                           # a narrower balanced launch: not modelled
        specs[key] = (lens, w, kvh, balanced, splits)
    add_spec(args.workload + (" full layer" if args.workload == "batch64_ragged" else ""),
             args.workload, 0, info["splits"][0], roofline.get("kernels_us"))
    if args.workload == "batch64_ragged":
        add_spec("batch64_ragged ring layer", "batch64_ragged", 1, info["splits"][1], None)
    if ragged is not None:
        add_spec("batch64_ragged full layer", "batch64_ragged", 0, ragged["splits"][0],
                 ragged["roofline"].get("kernels_us"))
        add_spec("batch64_ragged ring layer", "batch64_ragged", 1, ragged["splits"][1], None)
    for e in configs:
        if e.get("config") in ("gptoss_layer_8k", "long_131k_b1", "long_131k_b8",
                               "long_131k_b8_tp_share"):
            add_spec(e["config"], e["config"], 0, e["splits"], e.get("kernels_us"))
    floors = read_floors(sa, torch, timer, dev, specs, args.steps, args.warmup)

    def decode_us(kernels):
        k = kernels or {}
        return k.get("decode_stream_kernel") or k.get("decode_mfma_kernel")
    main_key = args.workload + (" full layer" if args.workload == "batch64_ragged" else "")
    if main_key in floors:
        roofline["read_floor"] = floor_fields(floors[main_key], roofline["avg_launch_us"],
                                              decode_us(roofline.get("kernels_us")))
    if ragged is not None:
        if "batch64_ragged full layer" in floors:
            ragged["roofline"]["read_floor"] = floor_fields(
                floors["batch64_ragged full layer"], ragged["roofline"]["avg_launch_us"],
                decode_us(ragged["roofline"].get("kernels_us")))
        ring = next((c for c in ragged["us_per_call"]
                     if "attention" in c["call"] and "(w=0)" not in c["call"]), None)
        if ring is not None and "batch64_ragged ring layer" in floors:
            ring["read_floor"] = floor_fields(floors["batch64_ragged ring layer"],
                                              ring["us_mean"])
    for e in configs:
        if e.get("config") in floors:
            e["read_floor"] = floor_fields(floors[e["config"]], e["us"],
                                           decode_us(e.get("kernels_us")))
        elif e.get("config") == "batch64_8k, attention alone" and "batch64_8k" in floors:
            e["read_floor"] = floor_fields(floors["batch64_8k"], e["us"],
                                           decode_us(e.get("kernels_us")))

    # the oracle on the host's cores, after every GPU timing but the loop's
    ho = HostOracle() if oc else None
    if args.configs == "all":
        loop = decode_loop_config(sa, torch, timer, dev, stream, args.variant, graph=args.graph,
                                  ho=ho, fused=not args.separate_append)
        configs.append(loop)
        print(f"# decode loop: {loop['us']} us per step, {loop['gbps']} GB/s", flush=True)
        if not args.graph:                   # the same loop replayed from a HIP graph per step
            gl = decode_loop_config(sa, torch, timer, dev, stream, args.variant, graph=True,
                                    ho=None, fused=not args.separate_append)
            gl["config"] = "decode_loop (HIP graph)"
            configs.append(gl)
            print(f"# decode loop, HIP graph: {gl['us']} us per step, {gl['gbps']} GB/s",
                  flush=True)
        if oc:
            print("# timing the oracle on the configurations...", flush=True)
            for e, h in zip(configs, hosts):
                if h is not None:
                    add_oracle(e, h, ho)

    cpu = None
    if ho is not None:
        print("# timing the oracle on the step...", flush=True)
        staged = [ho.stage(h) for h in main_hosts]
        ho.seconds(staged, append=info["with_append"])          # first touch, untimed
        sec = ho.seconds(staged, args.oracle_reps, append=info["with_append"])
        cpu = dict(value=round(step_bytes / sec / 1e9, 4), unit="GB/s", cores=ho.workers,
                   kind="oracle", seconds_per_step=round(sec, 3), blas_threads_per_core=1,
                   cores_available=len(os.sched_getaffinity(0)),
                   sample=f"the whole {args.workload} step (every sequence"
                          f"{', append then attention' if info['with_append'] else ''}), "
                          f"median of {args.oracle_reps} runs; {ho.describe()}")
        ho.close()

    wl = STEP_WORKLOADS[args.workload]
    res = dict(metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_per_step, 4), higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload=args.workload, batch=info["batch"], q_heads=64, kv_heads=8,
                           head_dim=64, block_size=16, context=wl, splits=info["splits"],
                           variant=args.variant,
                           step=("append inside attention, one launch per layer (plus the "
                                 "merge launch of a split call)" if info["fused"]
                                 else "append + attention per layer" if info["with_append"]
                                 else "attention")),
               us_per_call=per_call, step_bytes=step_bytes,
               frac_of_peak=round(value * 1e9 / PEAK_HBM, 4),
               roofline=roofline, cpu_baseline=cpu, read_ceiling=ceiling,
               batch64_ragged_step=ragged, configs=configs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
