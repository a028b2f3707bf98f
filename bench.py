#!/usr/bin/env python3
"""Benchmark of the decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batch64_ragged]

A step is one pass of the whole hot path over one batch: for the default
workload (batch 64, 64 query / 8 KV heads, D 64, block size 16, ragged
context 512..8192 plus one appended token) it is the KV append and decode
attention of a paged full-attention layer, then the KV append and decode
attention of a sliding-window-128 ring layer.  Inputs are seeded synthetic
bf16 N(0,1) values, resident in HBM before timing starts.

Reported (one JSON line): ``value`` is the step's algorithmic bytes divided by
its time (GB/s); the algorithmic bytes of an attention call are 2048 B per
attended token (K and V rows of 8 KV heads x 64 dims x bf16) plus 16 KiB per
sequence (its bf16 query and output rows), and an append moves 4 KiB per
sequence (read and write of K and V rows).  ``roofline`` covers the dominant
kernel (the full-layer attention call), timed with HIP events on the stream
it runs on.  ``cpu_baseline`` is the fp64 oracle timed on this host on the
same workload.  ``headline_uniform_8k`` is the attention call alone at batch
64 x 8192 tokens.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

_ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, _ROOT)

PEAK_HBM = 8.0e12            # MI355X HBM3E, bytes/s
METRIC = "decode-attn µs/call + achieved HBM GB/s (% of peak), batch 64, 8k ctx"
# sources of the dominant call's kernels; the committed counter summary is
# valid only for the exact sources it was taken on
KERNEL_SRCS = [os.path.join(_ROOT, "paged_gqa_decode_step_amd", "csrc", f)
               for f in ("decode_stream.hip", "mfma_attend.h")]
TRAFFIC_FILE = os.path.join(_ROOT, "profiles", "decode_attention_batch64_ragged_traffic.json")


def attn_bytes(lens, window, q_heads=64, kv_heads=8, head_dim=64):
    n = [min(int(L), window) if window > 0 else int(L) for L in lens]
    per_tok = kv_heads * head_dim * 2 * 2
    per_seq = q_heads * head_dim * 2 * 2
    return sum(n) * per_tok + len(lens) * per_seq


def append_bytes(batch, kv_heads=8, head_dim=64):
    return batch * kv_heads * head_dim * 2 * 2 * 2


def source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic():
    """Per-launch HBM bytes of the dominant kernel from the committed counter
    summary, or None if there is none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_digest():
        return None
    return t.get("bytes_per_launch")


def make_workload(name, device):
    import synth
    if name == "batch64_ragged":
        c = synth.CONFIGS[name]
        lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
        common = dict(batch=c["batch"], q_heads=c["q_heads"], kv_heads=c["kv_heads"],
                      head_dim=c["head_dim"], block_size=c["block_size"], lens=lens,
                      device=device)
        return [synth.make_layer(window=0, seed=c["seed"] + 10, **common),
                synth.make_layer(window=128, seed=c["seed"] + 20, **common)]
    if name in ("batch64_8k", "gptoss_layer_8k", "long_131k_b1", "long_131k_b8"):
        c = dict(synth.CONFIGS[name])
        return [synth.make_layer(device=device, **c)]
    raise SystemExit(f"unknown workload {name}")


def time_oracle(layers, reps):
    """Median wall time of the fp64 oracle over the whole step (append and
    attention of every layer), BLAS held to one thread."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits = None
    host = []
    for L in layers:
        host.append(dict(q=synth.to_bits(L.q), k=synth.to_bits(L.k_cache),
                         v=synth.to_bits(L.v_cache), bt=synth.to_bits(L.block_table),
                         lens=synth.to_bits(L.seq_lens), kn=synth.to_bits(L.k_new),
                         vn=synth.to_bits(L.v_new),
                         sinks=None if L.sinks is None else L.sinks.cpu().numpy(),
                         w=L.window))
    import contextlib
    times = []
    limit = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    with limit:
        for _ in range(reps):
            t0 = time.perf_counter()
            for h in host:
                k, v = oracle.kv_append(h["k"], h["v"], h["kn"], h["vn"], h["bt"], h["lens"], h["w"])
                oracle.decode_attention(h["q"], k, v, h["bt"], h["lens"], h["sinks"], h["w"])
            times.append(time.perf_counter() - t0)
    return statistics.median(times), np.__version__


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch64_ragged")
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-reps", type=int, default=3)
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

    layers = make_workload(args.workload, dev)
    outs = [torch.empty_like(L.q) for L in layers]
    wss = [sa.new_workspace(L.q, L.k_cache, L.v_cache, L.block_table, L.window,
                            variant=args.variant) for L in layers]
    splits = [sa.num_splits(L.q, L.k_cache, L.v_cache, L.block_table, L.window,
                            variant=args.variant) for L in layers]
    with_append = args.workload == "batch64_ragged"

    def calls_of_step():
        """The step's calls in order, as (name, bytes, thunk)."""
        out = []
        for L, o, ws in zip(layers, outs, wss):
            lens = L.seq_lens.cpu().tolist()
            if with_append:
                out.append((f"append(w={L.window})", append_bytes(L.batch),
                            lambda L=L: sa.kv_append(L.k_new, L.v_new, L.k_cache, L.v_cache,
                                                     L.block_table, L.seq_lens, L.window,
                                                     stream=stream)))
            out.append((f"attention(w={L.window})",
                        attn_bytes(lens, L.window, L.q_heads, L.kv_heads, L.head_dim),
                        lambda L=L, o=o, ws=ws: sa.decode_attention(
                            L.q, L.k_cache, L.v_cache, L.block_table, L.seq_lens, L.sinks,
                            L.window, out=o, workspace=ws, variant=args.variant,
                            stream=stream)))
        return out

    calls = calls_of_step()

    def step():
        for _, _, f in calls:
            f()

    def timed(fn, reps):
        """Mean microseconds of fn over reps back-to-back runs on the stream,
        bracketed by two HIP events (none in between, so no event gap)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    print(f"# workload {args.workload}: splits {splits}, warmup {args.warmup}", flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: exactly K steps, events at its two ends only
    ms_per_step = timed(step, args.steps) / 1e3
    step_bytes = sum(b for _, b, _ in calls)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # per-call means: each call alone, K times back to back
    per_call = []
    for nm, b, f in calls:
        us = timed(f, args.steps)
        per_call.append(dict(call=nm, us_mean=round(us, 2), bytes=b,
                             gbps=round(b / (us * 1e-6) / 1e9, 1),
                             frac_of_peak=round(b / (us * 1e-6) / PEAK_HBM, 4)))
        print(f"# {nm}: {us:.2f} us, {b / (us * 1e-6) / 1e9:.1f} GB/s", flush=True)

    # dominant kernel: the full-layer attention call
    dom = 1 if with_append else 0
    dom_us = per_call[dom]["us_mean"]
    achieved = calls[dom][1] / (dom_us * 1e-6) / 1e9
    traffic = load_traffic() if args.workload == "batch64_ragged" and args.variant == 0 else None
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                    frac=round(achieved * 1e9 / PEAK_HBM, 4), traffic=traffic,
                    kernel=("decode_stream_kernel + combine_stream_kernel (one attention call)"
                            if splits[0] > 1 and args.variant in (0, 4) else
                            "decode_mfma_kernel (+ combine_kernel when split)"),
                    algorithmic_bytes_per_launch=calls[dom][1], avg_launch_us=round(dom_us, 2))

    # headline: the attention call alone at batch 64 x 8192
    headline = None
    if args.workload == "batch64_ragged":
        H = make_workload("batch64_8k", dev)[0]
        ho = torch.empty_like(H.q)
        hws = sa.new_workspace(H.q, H.k_cache, H.v_cache, H.block_table, 0, variant=args.variant)
        for _ in range(args.warmup):
            sa.decode_attention(H.q, H.k_cache, H.v_cache, H.block_table, H.seq_lens, H.sinks, 0,
                                out=ho, workspace=hws, variant=args.variant, stream=stream)
        hmean = timed(lambda: sa.decode_attention(
            H.q, H.k_cache, H.v_cache, H.block_table, H.seq_lens, H.sinks, 0, out=ho,
            workspace=hws, variant=args.variant, stream=stream), args.steps)
        hb = attn_bytes([8192] * 64, 0)
        headline = dict(workload="batch 64 x 8192 tokens, 64/8 heads, D 64, paged bs 16",
                        us_mean=round(hmean, 2), bytes=hb,
                        gbps=round(hb / (hmean * 1e-6) / 1e9, 1),
                        frac_of_peak=round(hb / (hmean * 1e-6) / PEAK_HBM, 4))
        print(f"# headline batch64x8k: {hmean:.2f} us, {headline['gbps']} GB/s", flush=True)
        del H, ho, hws
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the oracle on the host...", flush=True)
        sec, npver = time_oracle(layers, args.oracle_reps)
        cpu = dict(value=round(step_bytes / sec / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                   seconds_per_step=round(sec, 3),
                   sample=f"the whole {args.workload} step (every sequence, every layer), "
                          f"median of {args.oracle_reps} runs, NumPy {npver} fp64, BLAS 1 thread")

    res = dict(metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_per_step, 4), higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload=args.workload, batch=64, q_heads=64, kv_heads=8, head_dim=64,
                           block_size=16, splits=splits, variant=args.variant,
                           step="append+attention per layer" if with_append else "attention"),
               us_per_call=per_call, step_bytes=step_bytes,
               frac_of_peak=round(value * 1e9 / PEAK_HBM, 4),
               roofline=roofline, cpu_baseline=cpu, headline_uniform_8k=headline)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
