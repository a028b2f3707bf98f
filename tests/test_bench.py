"""bench.py's byte accounting and its launch contract, on the CPU.

Algorithmic bytes per attention call are 2048 B per attended token per layer
(8 KV heads x 64 dims x 2 B, K and V) plus 16 KiB per sequence (q and out);
the expected values are the per-workload figures stated with the workloads
(the tiny case, the gpt-oss layer, the batch-64 ring layer, 131072-token
contexts and the batch-64 x 8192 headline)."""

import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_bytes_of_the_workloads():
    assert bench.attn_bytes([38], 0, q_heads=4, kv_heads=1) == 10_752
    assert bench.attn_bytes([8192], 0) == 16_793_600
    assert bench.attn_bytes([8192] * 64, 0) == 1_074_790_400
    assert bench.attn_bytes([131072], 0) == 268_451_840
    assert bench.attn_bytes([131072] * 8, 0) == 2_147_614_720
    # one GPU's share under 8-way KV-head parallelism: 1 KV head, 8 query heads
    assert bench.attn_bytes([131072] * 8, 0, q_heads=8, kv_heads=1) == 268_451_840


def test_ring_layer_reads_the_window_only():
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
    assert min(lens) > 128
    assert bench.attn_bytes(lens, 128) == 17_825_792
    # a full layer reads every position
    assert bench.attn_bytes(lens, 0) == int(sum(lens)) * 2048 + 64 * 16384


def test_append_bytes():
    # k_new and v_new read, and the same rows written into the pools
    assert bench.append_bytes(64) == 64 * 8 * 64 * 2 * 2 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one" in (r.stdout + r.stderr).lower()


def test_spread_percentiles():
    s = bench.spread([float(i) for i in range(1, 101)])
    assert s == dict(calls=100, us_median=50.5, us_p10=10.9, us_p90=90.1)


class _Pool:
    """HostOracle.tasks needs only the worker count."""
    def __init__(self, workers):
        self.workers = workers


def test_oracle_tasks_cover_every_sequence_and_head_once():
    for workers, B, Hkv in ((16, 64, 8), (16, 1, 8), (8, 8, 1), (16, 5, 2), (3, 64, 8)):
        c = dict(path="p", B=B, Hkv=Hkv, window=0)
        seen = []
        for path, seqs, g0, g1, append, window in bench.HostOracle.tasks(_Pool(workers), [c],
                                                                           True):
            assert path == "p" and append and window == 0
            seen += [(b, g) for b in seqs for g in range(g0, g1)]
        assert sorted(seen) == [(b, g) for b in range(B) for g in range(Hkv)]


def test_oracle_task_runs_the_oracle_on_its_share(tmp_path):
    """A worker's share gives the oracle's own output for those sequences and
    heads (the task only cuts out data): run in-process here."""
    import numpy as np
    import oracle
    L = synth.make_layer(batch=3, q_heads=8, kv_heads=2, lens=[40, 70, 17], seed=3)
    h = bench.host_inputs(L)
    for n in bench._ARRAYS:
        if h.get(n) is not None:
            np.save(tmp_path / (n + ".npy"), np.ascontiguousarray(h[n]))
    got = bench._oracle_task((str(tmp_path), [0, 2], 1, 2, True, 0))
    k, v = oracle.kv_append(h["k"], h["v"], h["kn"], h["vn"], h["bt"], h["lens"], 0)
    want = oracle.decode_attention(h["q"], k, v, h["bt"], h["lens"], h["sinks"], 0)
    assert np.array_equal(got, want[[0, 2]][:, 4:8])      # KV head 1: query heads 4..7
