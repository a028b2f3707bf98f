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
