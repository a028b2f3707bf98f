"""bench.py's byte accounting and its launch contract, on the CPU.

Algorithmic bytes per attention call are 2048 B per attended token per layer
(8 KV heads x 64 dims x 2 B, K and V) plus 16 KiB per sequence (q and out);
the expected values are the per-workload figures stated with the workloads
(the tiny case, the gpt-oss layer, the batch-64 ring layer, 131072-token
contexts and the batch-64 x 8192 headline)."""

import os
import subprocess
import sys

import numpy as np

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


def _check_floor_tiles(lens, window, kvh, balanced, splits):
    import numpy as np
    base = 1000
    t, waves, span = bench.floor_tiles(np.random.default_rng(5), lens, window, kvh, balanced,
                                       splits, base=base)
    nb = [-(-(min(L, window) if window > 0 else L) // 16) for L in lens]
    pool = sum(nb) * kvh
    assert span == 2 * pool
    k, v = t[0::2].astype(np.int64) - base, t[1::2].astype(np.int64) - base
    # a block's K tile, then its V tile at the same place in the V pool that
    # follows the K pool
    assert (k >= 0).all() and (k < pool).all() and np.array_equal(v, k + pool)
    # every (block, KV head) tile of the pools exactly once
    assert len(np.unique(k)) == len(k) == pool
    return k, waves


def test_floor_tiles_balanced_follow_the_units_in_order():
    lens = [40, 700, 3001, 16]
    k, waves = _check_floor_tiles(lens, 0, 4, True, 8)
    assert waves == bench.BALANCED_WAVES
    # unit (b, g): its blocks for head g, then the next unit
    nb = [3, 44, 188, 1]
    at = 0
    for b in range(4):
        blocks = None
        for g in range(4):
            seg = k[at:at + nb[b]]
            assert (seg % 4 == g).all()
            if blocks is None:
                blocks = seg // 4
            assert np.array_equal(seg // 4, blocks)      # the same blocks for every head
            at += nb[b]
    assert at == len(k)


def test_floor_tiles_static_one_partition_a_wavefront():
    import numpy as np
    # 2 sequences of 8192, 8 KV heads, 32 partitions: 512 wavefronts of 16 blocks
    k, waves = _check_floor_tiles([8192, 8192], 0, 8, False, 32)
    assert waves == 32 * 2 * 8
    per = len(k) // waves
    assert per == 16
    for w in range(waves):
        seg = k[w * per:(w + 1) * per]
        assert (seg % 8 == w % 8).all()                  # partition-major, head innermost
    # a ring layer: the window's blocks only
    k, waves = _check_floor_tiles([5000, 129], 128, 8, False, 1)
    assert waves == 16 and len(k) == 2 * 8 * 8


def test_balanced_width_matches_the_library():
    import re
    with open(os.path.join(ROOT, "paged_gqa_decode_step_amd", "csrc", "plan.h")) as f:
        m = re.search(r"#define SA_STREAM_WAVES (\d+)", f.read())
    assert int(m.group(1)) == bench.BALANCED_WAVES


def test_layer_lens_match_the_workloads():
    c = synth.CONFIGS["batch64_ragged"]
    lens = synth.ragged_lengths(c["seed"], c["batch"], *c["len_range"]) + 1
    layers = bench.layer_lens("batch64_ragged")
    assert [w for _, w, _ in layers] == [0, 128]
    assert layers[0][0] == lens.tolist()
    assert bench.layer_lens("long_131k_b8_tp_share") == [([131072] * 8, 0, 1)]


def test_floor_tiles_refuse_pools_past_the_buffer():
    import pytest
    with pytest.raises(ValueError):
        bench.floor_tiles(np.random.default_rng(0), [bench.FLOOR_TILES * 16], 0, 1, True, 8)
    t, waves, span = bench.floor_tiles(np.random.default_rng(0), [1024], 0, 8, True, 8,
                                       base=bench.FLOOR_TILES - 1024)
    assert span == 1024 and t.max() < bench.FLOOR_TILES
