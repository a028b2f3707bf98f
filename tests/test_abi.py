"""The C-ABI library on the CPU: it loads, exports what include/sa.h declares,
and rejects bad arguments with its status codes before launching anything.

No call here reaches a kernel launch: every case fails validation first, so
these run without a GPU (the pointers passed are never dereferenced).
"""

import ctypes
import os
import re

import pytest

import paged_gqa_decode_step_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")

SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE = -1, -2, -3
FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sa.load()


def good_dims(**kw):
    d = dict(num_seqs=2, num_q_heads=16, num_kv_heads=2, head_dim=64, block_size=16,
             max_blocks_per_seq=8, num_blocks=32, num_splits=0, variant=0,
             cache_layout=sa.LAYOUT_K2_V8)
    d.update(kw)
    return sa.Dims(**d)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sa.h but not exported"
    assert set(names) == set(sa.EXPORTS)


def test_status_strings(lib):
    assert sa.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert sa.status_string(s) not in ("ok", "unknown status")
    assert sa.status_string(-99) == "unknown status"


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=128), SA_ERR_UNSUPPORTED),
    (dict(num_q_heads=12, num_kv_heads=8), SA_ERR_UNSUPPORTED),   # Hq % Hkv
    (dict(num_q_heads=64, num_kv_heads=2), SA_ERR_UNSUPPORTED),   # G = 32 > 16
    (dict(block_size=12), SA_ERR_UNSUPPORTED),
    (dict(block_size=4), SA_ERR_UNSUPPORTED),
    (dict(block_size=128), SA_ERR_UNSUPPORTED),
    (dict(num_seqs=-1), SA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), SA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=0), SA_ERR_INVALID_ARG),
    (dict(num_blocks=0), SA_ERR_INVALID_ARG),
    (dict(num_splits=-2), SA_ERR_INVALID_ARG),
    (dict(variant=9), SA_ERR_INVALID_ARG),
    (dict(variant=6), SA_ERR_INVALID_ARG),
    (dict(num_query_tokens=-1), SA_ERR_INVALID_ARG),
    (dict(num_query_tokens=3), SA_ERR_UNSUPPORTED),               # 3 tokens x G 8 > 16
    (dict(max_blocks_per_seq=1 << 27), SA_ERR_UNSUPPORTED),       # capacity 2^31 tokens
    (dict(cache_layout=sa.LAYOUT_PLAIN), SA_ERR_UNSUPPORTED),     # [NB][Hkv][bs][D] pools
    (dict(cache_layout=2), SA_ERR_UNSUPPORTED),                   # no such layout
    (dict(cache_layout=-1), SA_ERR_UNSUPPORTED),
])
def test_bad_dims_rejected_everywhere(lib, kw, status):
    d = good_dims(**kw)
    assert lib.sa_decode_num_splits(ctypes.byref(d), 0) == status
    assert lib.sa_decode_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.sa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(d), None) == status
    assert lib.sa_decode_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                                   ctypes.byref(d), FAKE, 1 << 30, None) == status
    assert lib.sa_decode_partials(FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE,
                                  ctypes.byref(d), None) == status
    assert lib.sa_decode_attention_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                          FAKE, ctypes.byref(d), FAKE, 1 << 30, None) == status


def test_fused_append_needs_new_rows_and_an_mfma_variant(lib):
    d = good_dims()
    for i in (1, 2):                      # k_new, v_new
        args = [FAKE] * 8
        args[i] = None
        assert lib.sa_decode_attention_append(*args, 0, FAKE, ctypes.byref(d), FAKE, 1 << 30,
                                              None) == SA_ERR_INVALID_ARG
    d = good_dims(variant=3)
    assert lib.sa_decode_attention_append(*([FAKE] * 8), 0, FAKE, ctypes.byref(d), FAKE,
                                          1 << 30, None) == SA_ERR_UNSUPPORTED


def test_window_needs_room_in_the_table(lib):
    d = good_dims(max_blocks_per_seq=4)
    assert lib.sa_decode_num_splits(ctypes.byref(d), 64) >= 1
    assert lib.sa_decode_num_splits(ctypes.byref(d), 65) == SA_ERR_INVALID_ARG


def test_null_dims_and_pointers(lib):
    assert lib.sa_decode_num_splits(None, 0) == SA_ERR_INVALID_ARG
    d = good_dims()
    assert lib.sa_kv_append(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(d), None) \
        == SA_ERR_INVALID_ARG
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert lib.sa_kv_append(*args, 0, ctypes.byref(d), None) == SA_ERR_INVALID_ARG
    # sinks (index 5) may be NULL; every other pointer may not
    for i in (0, 1, 2, 3, 4):
        args = [FAKE] * 6
        args[i] = None
        assert lib.sa_decode_attention(*args, 0, FAKE, ctypes.byref(d), FAKE, 1 << 30,
                                       None) == SA_ERR_INVALID_ARG
    assert lib.sa_decode_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None,
                                   ctypes.byref(d), FAKE, 1 << 30, None) == SA_ERR_INVALID_ARG
    assert lib.sa_combine(None, FAKE, FAKE, 4, FAKE, ctypes.byref(d), None) == SA_ERR_INVALID_ARG
    assert lib.sa_combine(FAKE, FAKE, FAKE, 0, FAKE, ctypes.byref(d), None) == SA_ERR_INVALID_ARG
    assert lib.sa_combine(FAKE, FAKE, FAKE, 4, FAKE, None, None) == SA_ERR_INVALID_ARG


def test_workspace_too_small(lib):
    d = good_dims(max_blocks_per_seq=512, num_splits=4)
    need = lib.sa_decode_workspace_bytes(ctypes.byref(d), 0)
    assert need > 0
    assert lib.sa_decode_attention(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE,
                                   ctypes.byref(d), FAKE, need - 1, None) == SA_ERR_WORKSPACE
    assert lib.sa_decode_attention(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE,
                                   ctypes.byref(d), None, need, None) == SA_ERR_WORKSPACE


def test_empty_batch_is_a_noop(lib):
    d = good_dims(num_seqs=0)
    assert lib.sa_kv_append(None, None, None, None, None, None, 0, ctypes.byref(d), None) == 0
    assert lib.sa_decode_attention(None, None, None, None, None, None, 0, None,
                                   ctypes.byref(d), None, 0, None) == 0


def test_split_table_is_fixed_and_bounded(lib):
    # the headline shape: batch 64, 64/8 heads, 8192-slot capacity
    d = good_dims(num_seqs=64, num_q_heads=64, num_kv_heads=8, max_blocks_per_seq=512,
                  num_blocks=64 * 512 + 1)
    s = lib.sa_decode_num_splits(ctypes.byref(d), 0)
    assert s == lib.sa_decode_num_splits(ctypes.byref(d), 0)
    assert 1 <= s <= 8192 // 32
    # a ring of 128 slots never needs more than 4 partitions of 32
    assert 1 <= lib.sa_decode_num_splits(ctypes.byref(d), 128) <= 4
    # forced split counts: never more partitions than asked, never < 32 slots each
    for want in (1, 2, 7, 32, 256, 1000):
        d.num_splits = want
        s = lib.sa_decode_num_splits(ctypes.byref(d), 0)
        assert 1 <= s <= max(want, 8192 // 1024) and s <= 8192 // 32
    d.num_splits = 1
    assert lib.sa_decode_num_splits(ctypes.byref(d), 0) == 8   # partitions are at most 1024 slots


def test_read_probe_validates(lib):
    sink = ctypes.c_void_p(0x20000)
    assert lib.sa_read_bandwidth_probe(FAKE, 16, None, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_bandwidth_probe(None, 16, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_bandwidth_probe(FAKE, 20, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_bandwidth_probe(ctypes.c_void_p(0x10008), 16, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_bandwidth_probe(FAKE, 0, sink, None) == 0     # nothing launched


def test_rope_entry_validates(lib):
    d = good_dims()
    good = sa.Rope(0x30000, 0x40000, 16, 0)
    bad = [sa.Rope(None, 0x40000, 16, 0), sa.Rope(0x30000, None, 16, 0), sa.Rope(0x30000, 0x40000, 0, 0),
           sa.Rope(0x30000, 0x40000, 16, 2)]
    for r in bad:
        assert lib.sa_decode_attention_append_rope(*([FAKE] * 8), 0, ctypes.byref(r), FAKE,
                                                   ctypes.byref(d), FAKE, 1 << 30,
                                                   None) == SA_ERR_INVALID_ARG
    assert lib.sa_decode_attention_append_rope(*([FAKE] * 8), 0, None, FAKE, ctypes.byref(d),
                                               FAKE, 1 << 30, None) == SA_ERR_INVALID_ARG
    args = [FAKE] * 8
    args[1] = None                                    # no k_new
    assert lib.sa_decode_attention_append_rope(*args, 0, ctypes.byref(good), FAKE,
                                               ctypes.byref(d), FAKE, 1 << 30,
                                               None) == SA_ERR_INVALID_ARG
    dv = good_dims(variant=3)
    assert lib.sa_decode_attention_append_rope(*([FAKE] * 8), 0, ctypes.byref(good), FAKE,
                                               ctypes.byref(dv), FAKE, 1 << 30,
                                               None) == SA_ERR_UNSUPPORTED


def test_query_tiles_need_a_full_layer_and_mfma(lib):
    """Several query tokens: no ring window, no vector-ALU variant, no RoPE."""
    d = good_dims(num_query_tokens=2)
    assert lib.sa_decode_num_splits(ctypes.byref(d), 0) >= 1
    assert lib.sa_decode_num_splits(ctypes.byref(d), 16) == SA_ERR_UNSUPPORTED
    assert lib.sa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, ctypes.byref(d),
                            None) == SA_ERR_UNSUPPORTED
    dv = good_dims(num_query_tokens=2, variant=3)
    assert lib.sa_decode_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ctypes.byref(dv),
                                   FAKE, 1 << 30, None) == SA_ERR_UNSUPPORTED
    r = sa.Rope(0x30000, 0x40000, 16, 0)
    assert lib.sa_decode_attention_append_rope(*([FAKE] * 8), 0, ctypes.byref(r), FAKE,
                                               ctypes.byref(d), FAKE, 1 << 30,
                                               None) == SA_ERR_UNSUPPORTED
    # the workspace grows with the tile (more partial rows)
    d1, d2 = good_dims(num_splits=4), good_dims(num_splits=4, num_query_tokens=2)
    assert lib.sa_decode_workspace_bytes(ctypes.byref(d2), 0) > \
        lib.sa_decode_workspace_bytes(ctypes.byref(d1), 0)


def test_balanced_kernel_only_below_2_31_steps(lib):
    """The balanced kernel walks its steps in 32-bit arithmetic: when the
    table's capacity could give more than 2^31 - 1 steps the call takes the
    static split, whose workspace holds every partition's partials (here far
    larger than the balanced kernel's few MB)."""
    small = good_dims(num_seqs=2048, num_q_heads=64, num_kv_heads=8, max_blocks_per_seq=1 << 16)
    big = good_dims(num_seqs=2048, num_q_heads=64, num_kv_heads=8, max_blocks_per_seq=1 << 19)
    assert lib.sa_decode_workspace_bytes(ctypes.byref(small), 0) < (64 << 20)
    assert lib.sa_decode_workspace_bytes(ctypes.byref(big), 0) > (1 << 36)


def test_misaligned_pointers_rejected(lib):
    """Pointers read or written 16 bytes at a time must be 16-byte aligned;
    a misaligned one is refused before anything is launched."""
    d = ctypes.byref(good_dims())
    odd = ctypes.c_void_p(0x10008)
    ok = FAKE
    assert lib.sa_kv_append(odd, ok, ok, ok, ok, ok, 0, d, None) == SA_ERR_INVALID_ARG
    assert lib.sa_kv_append(ok, ok, ok, odd, ok, ok, 0, d, None) == SA_ERR_INVALID_ARG
    for i in (0, 1, 2, 7):            # q, k_cache, v_cache, out
        args = [ok, ok, ok, ok, ok, ok, 0, ok, d, ok, 1 << 30, None]
        args[i] = odd
        assert lib.sa_decode_attention(*args) == SA_ERR_INVALID_ARG, i
    assert lib.sa_decode_attention(ok, ok, ok, ok, ok, ok, 0, ok, d, odd, 1 << 30,
                                   None) == SA_ERR_INVALID_ARG        # workspace
    for i in (1, 2):                  # k_new, v_new
        args = [ok, ok, ok, ok, ok, ok, ok, ok, 0, ok, d, ok, 1 << 30, None]
        args[i] = odd
        assert lib.sa_decode_attention_append(*args) == SA_ERR_INVALID_ARG, i
    assert lib.sa_decode_partials(ok, ok, ok, ok, ok, 0, odd, ok, d, None) == SA_ERR_INVALID_ARG


def test_binding_checks_the_pool_layouts():
    """The binding refuses a K pool of plain rows ([NB][Hkv][bs][D]) before any
    call: the documented layout is [NB][Hkv][2][bs][D/2].  (On host tensors the
    shape test comes before the device test; a pool of the right shape on the
    host is refused for its device.)"""
    import pytest
    import torch
    bt = torch.zeros(1, 1, dtype=torch.int32)
    v = torch.zeros(3, 2, 2, 64, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_cache must have 5 dims"):
        sa._cache_dims(torch.zeros(3, 2, 16, 64, dtype=torch.bfloat16), v, bt, 1, 0, 0)
    with pytest.raises(ValueError, match="k_cache must be on a GPU device"):
        sa._cache_dims(torch.zeros(3, 2, 2, 16, 32, dtype=torch.bfloat16), v, bt, 1, 0, 0)


def test_small_grids_of_few_partitions_take_the_static_split(lib):
    """A static grid of burst partitions (4 or 8 steps) that fits one
    wavefront per SIMD, or of 512 to 1024 partitions, runs the static split
    (its workspace holds S partials for every output row); any other grid,
    the balanced kernel (two partial slots per wavefront of 1024).  Burst
    partitions are of 4 steps when that grid fits too, a row keeps at most 64
    partials, and a row passes 8 partials only where the 8-step grid holds
    fewer than 512 wavefronts."""
    counters = (1 << 18) * 4

    def ws(B, mbs, S, variant=0):
        d = good_dims(num_seqs=B, num_q_heads=64, num_kv_heads=8, max_blocks_per_seq=mbs,
                      variant=variant)
        assert lib.sa_decode_num_splits(ctypes.byref(d), 0) == S
        return lib.sa_decode_workspace_bytes(ctypes.byref(d), 0)

    def a256(x):                                         # regions start 256-byte aligned
        return (x + 255) & ~255

    def static(B, S):
        rows = B * 64 * S                                # B x Hq x S
        return counters + a256(rows * 64 * 4) + a256(rows * 4) + a256(B * 8 * 2 * 4)

    def balanced(B):
        rows = 1024 * 2 * 8                              # wavefronts x 2 slots x G
        return counters + a256(rows * 64 * 4) + a256(rows * 4) + a256(B * 8 * 2 * 4)

    def balanced_last_merges(B):
        return counters + 1024 * 2 * 17 * 64 * 4        # wavefronts x 2 segment slots
    assert ws(64, 128, 2) == static(64, 2)               # 1024 partitions
    assert ws(8, 512, 8) == static(8, 8)                 # 512

    assert ws(1, 512, 64) == static(1, 64)               # 512 of 4 steps: batch 1 x 8192
    assert ws(1, 8192, 64) == static(1, 64)              # 512 of 2048 slots: batch 1 x 131072
    assert ws(1, 8192, 128, variant=3) == static(1, 128)  # the vector-ALU engine: 1024 slots
    assert ws(1, 4096, 64) == static(1, 64)              # 1 x 65536: 64 partials, 1024 slots
    assert ws(128, 128, 2) == balanced(128)              # 2048
    assert ws(1, 128, 16) == static(1, 16)               # 128 of 4 steps (8-step grid: 64)
    assert ws(2, 512, 64) == static(2, 64)               # 1024 of 4 steps
    assert ws(4, 512, 32) == static(4, 32)               # 1024 of 8 steps (4 steps: 2048)
    assert ws(1, 1024, 64) == static(1, 64)              # 512 of 8 steps (4 steps: 128 a row)
    assert ws(8, 128, 8) == static(8, 8)                 # 512 of 8 steps: one-wavefront merge kept
    assert ws(2, 128, 16) == static(2, 16)               # 256 of 4 steps (8-step grid: 128)
    assert ws(3, 1024, 16) == balanced(3)                # 384 partitions of 32 steps
    assert ws(128, 128, 2, variant=5) == balanced_last_merges(128)
    assert ws(4, 512, 32, variant=4) == balanced(4)


def test_plain_row_pools_are_refused_not_misread(lib):
    """A caller describing pools of plain rows ([NB][Hkv][bs][D] for K and V),
    or one that left sa_dims zero-filled past the shapes, gets
    SA_ERR_UNSUPPORTED from every call that takes the pools, before any
    launch; sa_combine, which takes no pool, does not look at the field."""
    for layout in (sa.LAYOUT_PLAIN, 0):
        d = good_dims(cache_layout=layout)
        assert lib.sa_decode_num_splits(ctypes.byref(d), 0) == SA_ERR_UNSUPPORTED
        assert lib.sa_decode_workspace_bytes(ctypes.byref(d), 0) == 0
        assert lib.sa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(d),
                                None) == SA_ERR_UNSUPPORTED
        for W in (0, 64):
            assert lib.sa_decode_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W, FAKE,
                                           ctypes.byref(d), FAKE, 1 << 30, None) \
                == SA_ERR_UNSUPPORTED
            assert lib.sa_decode_attention_append(*([FAKE] * 8), W, FAKE, ctypes.byref(d),
                                                  FAKE, 1 << 30, None) == SA_ERR_UNSUPPORTED
        assert lib.sa_decode_partials(FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE,
                                      ctypes.byref(d), None) == SA_ERR_UNSUPPORTED
        r = sa.Rope(0x10000, 0x10000, 16, sa.ROPE_HALF)
        assert lib.sa_decode_attention_append_rope(*([FAKE] * 8), 0, ctypes.byref(r), FAKE,
                                                   ctypes.byref(d), FAKE, 1 << 30, None) \
            == SA_ERR_UNSUPPORTED
    assert sa.Dims().cache_layout == sa.LAYOUT_PLAIN     # what a zero-filled struct says
    # the combine's own checks still run first (here: no splits)
    d = good_dims(cache_layout=sa.LAYOUT_PLAIN)
    assert lib.sa_combine(FAKE, FAKE, None, 0, FAKE, ctypes.byref(d), None) == SA_ERR_INVALID_ARG



def test_noalloc_call_validates_before_touching_the_device(lib):
    """The no-allocation step checks its arguments, and that the call fits the
    library's scratch, before any HIP call (so these run without a GPU)."""
    d = good_dims()
    for i in range(8):                    # q, k_new, v_new, pools, table, lengths, (sinks)
        if i == 7:
            continue                      # sinks may be NULL
        args = [FAKE] * 8
        args[i] = None
        assert lib.sa_decode_attention_append_noalloc(*args, 0, FAKE, ctypes.byref(d),
                                                      None) == SA_ERR_INVALID_ARG
    assert lib.sa_decode_attention_append_noalloc(*([FAKE] * 8), 0, None, ctypes.byref(d),
                                                  None) == SA_ERR_INVALID_ARG
    d = good_dims(cache_layout=sa.LAYOUT_PLAIN)
    assert lib.sa_decode_attention_append_noalloc(*([FAKE] * 8), 0, FAKE, ctypes.byref(d),
                                                  None) == SA_ERR_UNSUPPORTED
    # a static split of 4096 x 64 heads x 8 partitions needs 512 MiB of partials
    big = good_dims(num_seqs=4096, num_q_heads=64, num_kv_heads=8, max_blocks_per_seq=512,
                    num_blocks=1 << 20, variant=1)
    need = lib.sa_decode_workspace_bytes(ctypes.byref(big), 0)
    assert need > sa.SCRATCH_BYTES
    assert lib.sa_decode_attention_append_noalloc(*([FAKE] * 8), 0, FAKE, ctypes.byref(big),
                                                  None) == sa.SA_ERR_SCRATCH
    assert "scratch" in sa.status_string(sa.SA_ERR_SCRATCH)


def test_tile_probe_validates(lib):
    sink = FAKE
    assert lib.sa_read_tiles_probe(FAKE, 1 << 20, FAKE, 10, 0, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(FAKE, 1 << 20, FAKE, 10, 65536, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(FAKE, 1 << 20, FAKE, -1, 4, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(FAKE, 1 << 20, None, 10, 4, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(FAKE, 1024, FAKE, 10, 4, sink, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(ctypes.c_void_p(0x10008), 1 << 20, FAKE, 10, 4, sink,
                                   None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(FAKE, 1 << 20, FAKE, 10, 4, None, None) == SA_ERR_INVALID_ARG
    assert lib.sa_read_tiles_probe(FAKE, 1 << 20, FAKE, 0, 4, sink, None) == 0
