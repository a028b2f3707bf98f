"""Python binding of libsa: paged GQA decode attention for MI355X (gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libsa.so`` behind the C ABI declared in ``include/sa.h``.  PyTorch
supplies device memory and streams; this module checks that tensors have the
documented dtypes, shapes and layouts, derives ``sa_dims`` from them, passes
raw device pointers and the current HIP stream, and turns a negative status
into an exception.  There is no fallback: without the built library every
call raises.

Layouts (see include/sa.h): q/out ``[B][Hq][D]`` bf16; k_new/v_new
``[B][Hkv][D]`` bf16; k_cache ``[NB][Hkv][2][bs][D/2]`` bf16 (each K row
in two halves, each half slot-major); v_cache ``[NB][Hkv][bs/8][D][8]`` bf16
(V transposed in chunks of 8 slots);
block_table ``[B][MBS]`` int32; seq_lens ``[B]`` int32 (length after the
append); sinks ``[Hq]`` fp32 or None.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsa.so")

SA_OK = 0
SA_ERR_SCRATCH = -5
SCRATCH_BYTES = 32 << 20      # the library's per-GPU scratch (SA_SCRATCH_BYTES)
LAYOUT_PLAIN = 0        # K and V [NB][Hkv][bs][D]: refused by the library
LAYOUT_K2_V8 = 1        # the pools this binding describes (see the module docstring)
VARIANT_DEFAULT = 0
VARIANT_MFMA_TWO_PASS = 1
VARIANT_MFMA_FUSED = 2
VARIANT_VALU = 3
VARIANT_MFMA_BALANCED = 4
VARIANT_MFMA_BALANCED_LAST_MERGES = 5


class Dims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("num_query_tokens", ctypes.c_int32),
        ("cache_layout", ctypes.c_int32),
    ]


ROPE_HALF = 0
ROPE_INTERLEAVED = 1


class Rope(ctypes.Structure):
    _fields_ = [
        ("cos_table", ctypes.c_void_p),
        ("sin_table", ctypes.c_void_p),
        ("max_positions", ctypes.c_int32),
        ("style", ctypes.c_int32),
    ]


class SAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None
EXPORTS = ("sa_kv_append", "sa_decode_num_splits", "sa_decode_workspace_bytes",
           "sa_decode_attention", "sa_decode_attention_append",
           "sa_decode_attention_append_noalloc", "sa_decode_attention_append_rope",
           "sa_decode_partials",
           "sa_combine", "sa_read_bandwidth_probe", "sa_read_tiles_probe", "sa_status_string")


def load(path: Optional[str] = None):
    """Load libsa.so (built by ``python -m paged_gqa_decode_step_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with "
                          "`python -m paged_gqa_decode_step_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(Dims)
    lib.sa_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, dp, vp]
    lib.sa_kv_append.restype = ctypes.c_int
    lib.sa_decode_num_splits.argtypes = [dp, i32]
    lib.sa_decode_num_splits.restype = i32
    lib.sa_decode_workspace_bytes.argtypes = [dp, i32]
    lib.sa_decode_workspace_bytes.restype = sz
    lib.sa_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, dp, vp, sz, vp]
    lib.sa_decode_attention.restype = ctypes.c_int
    lib.sa_decode_attention_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, dp, vp,
                                               sz, vp]
    lib.sa_decode_attention_append.restype = ctypes.c_int
    lib.sa_decode_attention_append_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                       vp, dp, vp]
    lib.sa_decode_attention_append_noalloc.restype = ctypes.c_int
    lib.sa_decode_attention_append_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                    ctypes.POINTER(Rope), vp, dp, vp, sz, vp]
    lib.sa_decode_attention_append_rope.restype = ctypes.c_int
    lib.sa_decode_partials.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, dp, vp]
    lib.sa_decode_partials.restype = ctypes.c_int
    lib.sa_combine.argtypes = [vp, vp, vp, i32, vp, dp, vp]
    lib.sa_combine.restype = ctypes.c_int
    lib.sa_read_bandwidth_probe.argtypes = [vp, sz, vp, vp]
    lib.sa_read_bandwidth_probe.restype = ctypes.c_int
    lib.sa_read_tiles_probe.argtypes = [vp, sz, vp, ctypes.c_int64, i32, vp, vp]
    lib.sa_read_tiles_probe.restype = ctypes.c_int
    lib.sa_status_string.argtypes = [ctypes.c_int]
    lib.sa_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sa_status_string(status).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    """The stream to launch on: the given one, else torch's current stream of
    the tensors' device."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on(device):
    """The tensors' device made current around a call: the library launches on
    the calling thread's current HIP device (torch's default stream is that
    device's null stream)."""
    return torch.cuda.device(device)


def _check(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _cache_dims(k_cache, v_cache, block_table, B, num_splits, variant):
    _check(k_cache, "k_cache", torch.bfloat16, 5)
    _check(v_cache, "v_cache", torch.bfloat16, 5, k_cache.device)
    _check(block_table, "block_table", torch.int32, 2, k_cache.device)
    NB, Hkv, halves, bs, half = k_cache.shape
    D = halves * half
    if halves != 2:
        raise ValueError(f"k_cache must be [NB][Hkv][2][bs][D/2], got {tuple(k_cache.shape)}")
    if bs % 8:
        raise ValueError(f"block_size must be a multiple of 8, got {bs}")
    if tuple(v_cache.shape) != (NB, Hkv, bs // 8, D, 8):
        raise ValueError(f"v_cache must be [NB][Hkv][bs/8][D][8] = {(NB, Hkv, bs // 8, D, 8)}, "
                         f"got {tuple(v_cache.shape)}")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    return Dims(B, 0, Hkv, D, bs, block_table.shape[1], NB, int(num_splits), int(variant), 0,
                LAYOUT_K2_V8)


def dims_for(q, k_cache, v_cache, block_table, num_splits=0, variant=VARIANT_DEFAULT) -> Dims:
    """sa_dims for q ``[B][Hq][D]`` (one token per sequence) or ``[B][T][Hq][D]``
    (T query tokens per sequence)."""
    _check(q, "q", torch.bfloat16, 4 if isinstance(q, torch.Tensor) and q.dim() == 4 else 3)
    d = _cache_dims(k_cache, v_cache, block_table, q.shape[0], num_splits, variant)
    if q.dim() == 4:
        d.num_query_tokens = q.shape[1]
    d.num_q_heads = q.shape[-2]
    if q.shape[-1] != d.head_dim:
        raise ValueError("q and the caches disagree on head_dim")
    return d


def _check_new_rows(k_new, v_new, d, dev):
    """k_new / v_new: ``[B][Hkv][D]``, or ``[B][T][Hkv][D]`` with T query tokens."""
    T = max(1, d.num_query_tokens)
    nd = 4 if T > 1 or (isinstance(k_new, torch.Tensor) and k_new.dim() == 4) else 3
    _check(k_new, "k_new", torch.bfloat16, nd, dev)
    _check(v_new, "v_new", torch.bfloat16, nd, dev)
    want = (d.num_seqs, d.num_kv_heads, d.head_dim) if nd == 3 else \
        (d.num_seqs, T, d.num_kv_heads, d.head_dim)
    if tuple(k_new.shape) != want or k_new.shape != v_new.shape:
        raise ValueError(f"k_new / v_new must be {list(want)}")


def _raise(st: int, what: str):
    if st != SA_OK:
        raise SAError(st, what)


# ---------------------------------------------------------------------------
# the C-ABI calls
# ---------------------------------------------------------------------------

def kv_append(k_new, v_new, k_cache, v_cache, block_table, seq_lens, window=0, stream=None):
    """Write each sequence's new K/V rows into their paged blocks or ring slots:
    ``[B][Hkv][D]`` (one token, position L-1) or ``[B][T][Hkv][D]`` (token t at
    position L-T+t)."""
    _check(seq_lens, "seq_lens", torch.int32, 1, k_cache.device)
    if not isinstance(k_new, torch.Tensor):
        raise TypeError("k_new must be a torch.Tensor")
    B = k_new.shape[0]
    d = _cache_dims(k_cache, v_cache, block_table, B, 0, 0)
    if k_new.dim() == 4:
        d.num_query_tokens = k_new.shape[1]
    _check_new_rows(k_new, v_new, d, k_cache.device)
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens must have one entry per sequence")
    d.num_q_heads = d.num_kv_heads
    with _on(k_cache.device):
        st = load().sa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_table), _ptr(seq_lens), int(window),
                                 ctypes.byref(d), _stream(stream, k_cache.device))
    _raise(st, "sa_kv_append")


def num_splits(q, k_cache, v_cache, block_table, window=0, num_splits=0,
               variant=VARIANT_DEFAULT) -> int:
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, variant)
    s = load().sa_decode_num_splits(ctypes.byref(d), int(window))
    _raise(min(s, 0), "sa_decode_num_splits")
    return int(s)


def workspace_bytes(q, k_cache, v_cache, block_table, window=0, num_splits=0,
                    variant=VARIANT_DEFAULT) -> int:
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, variant)
    return int(load().sa_decode_workspace_bytes(ctypes.byref(d), int(window)))


def new_workspace(q, k_cache, v_cache, block_table, window=0, num_splits=0,
                  variant=VARIANT_DEFAULT) -> Optional[torch.Tensor]:
    """A zero-filled device workspace of the size the call needs (None if 0)."""
    n = workspace_bytes(q, k_cache, v_cache, block_table, window, num_splits, variant)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def decode_attention(q, k_cache, v_cache, block_table, seq_lens, sinks=None, window=0,
                     out=None, workspace=None, num_splits=0, variant=VARIANT_DEFAULT,
                     stream=None):
    """Decode attention over the paged cache (window <= 0) or ring (window > 0).

    Returns ``out`` (bf16 ``[B][Hq][D]``).  ``workspace`` must be a zeroed
    uint8 device tensor of at least ``workspace_bytes(...)`` bytes when that
    is non-zero; one is allocated if none is given.
    """
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, variant)
    dev = q.device
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, 1, dev)
        if sinks.shape[0] != d.num_q_heads:
            raise ValueError("sinks must have one entry per query head")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, q.dim(), dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if workspace is None:
        workspace = new_workspace(q, k_cache, v_cache, block_table, window, num_splits, variant)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with _on(dev):
        st = load().sa_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                        _ptr(seq_lens), _ptr(sinks), int(window), _ptr(out),
                                        ctypes.byref(d), _ptr(workspace), ws_bytes,
                                        _stream(stream, dev))
    _raise(st, "sa_decode_attention")
    return out


def decode_attention_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                            sinks=None, window=0, out=None, workspace=None, num_splits=0,
                            variant=VARIANT_DEFAULT, stream=None):
    """The fused decode step: the KV append of k_new / v_new and the attention
    over the updated cache, in one launch.  Returns ``out``."""
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, variant)
    dev = q.device
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check_new_rows(k_new, v_new, d, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, 1, dev)
        if sinks.shape[0] != d.num_q_heads:
            raise ValueError("sinks must have one entry per query head")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, q.dim(), dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if workspace is None:
        workspace = new_workspace(q, k_cache, v_cache, block_table, window, num_splits, variant)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with _on(dev):
        st = load().sa_decode_attention_append(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(sinks), int(window), _ptr(out), ctypes.byref(d), _ptr(workspace),
            ws_bytes, _stream(stream, dev))
    _raise(st, "sa_decode_attention_append")
    return out


def decode_attention_append_noalloc(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                    out, sinks=None, window=0, num_splits=0,
                                    variant=VARIANT_DEFAULT, stream=None):
    """The fused decode step without a workspace: its partials live in the
    library's own per-GPU scratch array, so neither the library nor this
    binding allocates (``out`` is required).  Calls that may overlap on one
    GPU race on that array.  Returns ``out``."""
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, variant)
    dev = q.device
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check_new_rows(k_new, v_new, d, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, 1, dev)
        if sinks.shape[0] != d.num_q_heads:
            raise ValueError("sinks must have one entry per query head")
    _check(out, "out", torch.bfloat16, q.dim(), dev)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    with _on(dev):
        st = load().sa_decode_attention_append_noalloc(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(sinks), int(window), _ptr(out), ctypes.byref(d),
            _stream(stream, dev))
    _raise(st, "sa_decode_attention_append_noalloc")
    return out


def decode_attention_append_rope(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                 cos_table, sin_table, style=ROPE_HALF, sinks=None, window=0,
                                 out=None, workspace=None, num_splits=0, variant=VARIANT_DEFAULT,
                                 stream=None):
    """The fused decode step with the rotary embedding of q and k_new at each
    sequence's position L-1 (tables fp32 [positions][D/2]).  Returns ``out``."""
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, variant)
    dev = q.device
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check_new_rows(k_new, v_new, d, dev)
    for t, nm in ((cos_table, "cos_table"), (sin_table, "sin_table")):
        _check(t, nm, torch.float32, 2, dev)
        if t.shape[1] != d.head_dim // 2:
            raise ValueError(f"{nm} must be [positions][head_dim/2]")
    if cos_table.shape != sin_table.shape:
        raise ValueError("cos_table and sin_table must have the same shape")
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, 1, dev)
        if sinks.shape[0] != d.num_q_heads:
            raise ValueError("sinks must have one entry per query head")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, q.dim(), dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if workspace is None:
        workspace = new_workspace(q, k_cache, v_cache, block_table, window, num_splits, variant)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    r = Rope(cos_table.data_ptr(), sin_table.data_ptr(), cos_table.shape[0], int(style))
    with _on(dev):
        st = load().sa_decode_attention_append_rope(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(sinks), int(window), ctypes.byref(r), _ptr(out), ctypes.byref(d),
            _ptr(workspace), ws_bytes, _stream(stream, dev))
    _raise(st, "sa_decode_attention_append_rope")
    return out


def decode_partials(q, k_cache, v_cache, block_table, seq_lens, window=0, num_splits=0,
                    part_o=None, part_lse=None, stream=None):
    """Split-K partials ``(part_o [B][Hq][S][D], part_lse [B][Hq][S])`` without sink
    (with q ``[B][T][Hq][D]``: ``[B][T][Hq][S][D]`` and ``[B][T][Hq][S]``)."""
    d = dims_for(q, k_cache, v_cache, block_table, num_splits, VARIANT_DEFAULT)
    dev = q.device
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    S = load().sa_decode_num_splits(ctypes.byref(d), int(window))
    _raise(min(S, 0), "sa_decode_num_splits")
    lead, D = tuple(q.shape[:-1]), q.shape[-1]
    if part_o is None:
        part_o = torch.empty(lead + (S, D), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty(lead + (S,), dtype=torch.float32, device=dev)
    _check(part_o, "part_o", torch.float32, len(lead) + 2, dev)
    _check(part_lse, "part_lse", torch.float32, len(lead) + 1, dev)
    if tuple(part_o.shape) != lead + (S, D) or tuple(part_lse.shape) != lead + (S,):
        raise ValueError(f"partials must be {list(lead)}+[{S}][D] and {list(lead)}+[{S}]")
    with _on(dev):
        st = load().sa_decode_partials(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(seq_lens), int(window), _ptr(part_o), _ptr(part_lse),
                                       ctypes.byref(d), _stream(stream, dev))
    _raise(st, "sa_decode_partials")
    return part_o, part_lse


def combine(part_o, part_lse, sinks=None, out=None, stream=None):
    """Log-sum-exp combine of ``[B][Hq][S][D]`` (or ``[B][T][Hq][S][D]``)
    partials with the sink; returns ``[B][Hq][D]`` (or ``[B][T][Hq][D]``)."""
    if isinstance(part_o, torch.Tensor) and part_o.dim() == 5:      # rows (b*T + t)*Hq + h
        B, T, Hq, S, D = part_o.shape
        if out is not None:
            _check(out, "out", torch.bfloat16, 4, part_o.device)
            if tuple(out.shape) != (B, T, Hq, D):
                raise ValueError("out must be [B][T][Hq][D]")
        _check(part_lse, "part_lse", torch.float32, 4, part_o.device)
        res = combine(part_o.view(B * T, Hq, S, D), part_lse.view(B * T, Hq, S), sinks,
                      None if out is None else out.view(B * T, Hq, D), stream)
        return res.view(B, T, Hq, D)
    _check(part_o, "part_o", torch.float32, 4)
    dev = part_o.device
    _check(part_lse, "part_lse", torch.float32, 3, dev)
    B, Hq, S, D = part_o.shape
    if tuple(part_lse.shape) != (B, Hq, S):
        raise ValueError("part_lse must be [B][Hq][S]")
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, 1, dev)
        if sinks.shape[0] != Hq:
            raise ValueError("sinks must have one entry per query head")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 3, dev)
    d = Dims(B, Hq, 1, D, 16, 1, 1, 0, 0, 0, LAYOUT_K2_V8)
    with _on(dev):
        st = load().sa_combine(_ptr(part_o), _ptr(part_lse), _ptr(sinks), int(S), _ptr(out),
                               ctypes.byref(d), _stream(stream, dev))
    _raise(st, "sa_combine")
    return out


def read_bandwidth_probe(data, sink, stream=None):
    """Stream-read every byte of ``data`` once (the HBM read ceiling probe),
    XOR-folding its 32-bit words into ``sink`` (int32 device tensor, one
    element, start value set by the caller)."""
    if not isinstance(data, torch.Tensor) or not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous GPU tensor")
    _check(sink, "sink", torch.int32, 1, data.device)
    nbytes = data.numel() * data.element_size()
    with _on(data.device):
        st = load().sa_read_bandwidth_probe(_ptr(data), nbytes, _ptr(sink),
                                            _stream(stream, data.device))
    _raise(st, "sa_read_bandwidth_probe")


def read_tiles_probe(data, tiles, sink, waves=1024, stream=None):
    """Read the 2 KiB tiles of ``data`` that ``tiles`` (int32 tile numbers)
    lists, in the decode kernels' pattern, XOR-folding their 32-bit words into
    ``sink`` (int32 device tensor, one element, start value set by the caller)."""
    if not isinstance(data, torch.Tensor) or not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous GPU tensor")
    _check(tiles, "tiles", torch.int32, 1, data.device)
    _check(sink, "sink", torch.int32, 1, data.device)
    nbytes = data.numel() * data.element_size()
    with _on(data.device):
        st = load().sa_read_tiles_probe(_ptr(data), nbytes, _ptr(tiles), tiles.numel(), int(waves),
                                        _ptr(sink), _stream(stream, data.device))
    _raise(st, "sa_read_tiles_probe")
