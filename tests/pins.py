"""Independent routes that pin the oracle (CPU only, no GPU, no HIP library).

Every route here is written separately from ``oracle/``:

* ``History`` holds K/V per *logical position* (no blocks, no ring) and
  ``lay_out`` writes a history into the documented paged / ring layout the
  way a cache writer would, so the oracle's reader side is checked against a
  layout-free statement;
* ``brute_force`` is pure Python (``struct`` widening, ``math.exp``,
  ``math.fsum``) over an explicit dense mask with an extra sink column;
* ``sdpa_route`` is torch's fp64 ``scaled_dot_product_attention`` on the CPU
  with KV heads repeated per query head and the sink as one extra key whose
  value row is zero and whose additive bias is the sink logit.

Each ``pin_*`` function raises ``AssertionError`` when the oracle module it is
given disagrees; the planted-mistake tests rely on that.
"""

from __future__ import annotations

import dataclasses
import math
import struct

import numpy as np
import torch


# ---------------------------------------------------------------------------
# bf16 helpers (test side)
# ---------------------------------------------------------------------------

def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.uint16).numpy().copy()


def bits_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


# ---------------------------------------------------------------------------
# Layout-free history and its layout writer
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class History:
    q: np.ndarray        # uint16 [B][Hq][D]
    K: np.ndarray        # uint16 [B][Lmax][Hkv][D]   K of each logical position
    V: np.ndarray        # uint16 [B][Lmax][Hkv][D]
    lens: np.ndarray     # [B] context length (after the append)
    sinks: np.ndarray | None  # float32 [Hq]


def make_history(seed, B, Hq, Hkv, D, lens, sinks=True, q_zero=False):
    g = torch.Generator().manual_seed(seed)
    lens = np.asarray(lens, dtype=np.int64)
    Lmax = max(1, int(lens.max()))
    q = torch.randn(B, Hq, D, generator=g)
    if q_zero:
        q.zero_()
    K = torch.randn(B, Lmax, Hkv, D, generator=g)
    V = torch.randn(B, Lmax, Hkv, D, generator=g)
    s = torch.randn(Hq, generator=g).numpy().astype(np.float32) if sinks else None
    return History(bf16_bits(q), bf16_bits(K), bf16_bits(V), lens, s)


POISON_BITS = 0x4780   # bf16 65536.0: finite, and far outside N(0,1)


def lay_out(h: History, window: int, bs: int, table: str = "shuffled", seed: int = 0,
            cap_lens=None):
    """Write the history into a K pool [NB][Hkv][2][bs][D/2] (each K row in two
    halves, each half slot-major), a V pool [NB][Hkv][bs/c][D][c] (V
    transposed inside a block in chunks of c = min(8, bs) slots), the
    library's layouts for its block sizes, and a block table.

    A full layer (window <= 0) keeps every position p < L in slot p; a ring
    layer keeps the last ``window`` positions, position p in slot p % window.
    Every slot that holds no attended position keeps the poison value, and
    unused table entries name a poison block.  ``cap_lens`` (default: the
    lengths) sizes each full-layer sequence's blocks.
    """
    B, Lmax, Hkv, D = h.K.shape
    rng = np.random.default_rng(seed)
    if window > 0:
        nblk = [-(-window // bs)] * B
    else:
        nblk = [max(1, -(-int(L) // bs)) for L in (h.lens if cap_lens is None else cap_lens)]
    used = sum(nblk)
    NB = used + 2
    ids = rng.permutation(NB) if table == "shuffled" else np.arange(NB)
    poison_block = int(ids[used])
    mbs = max(nblk)
    bt = np.full((B, mbs), poison_block, dtype=np.int32)
    n = 2 if D % 2 == 0 else 1                 # K row pieces (the library's 2)
    kp = np.full((NB, Hkv, n, bs, D // n), POISON_BITS, dtype=np.uint16)
    c = min(8, bs)
    vp = np.full((NB, Hkv, bs // c, D, c), POISON_BITS, dtype=np.uint16)
    start = 0
    for b in range(B):
        bt[b, :nblk[b]] = ids[start:start + nblk[b]]
        start += nblk[b]
        L = int(h.lens[b])
        first = 0 if window <= 0 else max(0, L - window)
        for p in range(first, L):
            slot = p if window <= 0 else p % window
            blk = bt[b, slot // bs]
            off = slot % bs
            kp[blk, :, :, off, :] = h.K[b, p].reshape(Hkv, n, D // n)
            vp[blk, :, off // c, :, off % c] = h.V[b, p]
    return kp, vp, bt


# ---------------------------------------------------------------------------
# Route (i): pure-Python brute force over a dense mask plus a sink column
# ---------------------------------------------------------------------------

def brute_force(h: History, window: int):
    B, Hq, D = h.q.shape
    Hkv = h.K.shape[2]
    G = Hq // Hkv
    kv_of_head = [g for g in range(Hkv) for _ in range(G)]   # repetition, not division
    Lmax = h.K.shape[1]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(h.lens[b])
        mask = [p < L and (window <= 0 or p >= L - window) for p in range(Lmax)]
        for hh in range(Hq):
            g = kv_of_head[hh]
            qv = [bits_to_float(x) for x in h.q[b, hh]]
            row = []
            for p in range(Lmax):
                if mask[p]:
                    kv = [bits_to_float(x) for x in h.K[b, p, g]]
                    row.append(math.fsum(a * c for a, c in zip(qv, kv)) / math.sqrt(D))
                else:
                    row.append(-math.inf)
            sigma = -math.inf if h.sinks is None else float(h.sinks[hh])
            row.append(sigma)                      # the sink column
            m = max(row)
            if m == -math.inf:
                continue
            e = [math.exp(x - m) for x in row]
            Z = math.fsum(e)
            for d in range(D):
                terms = [e[p] * bits_to_float(h.V[b, p, g, d]) for p in range(Lmax) if mask[p]]
                out[b, hh, d] = math.fsum(terms) / Z   # the sink column has no value
    return out


# ---------------------------------------------------------------------------
# Route (ii): torch fp64 SDPA with the sink as an extra zero key
# ---------------------------------------------------------------------------

def _widen(bits):
    return torch.from_numpy(bits.astype(np.int32) << 16).view(torch.float32).double()


def sdpa_route(h: History, window: int):
    B, Hq, D = h.q.shape
    _, Lmax, Hkv, _ = h.K.shape
    G = Hq // Hkv
    q = _widen(h.q).unsqueeze(2)                                     # [B,Hq,1,D]
    K = _widen(h.K).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)   # [B,Hq,L,D]
    V = _widen(h.V).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    zero = torch.zeros(B, Hq, 1, D, dtype=torch.float64)
    K = torch.cat([K, zero], dim=2)
    V = torch.cat([V, zero], dim=2)
    bias = torch.full((B, Hq, 1, Lmax + 1), -math.inf, dtype=torch.float64)
    for b in range(B):
        L = int(h.lens[b])
        lo = 0 if window <= 0 else max(0, L - window)
        bias[b, :, 0, lo:L] = 0.0
    sig = (torch.full((Hq,), -math.inf, dtype=torch.float64) if h.sinks is None
           else torch.from_numpy(h.sinks.astype(np.float64)))
    bias[:, :, 0, Lmax] = sig
    out = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=bias,
                                                           scale=1.0 / math.sqrt(D))
    return out.squeeze(2).numpy()


# ---------------------------------------------------------------------------
# Pins: each takes the oracle module so a planted mistake can be checked
# ---------------------------------------------------------------------------

def run_oracle(oracle, h: History, window: int, bs: int, table="shuffled", seed=0):
    kp, vp, bt = lay_out(h, window, bs, table, seed)
    return oracle.decode_attention(h.q, kp, vp, bt, h.lens, h.sinks, window)


def assert_close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


BRUTE_CASES = [
    # (B, Hq, Hkv, D, lens, window, bs)
    (1, 4, 1, 64, [38], 0, 16),            # the tiny config: 37 cached + 1 new
    (1, 4, 1, 64, [37], 0, 16),
    (2, 4, 2, 64, [1, 2], 0, 16),
    (2, 4, 2, 64, [15, 16], 0, 16),
    (2, 4, 2, 64, [17, 33], 0, 16),
    (2, 4, 2, 64, [7, 20], 16, 16),         # ring, window == block size
    (2, 4, 2, 64, [5, 23], 5, 4),           # ring, window not a multiple of bs
    (2, 6, 3, 16, [9, 31], 12, 8),
]


def pin_brute_force(oracle, cases=BRUTE_CASES, seed=11):
    for i, (B, Hq, Hkv, D, lens, W, bs) in enumerate(cases):
        h = make_history(seed + i, B, Hq, Hkv, D, lens)
        assert_close(run_oracle(oracle, h, W, bs, seed=i), brute_force(h, W), 1e-12,
                     f"brute case {i}")
        h0 = make_history(seed + 100 + i, B, Hq, Hkv, D, lens, sinks=False)
        assert_close(run_oracle(oracle, h0, W, bs, seed=i), brute_force(h0, W), 1e-12,
                     f"brute no-sink case {i}")


SDPA_CASES = [
    (3, 8, 2, 64, [1, 50, 100], 0, 16),
    (3, 8, 2, 64, [40, 128, 129], 32, 16),
    (2, 16, 4, 32, [77, 200], 64, 32),
    (2, 8, 8, 64, [33, 65], 0, 8),
]


def pin_sdpa(oracle, cases=SDPA_CASES, seed=21):
    for i, (B, Hq, Hkv, D, lens, W, bs) in enumerate(cases):
        h = make_history(seed + i, B, Hq, Hkv, D, lens)
        assert_close(run_oracle(oracle, h, W, bs, seed=i), sdpa_route(h, W), 1e-12,
                     f"sdpa case {i}")


def pin_closed_forms(oracle, seed=31):
    D = 64
    # L = 1 with a sink: out = v0 * e^{s0} / (e^{s0} + e^{sigma})
    h = make_history(seed, 2, 4, 2, D, [1, 1])
    out = run_oracle(oracle, h, 0, 16)
    for b in range(2):
        for hh in range(4):
            g = hh // 2
            qv = h.q[b, hh].astype(np.int64)
            s0 = sum(bits_to_float(a) * bits_to_float(c) for a, c in zip(qv, h.K[b, 0, g])) / 8.0
            w = 1.0 / (1.0 + math.exp(float(h.sinks[hh]) - s0))
            expect = w * np.array([bits_to_float(x) for x in h.V[b, 0, g]])
            assert_close(out[b, hh], expect, 1e-12, "L=1 sigmoid")
    # L = 1 without a sink: out = v0 exactly
    h = make_history(seed + 1, 1, 2, 1, D, [1], sinks=False)
    out = run_oracle(oracle, h, 0, 16)
    v0 = np.array([bits_to_float(x) for x in h.V[0, 0, 0]])
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0), "L=1 no sink"
    # q = 0: uniform weights, out = mean(V) * n / (n + e^sigma), also through a ring
    for W, L in ((0, 45), (16, 45), (64, 45)):
        h = make_history(seed + 2, 1, 4, 1, D, [L], q_zero=True)
        out = run_oracle(oracle, h, W, 16)
        n = L if W <= 0 else min(L, W)
        Vw = np.array([[bits_to_float(x) for x in h.V[0, p, 0]] for p in range(L - n, L)])
        for hh in range(4):
            expect = Vw.mean(axis=0) * n / (n + math.exp(float(h.sinks[hh])))
            assert_close(out[0, hh], expect, 1e-12, f"q=0 W={W}")
    # all V rows equal c: out = c * sum e^s / (sum e^s + e^sigma)
    h = make_history(seed + 3, 1, 2, 1, D, [20])
    h.V[:] = h.V[0, 0, 0][None, None, None, :]
    out = run_oracle(oracle, h, 0, 16)
    c = np.array([bits_to_float(x) for x in h.V[0, 0, 0]])
    for hh in range(2):
        s = [sum(bits_to_float(a) * bits_to_float(k) for a, k in zip(h.q[0, hh], h.K[0, p, 0])) / 8.0
             for p in range(20)]
        es = sum(math.exp(x) for x in s)
        assert_close(out[0, hh], c * es / (es + math.exp(float(h.sinks[hh]))), 1e-12, "const V")
    # identical K rows: uniform weights over the window
    h = make_history(seed + 4, 1, 2, 1, D, [30])
    h.K[:] = h.K[0, 0][None, None, :, :]
    out = run_oracle(oracle, h, 0, 16)
    Vw = np.array([[bits_to_float(x) for x in h.V[0, p, 0]] for p in range(30)])
    for hh in range(2):
        s = sum(bits_to_float(a) * bits_to_float(k) for a, k in zip(h.q[0, hh], h.K[0, 0, 0])) / 8.0
        w = 30 * math.exp(s) / (30 * math.exp(s) + math.exp(float(h.sinks[hh])))
        assert_close(out[0, hh], Vw.mean(axis=0) * w, 1e-12, "identical K")


def pin_invariants(oracle, seed=41):
    D = 64
    lens = [1, 16, 17, 40, 100]
    h = make_history(seed, 5, 8, 2, D, lens)
    # sigma = -inf per head equals no sinks at all
    hn = dataclasses.replace(h, sinks=np.full(8, -np.inf, dtype=np.float32))
    h0 = dataclasses.replace(h, sinks=None)
    assert_close(run_oracle(oracle, hn, 0, 16), run_oracle(oracle, h0, 0, 16), 0.0, "-inf sink")
    # a window at least the context equals full attention (different layouts)
    assert_close(run_oracle(oracle, h, 100, 16), run_oracle(oracle, h, 0, 16), 1e-12, "W>=L")
    assert_close(run_oracle(oracle, h, 128, 16), run_oracle(oracle, h, 0, 16), 1e-12, "W>L")
    # paged with a shuffled table equals the identity (contiguous) table, exactly
    assert np.array_equal(run_oracle(oracle, h, 0, 16, "shuffled", 5),
                          run_oracle(oracle, h, 0, 16, "identity")), "paged vs contiguous"
    assert np.array_equal(run_oracle(oracle, h, 24, 8, "shuffled", 6),
                          run_oracle(oracle, h, 24, 8, "identity")), "ring paged vs contiguous"
    # the block size does not change the result
    assert_close(run_oracle(oracle, h, 0, 8), run_oracle(oracle, h, 0, 32), 1e-12, "block size")
    # GQA equals MHA with each KV head repeated for its query heads
    G = 4
    hm = dataclasses.replace(h, K=np.repeat(h.K, G, axis=2), V=np.repeat(h.V, G, axis=2))
    assert_close(run_oracle(oracle, h, 0, 16), run_oracle(oracle, hm, 0, 16), 1e-12, "GQA=MHA")
    assert_close(run_oracle(oracle, h, 24, 16), run_oracle(oracle, hm, 24, 16), 1e-12, "GQA=MHA ring")
    # stale slots and unused table entries never matter: NaN them out
    kp, vp, bt = lay_out(h, 0, 16)
    ref = oracle.decode_attention(h.q, kp, vp, bt, h.lens, h.sinks, 0)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[kp2 == POISON_BITS] = 0x7FC0     # bf16 NaN
    vp2[vp2 == POISON_BITS] = 0x7FC0
    assert np.array_equal(oracle.decode_attention(h.q, kp2, vp2, bt, h.lens, h.sinks, 0), ref), \
        "stale slots leak"


def pin_combine(oracle, seed=51):
    """combine(any partition of the attended positions) == one-shot."""
    D = 64
    rng = np.random.default_rng(seed)
    for W in (0, 20):
        h = make_history(seed, 3, 4, 2, D, [1, 37, 90])
        kp, vp, bt = lay_out(h, W, 16)
        ref = oracle.decode_attention(h.q, kp, vp, bt, h.lens, h.sinks, W)
        for S in (1, 2, 5, 17):
            po = np.zeros((3, 4, S, D))
            pl = np.full((3, 4, S), -np.inf)
            for b in range(3):
                L = int(h.lens[b])
                pos = list(range(0 if W <= 0 else max(0, L - W), L))
                owner = rng.integers(0, S, size=len(pos))        # random sets, some empty
                for hh in range(4):
                    for p in range(S):
                        sub = [x for x, o in zip(pos, owner) if o == p]
                        po[b, hh, p], pl[b, hh, p] = oracle.partial_attention(
                            h.q, kp, vp, bt, b, hh, sub, W)
            assert_close(oracle.combine(po, pl, h.sinks), ref, 1e-12, f"combine S={S} W={W}")
            assert_close(oracle.combine(po, pl, None),
                         oracle.decode_attention(h.q, kp, vp, bt, h.lens, None, W), 1e-12,
                         f"combine no-sink S={S}")


def pin_append(oracle, seed=61):
    """The oracle's append equals laying out the history that includes the new
    token, bit for bit; nothing else in the pool changes."""
    D = 64
    for W, bs, lens in ((0, 16, [1, 16, 17, 38]), (0, 8, [9, 3, 40, 64]),
                        (16, 16, [1, 16, 17, 50]), (12, 8, [5, 12, 13, 40])):
        h = make_history(seed, 4, 4, 2, D, lens)
        # the layout before: every position but the last
        before = dataclasses.replace(h, lens=h.lens - 1)
        kp0, vp0, bt = lay_out(before, W, bs, seed=3, cap_lens=h.lens)
        kp1, vp1, bt1 = lay_out(h, W, bs, seed=3)
        assert np.array_equal(bt, bt1)
        k_new = np.stack([h.K[b, h.lens[b] - 1] for b in range(4)])
        v_new = np.stack([h.V[b, h.lens[b] - 1] for b in range(4)])
        ka, va = oracle.kv_append(kp0, vp0, k_new, v_new, bt, h.lens, W)
        # in a ring the new token overwrites the position that has just left
        # the window, so the pool after is exactly the layout of h
        assert np.array_equal(ka, kp1) and np.array_equal(va, vp1), f"append W={W} bs={bs}"


def pin_append_past_capacity(oracle, seed=67):
    """A sequence whose new token's slot lies past its table row (a length
    beyond the table's capacity, which the library documents as appending
    nothing) leaves the pools untouched; the other sequences of the same call
    append as usual.  Checked against the history layouts, bit for bit."""
    D = 64
    for bs in (8, 16):
        h = make_history(seed, 3, 4, 2, D, [20, 30, 9])
        before = dataclasses.replace(h, lens=h.lens - 1)
        kp0, vp0, bt = lay_out(before, 0, bs, seed=5, cap_lens=h.lens)
        kp1, vp1, _ = lay_out(h, 0, bs, seed=5)
        cap = bt.shape[1] * bs
        k_new = np.stack([h.K[b, h.lens[b] - 1] for b in range(3)])
        v_new = np.stack([h.V[b, h.lens[b] - 1] for b in range(3)])
        for L1 in (cap + 1, cap + 8, 3 * cap + 5):
            lens = h.lens.copy()
            lens[1] = L1                             # new slot L1-1 >= cap: past the row
            ka, va = oracle.kv_append(kp0, vp0, k_new, v_new, bt, lens, 0)
            own1 = bt[1, :-(-int(h.lens[1]) // bs)]  # sequence 1's blocks: as before
            want_k, want_v = kp1.copy(), vp1.copy()
            want_k[own1], want_v[own1] = kp0[own1], vp0[own1]
            assert np.array_equal(ka, want_k) and np.array_equal(va, want_v), \
                f"append past capacity bs={bs} L={L1}"
