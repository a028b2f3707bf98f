"""Oracle for the paged GQA decode-attention step: TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 CPU statement of what the decode step
computes. It exists to check the HIP library, never to stand in for it:

* only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
  ``bench.py`` may import it;
* it shares no code, constants or helpers with ``paged_gqa_decode_step_amd``
  and imports nothing from it;
* every function states the passage of the source pages it follows.  The
  pages name the operations (a fused decode-attention kernel covering
  attention sinks, sliding window, GQA and the KV append; a paged KV cache
  for full-attention layers; a ring buffer for sliding-window layers) but
  print no formula, so each definition below is the plain textbook reading
  of the named concept, stated where it is used.

``oracle.rope`` adds the decode step with the rotary position embedding of
the new token's query and key (the SimpleLLM README lists a fused RoPE kernel), and
``oracle.multi_token`` the step with T > 1 causal query tokens per sequence.

Pins (tests/test_oracle_*.py, ``-m "not gpu"``): a pure-Python brute force
over a layout-free history, torch's fp64 ``scaled_dot_product_attention``
with the sink as an extra key, closed forms, invariants, a hand-derived
golden example, and planted-mistake tests showing that the pins catch a
dropped sink, a wrong head-to-group map and a wrong ring slot.
"""

from .decode_step import (  # noqa: F401
    bf16_bits_to_f64,
    query_group,
    attended_positions,
    storage_slot,
    locate,
    decode_attention,
    partial_attention,
    combine,
    kv_append,
)
from . import rope  # noqa: F401,E402
from . import multi_token  # noqa: F401,E402
