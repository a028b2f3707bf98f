"""Seeded synthetic inputs for the decode step: shared by the tests, the bench
and the smoke check.

This package holds no part of the attention arithmetic: it draws random
pools, shuffled block tables, lengths, queries, sinks and new-token rows, and
hands the same tensors to both the HIP library and the oracle.  It imports
neither of them.
"""

from .workloads import (  # noqa: F401
    Layer,
    make_layer,
    ragged_lengths,
    to_bits,
    CONFIGS,
)
