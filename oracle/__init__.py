"""fp64 CPU oracle of the Star Attention hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package; the HIP library never does.
"""
from .star_oracle import (  # noqa: F401
    ANCHORS, NEG_INF, attention, augmented_block, augmented_positions, exact_causal, merge, merge_pairwise_literal,
    phase1, phase1_block, phase2_partials, phase2_plain, rope, rope_inv_freq, tail_keys,
)
