"""Seeded synthetic inputs for the sparse-FFN decode path.

This package builds inputs only: random weight matrices, per-neuron firing
probabilities, the biases that produce those probabilities, and tokens.  It
holds none of the method's arithmetic (no predictor, threshold, compaction,
FFN, profile or reorder), so both the HIP path and the CPU oracle can be fed
from it without sharing any of the computation under test.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    firing_law,
    solve_exponent,
    rank_probabilities,
    make_layer,
    make_tokens,
    make_calibration,
    custom_config,
)
