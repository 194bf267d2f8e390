"""CPU oracle for the neuron-aware sparse FFN decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything under this directory: only the test suite, the smoke
check at the repository root (smoke()), and the benchmark's cpu_baseline
leg use it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or pre/post-processing) and never reads a value the
HIP library produced except the index list it is asked to evaluate y on.

Everything is plain numpy in float64: every fp16 input is widened exactly,
every product and sum is taken in double precision, library matmul is the only
primitive used.  See `oracle.ffn` for the functions and the passages of the
PowerInfer pages each one follows.

Pins: every function here is checked by the `-m "not gpu"` tests against
exact rational brute force on tiny inputs, closed forms, invariants and
hand-worked fixtures (tests/golden).  No function is "parity unpinned".
"""

from .ffn import (  # noqa: F401
    widen,
    logit_threshold,
    predictor_hidden,
    predictor_logits,
    predict,
    predict_hot,
    neuron_preactivations,
    neuron_activations,
    silu,
    sparse_ffn,
    dense_ffn,
    decode_step,
    batched_sparse_ffn,
    union_rows,
    profile_preactivations,
    profile_counts,
    rows_of,
    reorder_plan,
    permute_rows,
    quantize_rows,
    dequantize_rows,
)
