"""MI355X (gfx950) neuron-aware sparse FFN for one decode step.

The computation lives in the HIP library libpi.so (C ABI in include/pi.h):
predictor MLP -> ordered index compaction -> gathered up/gate GEMV ->
neuron-major W_down accumulate, plus the offline profile and hot-first
reorder.  `binding` exposes the C entry points under the same names and
`runtime` adds device-buffer plumbing (workspaces, layer bundles).
"""

from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    PI_OK, PI_DENSE, PI_FFN_RELU, PI_FFN_REGLU, PI_ACT_RELU, PI_ACT_NONE,
    PI_OP_PREDICT, PI_OP_SPARSE, PI_OP_PROFILE, PiError,
)
