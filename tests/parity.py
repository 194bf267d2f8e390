"""Parity rules between the HIP path and the oracle.

Index lists: bit-exact (ascending, no duplicates) except neurons whose oracle
logit lies within 1e-3 of the decision threshold ln(tau/(1-tau)); such a
neuron may appear or not.  y: the oracle is evaluated on the GPU's own index
list, and must match with relative L2 error <= 1e-3 and max-abs error
<= 2e-3 * ||y_oracle||_inf; an all-zero oracle output must be matched
exactly.  Profile counts: every neuron's count lies between the number of
tokens whose oracle pre-activation exceeds +1e-3 and the number exceeding
-1e-3 (tokens within the band may go either way).
"""

import math

import numpy as np

BAND = 1e-3
REL_L2 = 1e-3
MAX_ABS = 2e-3


def check_idx(gpu_idx, z, thr, band=BAND, where=""):
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    ffn = len(z)
    assert np.all(np.diff(gpu_idx) > 0), f"{where}: index list not strictly ascending"
    assert gpu_idx.size == 0 or (gpu_idx[0] >= 0 and gpu_idx[-1] < ffn), f"{where}: index out of range"
    must = np.flatnonzero(z > thr + band)
    may = np.flatnonzero(np.abs(z - thr) <= band)
    got = set(gpu_idx.tolist())
    missing = set(must.tolist()) - got
    extra = got - set(must.tolist()) - set(may.tolist())
    assert not missing and not extra, (
        f"{where}: {len(missing)} missing (e.g. {sorted(missing)[:5]}), "
        f"{len(extra)} extra (e.g. {sorted(extra)[:5]}) of {len(must)} required")
    return len(may)


def check_y(y_gpu, y_ref, where=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, f"{where}: shape {y_gpu.shape} vs {y_ref.shape}"
    assert np.all(np.isfinite(y_gpu)), f"{where}: non-finite output"
    inf = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    if inf == 0.0:
        assert np.all(y_gpu == 0.0), f"{where}: oracle output is 0 but GPU max |y| = {np.max(np.abs(y_gpu))}"
        return 0.0
    diff = y_gpu - y_ref
    rel = float(np.linalg.norm(diff) / np.linalg.norm(y_ref))
    mx = float(np.max(np.abs(diff)))
    assert rel <= REL_L2, f"{where}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS * inf, f"{where}: max abs {mx:.3e} > {MAX_ABS} * {inf:.3e}"
    return rel


def check_counts(gpu_counts, pre, band=BAND, where=""):
    """pre: (n, ffn) oracle pre-activations."""
    lo = (pre > band).sum(axis=0)
    hi = (pre > -band).sum(axis=0)
    c = np.asarray(gpu_counts, dtype=np.int64)
    bad = np.flatnonzero((c < lo) | (c > hi))
    assert bad.size == 0, f"{where}: {bad.size} counts outside their band, e.g. neuron {bad[:5]}: {c[bad[:5]]} vs [{lo[bad[:5]]}, {hi[bad[:5]]}]"


def logit(tau):
    return math.log(tau / (1.0 - tau))
