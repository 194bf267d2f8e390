"""Plain float64 definitions of every step of the sparse-FFN decode path.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources ("the pages"):
  [R] PowerInfer reading report, egguo-blog "PowerInfer_2312.12456",
      Part A section 2.3 (operational definitions: sparsity, hot/cold split,
      neuron impact v_i = f_i; the five system modules), section 3.1
      (power-law finding), section 4.3 (neuron-aware operator avoids sparse
      formats), Part B (method formula).
  [B] the benchmark spec of the path this repository builds: a d -> r -> ffn
      predictor with a sigmoid over a threshold tau, neuron-major W_down rows,
      ReLU / ReGLU, no output bias.

Readings where the pages are silent (each one is listed with its reason in the
design notes of this repository):
  * predictor hidden nonlinearity is ReLU (or none); b1 optional;
  * "sigmoid(z) > tau" is taken strictly and evaluated as z > ln(tau/(1-tau));
  * the active index list is ascending with no duplicates;
  * ReGLU is a = max(W_gate x + b_gate, 0) * (W_up x + b_up), the gated form
    with the ReLU on the gate; ReLU is a = max(W_up x + b_up, 0);
  * SwiGLU ([R] Part A 2.3 and 4.4 name SiLU-gated models and their softer
    sparsity) is a = SiLU(W_gate x + b_gate) * (W_up x + b_up) with
    SiLU(g) = g / (1 + e^-g), over the listed neurons only;
  * a neuron "fires" for the profiler when its ReLU input is > 0 (strict);
  * reorder = stable sort by descending count (ties to the lower index), hot
    set = shortest prefix whose counts reach hot_share of the total.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


def widen(a) -> Optional[np.ndarray]:
    """fp16 / fp32 / torch / list -> float64 numpy (exact widening); None stays None."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor, possibly on a device
        a = a.detach().cpu().numpy()
    return np.asarray(a, dtype=F64)


def rows_of(W, rows) -> np.ndarray:
    """W[rows] widened to float64 (rows taken first, so a large matrix is never widened whole)."""
    rows = np.asarray(rows, dtype=np.int64)
    if hasattr(W, "detach"):
        W = W.detach().cpu().numpy()
    return np.asarray(np.asarray(W)[rows], dtype=F64)


def logit_threshold(tau: float) -> float:
    """The predictor marks neuron i active when sigmoid(z_i) > tau [B].

    sigmoid is strictly increasing, so sigmoid(z) > tau  <=>  z > ln(tau/(1-tau)).
    """
    if not (0.0 < tau < 1.0):
        raise ValueError("tau must lie in (0, 1)")
    return math.log(tau / (1.0 - tau))


def predictor_hidden(x, P1, b1=None, act: str = "relu") -> np.ndarray:
    """Hidden layer of the per-layer predictor MLP ([R] Part A 2.3, module 3).

    s = P1 x + b1 (P1 is r x d), h = ReLU(s) (act "relu") or h = s ("none").
    """
    x, P1, b1 = widen(x), widen(P1), widen(b1)
    s = P1 @ x
    if b1 is not None:
        s = s + b1
    if act == "relu":
        return np.maximum(s, 0.0)
    if act == "none":
        return s
    raise ValueError(f"unknown predictor activation {act!r}")


def predictor_logits(x, P1, b1, act, P2, b2) -> np.ndarray:
    """z = P2 h + b2 (P2 is ffn x r); one logit per FFN neuron."""
    h = predictor_hidden(x, P1, b1, act)
    z = widen(P2) @ h
    if b2 is not None:
        z = z + widen(b2)
    return z


def predict(x, P1, b1, act, P2, b2, tau) -> Tuple[np.ndarray, np.ndarray]:
    """Active-neuron list of one token: ascending i with sigmoid(z_i) > tau.

    Returns (idx int64 ascending, z float64).  count = len(idx).
    """
    z = predictor_logits(x, P1, b1, act, P2, b2)
    idx = np.flatnonzero(z > logit_threshold(tau))
    return idx, z


def predict_hot(x, P1, b1, act, P2, b2, tau, n_hot) -> Tuple[np.ndarray, np.ndarray]:
    """The list of a hot-first layer whose first n_hot neurons are always listed.

    After profiling and the hot-first reorder ([R] Part A 2.3 modules 1-2: the
    hot neurons are the frequent ones, placed up front), neurons 0..n_hot-1 are
    active without consulting the predictor; the predictor decides the rest
    from rows n_hot.. of P2 and b2 alone.  idx = 0..n_hot-1, then n_hot + the
    ascending active positions among the others; z is +inf on the prefix.
    """
    n_hot = int(n_hot)
    P2c = np.asarray(P2)[n_hot:]
    b2c = None if b2 is None else np.asarray(b2)[n_hot:]
    z_rest = predictor_logits(x, P1, b1, act, P2c, b2c)
    rest = n_hot + np.flatnonzero(z_rest > logit_threshold(tau))
    idx = np.concatenate([np.arange(n_hot, dtype=np.int64), rest.astype(np.int64)])
    return idx, np.concatenate([np.full(n_hot, np.inf), z_rest])


def neuron_preactivations(kind, x, W_up, b_up, W_gate, b_gate, rows) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """u_i = W_up[i] x + b_up_i and (ReGLU) g_i = W_gate[i] x + b_gate_i for i in rows.

    The neuron-aware operator works on whole neuron rows with no sparse
    format ([R] Part A 2.3 module 4, 4.3): row i of each matrix is neuron i.
    """
    rows = np.asarray(rows, dtype=np.int64)
    x = widen(x)
    u = rows_of(W_up, rows) @ x
    if b_up is not None:
        u = u + rows_of(b_up, rows)
    g = None
    if kind in ("reglu", "swiglu"):
        g = rows_of(W_gate, rows) @ x
        if b_gate is not None:
            g = g + rows_of(b_gate, rows)
    elif kind != "relu":
        raise ValueError(f"unknown FFN kind {kind!r}")
    return u, g


def silu(g) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + e^-g), in float64 (e^-g may overflow
    to inf for g below about -709, which gives the limit -0)."""
    g = np.asarray(g, dtype=F64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def neuron_activations(kind, x, W_up, b_up, W_gate, b_gate, rows) -> np.ndarray:
    """a_i = max(u_i, 0) (ReLU), max(g_i, 0) * u_i (ReGLU) or SiLU(g_i) * u_i
    (SwiGLU) for i in rows."""
    u, g = neuron_preactivations(kind, x, W_up, b_up, W_gate, b_gate, rows)
    if kind == "relu":
        return np.maximum(u, 0.0)
    if kind == "swiglu":
        return silu(g) * u
    return np.maximum(g, 0.0) * u


def sparse_ffn(kind, x, W_up, b_up, W_gate, b_gate, W_down, idx) -> np.ndarray:
    """y = sum over i in idx (ascending) of a_i * W_down[i, :]; no output bias.

    W_down is neuron-major (ffn x d): row i is neuron i's output vector, so
    only the rows of active neurons are touched ([R] Part A 2.3 module 4).
    """
    idx = np.asarray(idx, dtype=np.int64)
    y = np.zeros(np.shape(W_down)[1], dtype=F64)
    if idx.size == 0:
        return y
    a = neuron_activations(kind, x, W_up, b_up, W_gate, b_gate, idx)
    Wd = rows_of(W_down, idx)
    for ai, wrow in zip(a, Wd):        # ascending accumulation order
        y += ai * wrow
    return y


def dense_ffn(kind, x, W_up, b_up, W_gate, b_gate, W_down) -> np.ndarray:
    """The dense FFN: every neuron computed, no predictor."""
    ffn = np.shape(W_up)[0]
    return sparse_ffn(kind, x, W_up, b_up, W_gate, b_gate, W_down, np.arange(ffn))


def decode_step(layer: dict, x) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Predict the active set of one token, then compute only those neurons.

    Returns (y, idx, z).  `layer` holds the tensors named as in the C ABI.
    """
    idx, z = predict(x, layer["P1"], layer.get("b1"), layer.get("pred_act", "relu"),
                     layer["P2"], layer["b2"], layer["tau"])
    y = sparse_ffn(layer["kind"], x, layer["W_up"], layer.get("b_up"), layer.get("W_gate"),
                   layer.get("b_gate"), layer["W_down"], idx)
    return y, idx, z


def batched_sparse_ffn(kind, X, W_up, b_up, W_gate, b_gate, W_down,
                       idx_lists: Sequence[Sequence[int]]) -> np.ndarray:
    """Batch of B tokens: token t uses only its own active list (per-token masks).

    The result for token t is by definition the single-token result; loading
    the union of the lists once is an implementation choice that must not
    change it.
    """
    X = widen(X)
    return np.stack([sparse_ffn(kind, X[t], W_up, b_up, W_gate, b_gate, W_down, idx_lists[t])
                     for t in range(X.shape[0])])


def union_rows(idx_lists: Sequence[Sequence[int]]) -> np.ndarray:
    """Ascending union of the per-token active lists."""
    if len(idx_lists) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate([np.asarray(l, dtype=np.int64) for l in idx_lists]))


def profile_preactivations(X, W_fire, b_fire) -> np.ndarray:
    """pre[t, i] = W_fire[i] x_t + b_fire_i, the ReLU input of neuron i for token t."""
    X, W = widen(X), widen(W_fire)
    pre = X @ W.T                       # (n, ffn)
    if b_fire is not None:
        pre = pre + widen(b_fire)[None, :]
    return pre


def profile_counts(kind, X, W_fire, b_fire) -> np.ndarray:
    """Offline profiler: per-neuron activation counts over calibration tokens.

    counts_i = #{t : W_fire[i] x_t + b_fire_i > 0}, the number of tokens for
    which neuron i's ReLU input is positive ([R] Part A 2.2 profiling data,
    2.3 module 1 and the neuron impact v_i = f_i = counts_i / n).  W_fire is
    W_up for ReLU FFNs and W_gate for ReGLU FFNs.
    """
    if kind not in ("relu", "reglu"):
        raise ValueError(f"unknown FFN kind {kind!r}")
    return (profile_preactivations(X, W_fire, b_fire) > 0.0).sum(axis=0).astype(np.int64)


def reorder_plan(counts, hot_share: float = 0.8) -> Tuple[np.ndarray, int]:
    """Hot-first neuron order and the size of the hot set.

    perm (new -> old) sorts neurons by descending count, ties kept in original
    order.  hot_count is the smallest k whose first k sorted counts reach
    hot_share of all activations: the hot neurons are the minority that
    carries 80% of the activations ([R] Part A 2.3 "hot/cold neurons", 3.1).
    hot_count is 0 when no neuron ever fired.
    """
    counts = np.asarray(counts, dtype=np.int64)
    perm = np.argsort(-counts, kind="stable")
    total = int(counts.sum())
    if total == 0:
        return perm.astype(np.int64), 0
    target = float(hot_share) * float(total)
    running = 0
    for k, i in enumerate(perm, start=1):
        running += int(counts[i])
        if float(running) >= target:
            return perm.astype(np.int64), k
    return perm.astype(np.int64), len(perm)


def permute_rows(src, perm) -> np.ndarray:
    """dst[j] = src[perm[j]]: apply a new -> old neuron order to a row-major tensor."""
    if hasattr(src, "detach"):
        src = src.detach().cpu().numpy()
    src = np.asarray(src)
    return src[np.asarray(perm, dtype=np.int64)].copy()


def quantize_rows(W) -> Tuple[np.ndarray, np.ndarray]:
    """INT4 rows, the library's own group-wise format ([R] Part A 3.1 reports
    INT4 results without a format).  Per group of 64 weights of a row, in fp32:
    s = fp16(max|w| / 7) (IEEE division, round to nearest even), code =
    clamp(rint(w / s), -8, 7) + 8 (rint: half to even; 8 when s = 0).  Codes
    are packed two per byte, the even weight in the low nibble.  Returns
    (codes rows x d/2 uint8, scales rows x d/64 float16)."""
    W32 = np.asarray(W, dtype=np.float16).astype(np.float32)
    rows, d = W32.shape
    G = W32.reshape(rows, d // 64, 64)
    amax = np.abs(G).max(axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    c = np.zeros(G.shape, dtype=np.int64)
    nz = np.broadcast_to(s32 != 0, G.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        c[nz] = np.clip(np.rint(G / s32), -8, 7)[nz].astype(np.int64)
    codes = (c + 8).reshape(rows, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, s16


def dequantize_rows(q, s, d: int) -> np.ndarray:
    """The weights INT4 rows stand for, in float64: (code - 8) * s."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.empty((q.shape[0], d), dtype=np.int64)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    scale = np.repeat(np.asarray(s, dtype=np.float16).astype(F64), 64, axis=1)
    return (codes - 8).astype(F64) * scale
