"""Device-buffer plumbing around the C ABI: workspaces, outputs, layer bundles.

Nothing here computes part of the path.  torch provides device memory and the
stream; every arithmetic step runs in libpi's HIP kernels via `binding`.
A layer is a dict of device tensors named as in the C ABI (W_up, W_gate,
W_down, b_up, b_gate, P1, b1, P2, b2) plus kind, tau and sizes.
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import torch

from . import binding as B


class Workspace:
    """A grow-only device byte buffer, 256-byte aligned (torch allocations are)."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> Tuple[Optional[torch.Tensor], int]:
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            # zero-filled once: the library keeps epoch-tagged sync words in its header
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


_WS: Dict[Tuple[str, int], Workspace] = {}


def workspace(tag: str, device=None) -> Workspace:
    """The workspace kept under `tag` on a device.  Each layout (single-token
    and batched calls of an entry point, the dense baseline) gets its own tag,
    so that calls alternating between layouts never make the library clear a
    workspace, and a captured graph never meets a workspace that another
    layout wrote between its replays."""
    dev = torch.device(device or "cuda")
    key = (tag, dev.index if dev.index is not None else torch.cuda.current_device())
    if key not in _WS:
        _WS[key] = Workspace(dev)
    return _WS[key]


def _bits(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """fp16 tensors are passed by address; make sure they are contiguous fp16."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpi must be contiguous")
    return t


def predict(layer: dict, x: torch.Tensor, idx: Optional[torch.Tensor] = None,
            count: Optional[torch.Tensor] = None, act: str = "relu",
            tau: Optional[float] = None, n_hot: int = 0, stream=None):
    """idx (B x ffn int32) and count (B int32) for tokens x (B x d fp16).
    n_hot > 0: neurons [0, n_hot) of a hot-first layer are always listed and
    skip the predictor (pi_ffn_predict_hot)."""
    Bt, d = x.shape
    ffn, r = layer["ffn"], layer["r"]
    if idx is None:
        idx = torch.empty(Bt, ffn, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(Bt, dtype=torch.int32, device=x.device)
    nbytes = B.pi_workspace_size(B.PI_OP_PREDICT, Bt, d, r, ffn)
    ws, wsb = workspace("predict" if Bt == 1 else "predict_batch", x.device).get(nbytes)
    t = float(layer["tau"] if tau is None else tau)
    if n_hot:
        st = B.pi_ffn_predict_hot(_bits(x), Bt, d, layer["P1"], layer.get("b1"), B.ACTS[act], layer["P2"],
                                  layer.get("b2"), r, ffn, int(n_hot), t, idx, count, ws, wsb, stream)
        B.check(st, "pi_ffn_predict_hot")
    else:
        st = B.pi_ffn_predict(_bits(x), Bt, d, layer["P1"], layer.get("b1"), B.ACTS[act], layer["P2"],
                              layer.get("b2"), r, ffn, t, idx, count, ws, wsb, stream)
        B.check(st, "pi_ffn_predict")
    return idx, count


def sparse(layer: dict, x: torch.Tensor, idx: Optional[torch.Tensor],
           count: Optional[torch.Tensor], y: Optional[torch.Tensor] = None,
           dense: bool = False, per_token: bool = False, check_idx: bool = False,
           stream=None) -> torch.Tensor:
    """y (B x d fp32) from the active rows (or every row with dense=True).

    For B >= 2 the library reads the union of the tokens' rows once (matrix
    cores); per_token=True runs each token through the single-token kernels.
    check_idx=True has the device check each list afterwards and fill y_t with
    NaN where it breaks the contract (ids in [0, ffn), strictly ascending).
    """
    Bt, d = x.shape
    ffn = layer["ffn"]
    if y is None:
        y = torch.empty(Bt, d, dtype=torch.float32, device=x.device)
    nbytes = B.pi_workspace_size(B.PI_OP_SPARSE, Bt, d, layer.get("r", 8), ffn)
    tag = "sparse_dense" if dense else ("sparse" if Bt == 1 or per_token else "sparse_batch")
    ws, wsb = workspace(tag, x.device).get(nbytes)
    st = B.pi_ffn_sparse(B.KINDS[layer["kind"]], _bits(x), Bt, d, ffn, layer["W_up"],
                         layer.get("b_up"), layer.get("W_gate"), layer.get("b_gate"),
                         layer["W_down"], None if dense else idx, None if dense else count, y,
                         (B.PI_DENSE if dense else 0) | (B.PI_PER_TOKEN if per_token else 0)
                         | (B.PI_CHECK_IDX if check_idx else 0),
                         ws, wsb, stream)
    B.check(st, "pi_ffn_sparse")
    return y


def quantize_rows(W: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """INT4 codes (rows x d/2 uint8) and scales (rows x d/64 fp16) of fp16 rows W."""
    rows, d = W.shape
    q = torch.empty(rows, d // 2, dtype=torch.uint8, device=W.device)
    s = torch.empty(rows, d // 64, dtype=torch.float16, device=W.device)
    B.check(B.pi_quantize_rows(_bits(W), rows, d, q, s, stream), "pi_quantize_rows")
    return q, s


def quantize_layer(layer: dict, stream=None) -> dict:
    """The layer with W_up, W_gate, W_down and the predictor's P1, P2 as INT4
    rows (q_*, s_*); the biases are kept.  The predictor is quantised only
    when r is a multiple of 64 (the group); otherwise q_P1 .. s_P2 are None."""
    out = {k: v for k, v in layer.items() if k not in ("W_up", "W_gate", "W_down", "P1", "P2")}
    pred_ok = layer.get("P2") is not None and layer["P2"].shape[1] % 64 == 0
    for k, name in (("W_up", "up"), ("W_gate", "gate"), ("W_down", "down"), ("P1", "P1"), ("P2", "P2")):
        if layer.get(k) is not None and (pred_ok or k not in ("P1", "P2")):
            out["q_" + name], out["s_" + name] = quantize_rows(layer[k], stream)
        else:
            out["q_" + name], out["s_" + name] = None, None
    return out


def predict_q4(layer_q: dict, x: torch.Tensor, idx: Optional[torch.Tensor] = None,
               count: Optional[torch.Tensor] = None, act: str = "relu", tau: Optional[float] = None,
               n_hot: int = 0, stream=None):
    """pi_ffn_predict_q4 over a layer from quantize_layer: idx and count as predict()."""
    Bt, d = x.shape
    ffn, r = layer_q["ffn"], layer_q["r"]
    if idx is None:
        idx = torch.empty(Bt, ffn, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(Bt, dtype=torch.int32, device=x.device)
    nbytes = B.pi_workspace_size(B.PI_OP_PREDICT, Bt, d, r, ffn)
    ws, wsb = workspace("predict_q4", x.device).get(nbytes)
    t = float(layer_q["tau"] if tau is None else tau)
    st = B.pi_ffn_predict_q4(_bits(x), Bt, d, layer_q["q_P1"], layer_q["s_P1"], layer_q.get("b1"), B.ACTS[act],
                             layer_q["q_P2"], layer_q["s_P2"], layer_q.get("b2"), r, ffn, int(n_hot), t, idx,
                             count, ws, wsb, stream)
    B.check(st, "pi_ffn_predict_q4")
    return idx, count


def sparse_q4(layer_q: dict, x: torch.Tensor, idx: Optional[torch.Tensor], count: Optional[torch.Tensor],
              y: Optional[torch.Tensor] = None, dense: bool = False, stream=None) -> torch.Tensor:
    """pi_ffn_sparse_q4 over a layer from quantize_layer."""
    Bt, d = x.shape
    ffn = layer_q["ffn"]
    if y is None:
        y = torch.empty(Bt, d, dtype=torch.float32, device=x.device)
    nbytes = B.pi_workspace_size(B.PI_OP_SPARSE, Bt, d, layer_q.get("r", 8), ffn)
    ws, wsb = workspace("sparse_q4", x.device).get(nbytes)
    st = B.pi_ffn_sparse_q4(B.KINDS[layer_q["kind"]], _bits(x), Bt, d, ffn, layer_q["q_up"], layer_q["s_up"],
                            layer_q.get("b_up"), layer_q["q_gate"], layer_q["s_gate"], layer_q.get("b_gate"),
                            layer_q["q_down"], layer_q["s_down"], None if dense else idx,
                            None if dense else count, y, B.PI_DENSE if dense else 0, ws, wsb, stream)
    B.check(st, "pi_ffn_sparse_q4")
    return y


def decode(layer: dict, x: torch.Tensor, y: Optional[torch.Tensor] = None,
           idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
           act: str = "relu", tau: Optional[float] = None, per_token: bool = False,
           check_idx: bool = False, stream=None):
    """One decode step through pi_ffn_decode: the predicted list and the sparse
    FFN over it (one kernel for a single token).  Returns (y, idx, count)."""
    Bt, d = x.shape
    ffn, r = layer["ffn"], layer["r"]
    if y is None:
        y = torch.empty(Bt, d, dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty(Bt, ffn, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(Bt, dtype=torch.int32, device=x.device)
    nbytes = B.pi_workspace_size(B.PI_OP_DECODE, Bt, d, r, ffn)
    ws, wsb = workspace("decode", x.device).get(nbytes)
    st = B.pi_ffn_decode(B.KINDS[layer["kind"]], _bits(x), Bt, d, ffn, layer["P1"], layer.get("b1"),
                         B.ACTS[act], layer["P2"], layer.get("b2"), r,
                         float(layer["tau"] if tau is None else tau), layer["W_up"], layer.get("b_up"),
                         layer.get("W_gate"), layer.get("b_gate"), layer["W_down"], idx, count, y,
                         (B.PI_PER_TOKEN if per_token else 0) | (B.PI_CHECK_IDX if check_idx else 0),
                         ws, wsb, stream)
    B.check(st, "pi_ffn_decode")
    return y, idx, count


def decode_hot(layer: dict, x: torch.Tensor, n_hot: int, y: Optional[torch.Tensor] = None,
               idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
               act: str = "relu", tau: Optional[float] = None, per_token: bool = False,
               check_idx: bool = False, stream=None):
    """One decode step of a hot-first layer through pi_ffn_decode_hot: neurons
    [0, n_hot) always listed (their FFN computed beside the predictor for a
    single token), the rest predicted.  Returns (y, idx, count)."""
    Bt, d = x.shape
    ffn, r = layer["ffn"], layer["r"]
    if y is None:
        y = torch.empty(Bt, d, dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty(Bt, ffn, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(Bt, dtype=torch.int32, device=x.device)
    nbytes = B.pi_workspace_size(B.PI_OP_DECODE_HOT, Bt, d, r, ffn)
    ws, wsb = workspace("decode_hot" if Bt == 1 else "decode_hot_batch", x.device).get(nbytes)
    st = B.pi_ffn_decode_hot(B.KINDS[layer["kind"]], _bits(x), Bt, d, ffn, layer["P1"], layer.get("b1"),
                             B.ACTS[act], layer["P2"], layer.get("b2"), r, int(n_hot),
                             float(layer["tau"] if tau is None else tau), layer["W_up"], layer.get("b_up"),
                             layer.get("W_gate"), layer.get("b_gate"), layer["W_down"], idx, count, y,
                             (B.PI_PER_TOKEN if per_token else 0) | (B.PI_CHECK_IDX if check_idx else 0),
                             ws, wsb, stream)
    B.check(st, "pi_ffn_decode_hot")
    return y, idx, count


def hot_workspace(layer: dict, device=None) -> torch.Tensor:
    """A fresh zero-filled workspace for the single-token hot decode of this
    layer's shape (for callers that keep one per layer)."""
    nbytes = B.pi_workspace_size(B.PI_OP_DECODE_HOT, 1, layer["d"], layer["r"], layer["ffn"])
    return torch.zeros(nbytes, dtype=torch.uint8, device=device or layer["W_up"].device)


def decode_hot_begin(layer: dict, x: torch.Tensor, n_hot: int, idx: torch.Tensor, count: torch.Tensor,
                     ws: Optional[torch.Tensor] = None, act: str = "relu", tau: Optional[float] = None,
                     stream=None):
    """First launch of a single-token hot decode step (pi_ffn_decode_hot_begin):
    the list into idx / count and the hot prefix's FFN sum into the workspace."""
    d, ffn, r = layer["d"], layer["ffn"], layer["r"]
    if ws is None:
        ws, wsb = workspace("decode_hot", x.device).get(B.pi_workspace_size(B.PI_OP_DECODE_HOT, 1, d, r, ffn))
    else:
        wsb = ws.numel()
    st = B.pi_ffn_decode_hot_begin(B.KINDS[layer["kind"]], _bits(x), d, ffn, layer["P1"], layer.get("b1"), B.ACTS[act],
                                   layer["P2"], layer.get("b2"), r, int(n_hot),
                                   float(layer["tau"] if tau is None else tau), layer["W_up"], layer.get("b_up"),
                                   layer.get("W_gate"), layer.get("b_gate"), layer["W_down"], idx, count, ws, wsb,
                                   stream)
    B.check(st, "pi_ffn_decode_hot_begin")


def decode_hot_end(layer: dict, x: torch.Tensor, n_hot: int, idx: torch.Tensor, count: torch.Tensor,
                   y: torch.Tensor, ws: Optional[torch.Tensor] = None, check_idx: bool = False, stream=None):
    """Second launch (pi_ffn_decode_hot_end): the FFN over the list from n_hot on,
    plus the prefix's sum left by decode_hot_begin on the same workspace."""
    d, ffn, r = layer["d"], layer["ffn"], layer["r"]
    if ws is None:
        ws, wsb = workspace("decode_hot", x.device).get(B.pi_workspace_size(B.PI_OP_DECODE_HOT, 1, d, r, ffn))
    else:
        wsb = ws.numel()
    st = B.pi_ffn_decode_hot_end(B.KINDS[layer["kind"]], _bits(x), d, ffn, r, int(n_hot), layer["W_up"],
                                 layer.get("b_up"), layer.get("W_gate"), layer.get("b_gate"), layer["W_down"], idx,
                                 count, y, B.PI_CHECK_IDX if check_idx else 0, ws, wsb, stream)
    B.check(st, "pi_ffn_decode_hot_end")
    return y


def profile(X: torch.Tensor, W_fire: torch.Tensor, b_fire: Optional[torch.Tensor],
            counts: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    n, d = X.shape
    ffn = W_fire.shape[0]
    if counts is None:
        counts = torch.zeros(ffn, dtype=torch.int32, device=X.device)
    B.check(B.pi_profile(_bits(X), n, d, ffn, W_fire, b_fire, counts, None, 0, stream), "pi_profile")
    return counts


def reorder(counts_host, hot_share: float = 0.8):
    """Host plan: (perm int32 numpy new->old, hot_count)."""
    import numpy as np
    c = np.ascontiguousarray(np.asarray(counts_host, dtype=np.uint32))
    perm = np.empty(c.size, dtype=np.int32)
    hot = np.zeros(1, dtype=np.int32)
    B.check(B.pi_reorder(c, c.size, hot_share, perm, hot), "pi_reorder")
    return perm, int(hot[0])


def permute_rows(src: torch.Tensor, perm_dev: torch.Tensor, stream=None) -> torch.Tensor:
    dst = torch.empty_like(src)
    rows = src.shape[0]
    row_bytes = src[0].numel() * src.element_size() if src.dim() > 1 else src.element_size()
    B.check(B.pi_permute_rows(src, dst, rows, row_bytes, perm_dev, stream), "pi_permute_rows")
    return dst


ROW_KEYS = ("W_up", "W_gate", "W_down", "P2", "b_up", "b_gate", "b2")


def permute_layer(layer: dict, perm_dev: torch.Tensor, stream=None) -> dict:
    """Hot-first copy of a layer: every neuron-indexed tensor gathered by perm."""
    out = dict(layer)
    for k in ROW_KEYS:
        if layer.get(k) is not None:
            out[k] = permute_rows(layer[k], perm_dev, stream)
    return out


def to_device(layer: dict, device="cuda") -> dict:
    out = {}
    for k, v in layer.items():
        out[k] = v.to(device).contiguous() if isinstance(v, torch.Tensor) else v
    return out
