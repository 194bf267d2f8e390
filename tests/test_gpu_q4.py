"""INT4 neuron rows on the GPU: pi_quantize_rows bit-exact against the
oracle's quantiser, and pi_ffn_sparse_q4 against the oracle's FFN over the
weights the oracle itself dequantises (y within the parity tolerances)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from activation_sparse_predictor_amd import runtime as R
from synthetic import CONFIGS, custom_config, make_layer, make_tokens
from tests.parity import check_idx, check_y

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(layer):
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}


@pytest.mark.parametrize("rows,d", [(5, 64), (37, 512), (300, 7168)])
def test_quantize_rows_bit_exact(rows, d):
    rng = np.random.default_rng(rows + d)
    W = (rng.standard_normal((rows, d)) * np.exp(rng.standard_normal((rows, 1)) * 2)).astype(np.float16)
    W[0, :64] = 0                       # a zero group
    W[1 % rows, 64 % d:] *= np.float16(1e-4)   # tiny weights (fp16 subnormal scales)
    q, s = R.quantize_rows(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    oq, osc = O.quantize_rows(W)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), osc.view(np.uint16))


def _oracle_q4_y(H, x, idx):
    d = H["d"]
    deq = {k: (None if H.get(k) is None else O.dequantize_rows(*O.quantize_rows(H[k].numpy()), d))
           for k in ("W_up", "W_gate", "W_down")}
    return O.sparse_ffn(H["kind"], x, deq["W_up"], H.get("b_up"), deq["W_gate"], H.get("b_gate"), deq["W_down"], idx)


@pytest.mark.parametrize("kind", ["relu", "reglu", "swiglu"])
@pytest.mark.parametrize("Bt", [1, 3])
def test_q4_ffn_parity(kind, Bt):
    cfg = custom_config(kind, 512, 1000, 64, mean=0.2, number=99)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, Bt).to(DEV)
    idx, cnt = R.predict(L, X)
    Y = R.sparse_q4(Q, X, idx, cnt)
    Yd = R.sparse_q4(Q, X, None, None, dense=True)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    for t in range(Bt):
        c = int(cnt[t].cpu())
        gi = idx[t, :c].cpu().numpy()
        xh = X[t].cpu()
        z = O.predictor_logits(xh, H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(gi, z, thr, where=f"q4 {kind} t={t}")
        check_y(Y[t].cpu().numpy(), _oracle_q4_y(H, xh, gi), where=f"q4 {kind} B={Bt} t={t}")
        check_y(Yd[t].cpu().numpy(), _oracle_q4_y(H, xh, np.arange(cfg.ffn)), where=f"q4 dense {kind} t={t}")


def test_q4_ffn_empty_list_is_zero():
    cfg = custom_config("relu", 256, 512, 16, mean=0.1, number=100)
    L = R.to_device(make_layer(cfg), DEV)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 2).to(DEV)
    idx = torch.zeros(2, cfg.ffn, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(2, dtype=torch.int32, device=DEV)
    Y = R.sparse_q4(Q, X, idx, cnt)
    torch.cuda.synchronize()
    assert not torch.any(Y)


def test_full_size_q4():
    cfg = CONFIGS["c2"]
    L = make_layer(cfg, layer=0, device=DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 1, device=DEV, layer=0)
    idx, cnt = R.predict(L, X)
    Y = R.sparse_q4(Q, X, idx, cnt)
    torch.cuda.synchronize()
    c = int(cnt[0].cpu())
    gi = idx[0, :c].cpu().numpy()
    check_y(Y[0].cpu().numpy(), _oracle_q4_y(H, X[0].cpu(), gi), where="c2 q4")


def test_q4_single_token_edges():
    """The fused single-token INT4 kernel: an empty list gives exactly 0, a
    one-neuron list and a ragged width (d = 576: a partial 512-column tile)
    match the oracle."""
    cfg = custom_config("reglu", 576, 1000, 64, mean=0.2, number=101)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 2).to(DEV)
    x = X[:1].contiguous()
    idx = torch.zeros(1, cfg.ffn, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    y0 = R.sparse_q4(Q, x, idx, cnt)
    idx[0, 0] = cfg.ffn - 1
    cnt.fill_(1)
    y1 = R.sparse_q4(Q, x, idx, cnt)
    i2, c2 = R.predict(L, X[1:2].contiguous())
    y2 = R.sparse_q4(Q, X[1:2].contiguous(), i2, c2)
    torch.cuda.synchronize()
    assert not torch.any(y0)
    check_y(y1[0].cpu().numpy(), _oracle_q4_y(H, X[0].cpu(), [cfg.ffn - 1]), where="q4 one neuron")
    gi = i2[0, :int(c2[0].cpu())].cpu().numpy()
    check_y(y2[0].cpu().numpy(), _oracle_q4_y(H, X[1].cpu(), gi), where="q4 d=576")
