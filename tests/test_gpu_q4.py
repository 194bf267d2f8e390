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


def _oracle_q4_y_rows(H, x, lst):
    """The oracle's FFN over the dequantised INT4 rows of the listed neurons
    only (the quantiser works row by row, so a subset of rows quantises as in
    the whole matrix)."""
    rows = np.asarray(lst, dtype=np.int64)
    d = H["d"]

    def deq(k):
        return None if H.get(k) is None else O.dequantize_rows(*O.quantize_rows(H[k].numpy()[rows]), d)

    def sub(k):
        return None if H.get(k) is None else H[k].numpy()[rows]
    return O.sparse_ffn(H["kind"], x, deq("W_up"), sub("b_up"), deq("W_gate"), sub("b_gate"), deq("W_down"),
                        np.arange(rows.size))


@pytest.mark.parametrize("d,n", [(8256, 6143), (8256, 16000), (9216, 6145), (9216, 16000), (9216, 6143)])
def test_q4_fused_wide_rows_and_long_lists(d, n):
    """The fused single-token INT4 kernel where its loops take more than one
    round: d > 8192 (x staged in LDS in a second round) and lists longer than
    48 chunks x 128 rows, where each W_down row group takes several batches of
    16 rows in turn (the INT4 counterpart of the fp16 list-length test)."""
    cfg = custom_config("relu", d, 16384, 16, mean=0.3, number=102)
    L = make_layer(cfg, device=DEV)
    Q = R.quantize_layer(L)
    H = _host(L)
    del L
    x = make_tokens(cfg, 1, device=DEV)
    rng = np.random.default_rng(d + n)
    lst = np.sort(rng.choice(cfg.ffn, size=n, replace=False))
    idx = torch.zeros(1, cfg.ffn, dtype=torch.int32, device=DEV)
    idx[0, :n] = torch.from_numpy(lst.astype(np.int32)).to(DEV)
    cnt = torch.tensor([n], dtype=torch.int32, device=DEV)
    y = R.sparse_q4(Q, x, idx, cnt)
    torch.cuda.synchronize()
    check_y(y[0].cpu().numpy(), _oracle_q4_y_rows(H, x[0].cpu(), lst), where=f"q4 d={d} list len {n}")


# ---------------------------------------------------------------------------
# pi_ffn_predict_q4: the predictor over INT4 rows of P1 and P2.

def _deq(W):
    """The oracle's dequantised INT4 rows of an fp16 matrix (host)."""
    W = W.detach().cpu().numpy() if isinstance(W, torch.Tensor) else W
    return O.dequantize_rows(*O.quantize_rows(W), W.shape[1])


def _q4_logits(H, xh, act="relu"):
    return O.predictor_logits(xh, _deq(H["P1"]), H.get("b1"), act, _deq(H["P2"]), H["b2"])


@pytest.mark.parametrize("d,ffn,r,Bt", [(512, 1000, 64, 1), (576, 1000, 128, 3), (256, 300, 2048, 2),
                                        (8256, 100, 64, 1)])
def test_q4_predict_parity(d, ffn, r, Bt):
    """Ragged last tile (ffn % 32 != 0), the smallest r (two chunks a row),
    r = 2048 (two column batches per logits lane) and d > 8192 (x staged in
    two rounds)."""
    cfg = custom_config("relu", d, ffn, r, mean=0.2, number=110 + r)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, Bt).to(DEV)
    idx, cnt = R.predict_q4(Q, X)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    for t in range(Bt):
        c = int(cnt[t].cpu())
        assert 0 <= c <= ffn
        check_idx(idx[t, :c].cpu().numpy(), _q4_logits(H, X[t].cpu()), thr, where=f"q4 predict d={d} r={r} t={t}")


def test_q4_predict_bias_and_identity_act():
    """A hidden bias b1 and act = none (h = P1 x + b1, no ReLU)."""
    cfg = custom_config("relu", 512, 700, 128, mean=0.3, number=120)
    L = R.to_device(make_layer(cfg), DEV)
    L["b1"] = (torch.randn(cfg.r, generator=torch.Generator().manual_seed(7)) * 0.05).to(DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 2).to(DEV)
    thr = O.logit_threshold(L["tau"])
    for act in ("relu", "none"):
        idx, cnt = R.predict_q4(Q, X, act=act)
        torch.cuda.synchronize()
        for t in range(2):
            c = int(cnt[t].cpu())
            check_idx(idx[t, :c].cpu().numpy(), _q4_logits(H, X[t].cpu(), act), thr, where=f"q4 predict {act} t={t}")


def test_q4_predict_hot_prefix():
    """n_hot = 64: neurons [0, 64) always listed, the rest predicted."""
    cfg = custom_config("relu", 512, 1000, 64, mean=0.1, number=121)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 2).to(DEV)
    idx, cnt = R.predict_q4(Q, X, n_hot=64)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    for t in range(2):
        gi = idx[t, :int(cnt[t].cpu())].cpu().numpy()
        assert np.array_equal(gi[:64], np.arange(64))
        z = _q4_logits(H, X[t].cpu())
        check_idx(gi[64:] - 64, z[64:], thr, where=f"q4 predict hot t={t}")


@pytest.mark.parametrize("ffn,n_hot", [(1000, 160), (1000, 992), (1024, 1024), (40000, 0), (40000, 4096)])
def test_q4_predict_list_edges(ffn, n_hot):
    """The list the INT4 predictor's logits workgroups (four tiles each) write
    themselves after a look-back over the earlier workgroups' counts: a
    workgroup of prefix tiles only (n_hot 160), a workgroup whose last tile
    alone is predicted and ragged (992 of 1000), every tile in the prefix (no
    hidden rows, count = ffn), and 313 workgroups (more than one look-back
    round of 256), with and without 32 prefix workgroups."""
    cfg = custom_config("relu", 256, ffn, 64, mean=0.15, number=123)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 2).to(DEV)
    thr = O.logit_threshold(L["tau"])
    for rep in range(2):   # a second launch on the advanced epoch
        idx, cnt = R.predict_q4(Q, X, n_hot=n_hot)
        torch.cuda.synchronize()
        for t in range(2):
            c = int(cnt[t].cpu())
            assert n_hot <= c <= ffn, (ffn, n_hot, c)
            gi = idx[t, :c].cpu().numpy()
            assert np.array_equal(gi[:n_hot], np.arange(n_hot))
            if n_hot == ffn:
                assert c == ffn
                continue
            z = _q4_logits(H, X[t].cpu())
            check_idx(gi[n_hot:] - n_hot, z[n_hot:], thr, where=f"q4 list ffn={ffn} hot={n_hot} t={t} rep={rep}")


def test_full_size_q4_step():
    """The OPT-30B-shaped layer (d 7168, ffn 28672, r 1024) with every matrix
    as INT4 rows: the predicted list against the oracle's logits over the
    dequantised predictor, and y of the INT4 FFN over that list."""
    cfg = CONFIGS["c2"]
    L = make_layer(cfg, layer=0, device=DEV)
    H = _host(L)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 2, device=DEV, layer=0)
    thr = O.logit_threshold(L["tau"])
    for t in range(2):
        x = X[t:t + 1].contiguous()
        idx, cnt = R.predict_q4(Q, x)
        Y = R.sparse_q4(Q, x, idx, cnt)
        torch.cuda.synchronize()
        c = int(cnt[0].cpu())
        gi = idx[0, :c].cpu().numpy()
        check_idx(gi, _q4_logits(H, X[t].cpu()), thr, where=f"c2 q4 predict t={t}")
        check_y(Y[0].cpu().numpy(), _oracle_q4_y(H, X[t].cpu(), gi), where=f"c2 q4 step t={t}")


def test_q4_predict_graph_replay():
    """Captured once, replayed three times on new tokens: each replay's list
    matches the eager call (the epochs advance on the device)."""
    cfg = custom_config("relu", 512, 1000, 64, mean=0.2, number=122)
    L = R.to_device(make_layer(cfg), DEV)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 4).to(DEV)
    x = X[:1].clone()
    idx = torch.empty(1, cfg.ffn, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.predict_q4(Q, x, idx, cnt)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            R.predict_q4(Q, x, idx, cnt)
    torch.cuda.synchronize()
    for t in range(1, 4):
        x.copy_(X[t:t + 1])
        g.replay()
        torch.cuda.synchronize()
        gi, gc = idx.clone(), int(cnt.cpu())
        ei, ec = R.predict_q4(Q, X[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert gc == int(ec.cpu())
        assert torch.equal(gi[0, :gc], ei[0, :gc])
