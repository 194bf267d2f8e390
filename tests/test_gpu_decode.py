"""pi_ffn_decode: one call for the whole decode step (predictor, list, sparse
FFN).  Parity with the oracle (list: bit-exact outside the 1e-3 logit band;
y: the tolerances of tests.parity), bitwise equality with the two separate
calls, repeatability and graph replay, and workspace sharing with the other
operations."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from activation_sparse_predictor_amd import binding as B
from activation_sparse_predictor_amd import runtime as R
from synthetic import CONFIGS, custom_config, make_calibration, make_layer, make_tokens
from tests.parity import check_idx, check_y

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(layer):
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}


def _args(L, x, idx, cnt, y, ws, wsb, act=B.PI_ACT_RELU, flags=0):
    kind = B.KINDS[L["kind"]]
    return (kind, x, x.shape[0], L["d"], L["ffn"], L["P1"], L.get("b1"), act, L["P2"], L.get("b2"), L["r"],
            float(L["tau"]), L["W_up"], L.get("b_up"), L.get("W_gate"), L.get("b_gate"), L["W_down"], idx, cnt,
            y, flags, ws, wsb)


def _check_step(L, X, act="relu", where=""):
    """pi_ffn_decode one token at a time against the oracle and against the
    two-call path; returns the active counts."""
    H = _host(L)
    thr = O.logit_threshold(L["tau"])
    counts = []
    for t in range(X.shape[0]):
        x = X[t:t + 1].contiguous()
        y, idx, cnt = R.decode(L, x, act=act)
        idx2, cnt2 = R.predict(L, x, act=act)
        y2 = R.sparse(L, x, idx2, cnt2)
        torch.cuda.synchronize()
        c = int(cnt.cpu()[0])
        assert 0 <= c <= L["ffn"], f"{where} t={t}: count {c}"
        assert c == int(cnt2.cpu()[0]), f"{where} t={t}: count differs from pi_ffn_predict"
        gi = idx[0, :c].cpu().numpy()
        assert np.array_equal(gi, idx2[0, :c].cpu().numpy()), f"{where} t={t}: list differs from pi_ffn_predict"
        xh = X[t].cpu()
        z = O.predictor_logits(xh, H["P1"], H.get("b1"), act, H["P2"], H.get("b2"))
        check_idx(gi, z, thr, where=f"{where} t={t}")
        yo = O.sparse_ffn(H["kind"], xh, H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                          H["W_down"], gi)
        check_y(y[0].cpu().numpy(), yo, where=f"{where} t={t}")
        assert np.array_equal(y[0].cpu().numpy(), y2[0].cpu().numpy()), f"{where} t={t}: y differs from the two calls"
        counts.append(c)
    return counts


SHAPES = [
    ("relu", 64, 64, 8, 0.10),        # one column tile, one mask tile pair
    ("relu", 256, 1024, 64, 0.10),
    ("relu", 520, 1000, 72, 0.10),    # ragged: d % 512, ffn % 32, r % 64
    ("reglu", 520, 1000, 16, 0.20),
    ("reglu", 256, 1024, 64, 0.50),
    ("relu", 2048, 4160, 256, 0.05),
    ("relu", 1032, 2080, 136, 0.90),  # nearly every neuron active
    ("swiglu", 520, 1000, 72, 0.50),  # SiLU gate
]


@pytest.mark.parametrize("kind,d,ffn,r,mean", SHAPES)
def test_decode_step_parity(kind, d, ffn, r, mean):
    cfg = custom_config(kind, d, ffn, r, mean=mean, number=70 + d % 37)
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, 5).to(DEV)
    counts = _check_step(L, X, where=f"{kind} d{d} ffn{ffn} r{r}")
    assert sum(counts) > 0


@pytest.mark.parametrize("tau", [0.01, 0.5, 0.999999])
def test_decode_step_tau_extremes(tau):
    """tau near 0: nearly every neuron; tau near 1: few or none (count 0 gives y = 0)."""
    cfg = custom_config("relu", 520, 1000, 72, mean=0.2, number=71)
    L = R.to_device(make_layer(cfg), DEV)
    L["tau"] = tau
    _check_step(L, make_tokens(cfg, 3).to(DEV), where=f"tau={tau}")


def test_decode_step_empty_list():
    """b2 far below the threshold: no neuron is active, y must be exactly 0."""
    cfg = custom_config("reglu", 264, 2080, 136, mean=0.3, number=72)
    L = R.to_device(make_layer(cfg), DEV)
    L["b2"] = torch.full((cfg.ffn,), -1e4, dtype=torch.float32, device=DEV)
    y, idx, cnt = R.decode(L, make_tokens(cfg, 1).to(DEV))
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0
    assert torch.count_nonzero(y).item() == 0


def test_decode_step_linear_predictor():
    cfg = custom_config("relu", 520, 1000, 72, number=73)
    L = R.to_device(make_layer(cfg), DEV)
    L["b1"] = torch.linspace(-0.5, 0.5, 72, device=DEV, dtype=torch.float32)
    _check_step(L, make_tokens(cfg, 2).to(DEV), act="none", where="act=none")


def test_decode_step_repeatable_and_check_flag():
    cfg = custom_config("reglu", 1032, 2080, 136, mean=0.3, number=74)
    L = R.to_device(make_layer(cfg), DEV)
    x = make_tokens(cfg, 1).to(DEV)
    outs = []
    for rep in range(3):
        y, idx, cnt = R.decode(L, x, check_idx=(rep == 2))
        torch.cuda.synchronize()
        c = int(cnt.item())
        outs.append((c, idx[0, :c].cpu().numpy().copy(), y.cpu().numpy().copy()))
    for c, i, y in outs[1:]:
        assert c == outs[0][0] and np.array_equal(i, outs[0][1]) and np.array_equal(y, outs[0][2])


@pytest.mark.parametrize("kind", ["relu", "reglu", "swiglu"])
def test_decode_step_graph_replay(kind):
    """pi_ffn_decode for three tokens captured in a HIP graph and replayed
    several times, with eager decode steps on the same workspace between the
    replays: every replay equals the eager result bitwise."""
    cfg = custom_config(kind, 520, 1000, 72, mean=0.2, number=75)
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, 6).to(DEV)
    ffn, d = L["ffn"], L["d"]
    wsb = B.pi_workspace_size(B.PI_OP_DECODE, 1, d, L["r"], ffn)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    bufs = [(torch.empty(1, ffn, dtype=torch.int32, device=DEV), torch.empty(1, dtype=torch.int32, device=DEV),
             torch.empty(1, d, dtype=torch.float32, device=DEV)) for _ in range(3)]

    def run(t, b):
        B.check(B.pi_ffn_decode(*_args(L, X[t:t + 1], b[0], b[1], b[2], ws, wsb)), "decode")

    for t in range(3):
        run(t, bufs[t])
    torch.cuda.synchronize()
    ref = [(int(b[1].item()), b[0][0, :int(b[1].item())].cpu().clone(), b[2].cpu().clone()) for b in bufs]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for t in range(3):
                run(t, bufs[t])
    torch.cuda.synchronize()
    scratch = (torch.empty(1, ffn, dtype=torch.int32, device=DEV), torch.empty(1, dtype=torch.int32, device=DEV),
               torch.empty(1, d, dtype=torch.float32, device=DEV))
    for rep in range(4):
        for b in bufs:
            b[1].fill_(-7)
            b[2].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t, b in enumerate(bufs):
            c = int(b[1].item())
            assert c == ref[t][0], f"replay {rep} token {t}: count {c} vs {ref[t][0]}"
            assert torch.equal(b[0][0, :c].cpu(), ref[t][1]), f"replay {rep} token {t}: idx differs"
            assert torch.equal(b[2].cpu(), ref[t][2]), f"replay {rep} token {t}: y differs"
        run(3 + rep % 3, scratch)
        torch.cuda.synchronize()
    H = _host(L)
    for t in range(3):
        yo = O.sparse_ffn(H["kind"], X[t].cpu(), H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                          H["W_down"], ref[t][1].numpy())
        check_y(ref[t][2][0].numpy(), yo, where=f"graph t={t}")


def test_decode_step_shares_a_workspace():
    """One workspace for decode, predict and sparse calls (single token and a
    batch) in turn: each call finds another layout than it left."""
    cfg = custom_config("relu", 520, 1000, 72, mean=0.2, number=76)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, 4).to(DEV)
    ffn, d = L["ffn"], L["d"]
    wsb = max(B.pi_workspace_size(op, Bt, d, L["r"], ffn)
              for op in (B.PI_OP_PREDICT, B.PI_OP_SPARSE, B.PI_OP_DECODE) for Bt in (1, 4))
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    thr = O.logit_threshold(L["tau"])
    for rnd in range(3):
        for Bt in (1, 4, 1):
            x = X[:Bt].contiguous()
            idx = torch.empty(Bt, ffn, dtype=torch.int32, device=DEV)
            cnt = torch.empty(Bt, dtype=torch.int32, device=DEV)
            y = torch.empty(Bt, d, dtype=torch.float32, device=DEV)
            if rnd == 1:   # the two calls, on the same workspace
                kind = B.PI_FFN_RELU
                B.check(B.pi_ffn_predict(x, Bt, d, L["P1"], None, B.PI_ACT_RELU, L["P2"], L["b2"], L["r"], ffn,
                                         float(L["tau"]), idx, cnt, ws, wsb), "predict")
                B.check(B.pi_ffn_sparse(kind, x, Bt, d, ffn, L["W_up"], L.get("b_up"), None, None, L["W_down"],
                                        idx, cnt, y, 0, ws, wsb), "sparse")
            else:
                B.check(B.pi_ffn_decode(*_args(L, x, idx, cnt, y, ws, wsb)), "decode")
            torch.cuda.synchronize()
            for t in range(Bt):
                c = int(cnt[t].item())
                gi = idx[t, :c].cpu().numpy()
                xh = X[t].cpu()
                z = O.predictor_logits(xh, H["P1"], None, "relu", H["P2"], H["b2"])
                where = f"round {rnd} B={Bt} t={t}"
                check_idx(gi, z, thr, where=where)
                yo = O.sparse_ffn("relu", xh, H["W_up"], H.get("b_up"), None, None, H["W_down"], gi)
                check_y(y[t].cpu().numpy(), yo, where=where)


def test_decode_dense_flag_rejected():
    cfg = custom_config("relu", 64, 64, 8, number=77)
    L = R.to_device(make_layer(cfg), DEV)
    x = make_tokens(cfg, 1).to(DEV)
    idx = torch.empty(1, 64, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    y = torch.empty(1, 64, dtype=torch.float32, device=DEV)
    wsb = B.pi_workspace_size(B.PI_OP_DECODE, 1, 64, 8, 64)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    assert B.pi_ffn_decode(*_args(L, x, idx, cnt, y, ws, wsb, flags=B.PI_DENSE)) == B.PI_ERR_INVALID_ARG


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_decode_step_hot_first_layer(kind):
    """A hot-first reordered layer: the active neurons crowd into the first
    logits tiles, so a few tiles append most of the up workers' queue."""
    cfg = custom_config(kind, 1032, 4160, 136, mean=0.15, exponent=1.3, number=95)
    L = R.to_device(make_layer(cfg), DEV)
    Xc = make_calibration(cfg, 512).to(DEV)
    Wf = L["W_up"] if kind == "relu" else L["W_gate"]
    bf = L["b_up"] if kind == "relu" else L["b_gate"]
    counts = R.profile(Xc, Wf, bf).cpu().numpy()
    perm, _ = R.reorder(counts, 0.8)
    P = R.permute_layer(L, torch.from_numpy(perm).to(DEV))
    X = make_tokens(cfg, 4).to(DEV)
    got = _check_step(P, X, where=f"hot-first {kind}")
    # most of each list sits in the first quarter of the neurons
    idx, cnt = R.predict(P, X[:1].contiguous())
    c = int(cnt.cpu()[0])
    assert sum(got) > 0 and np.mean(idx[0, :c].cpu().numpy() < cfg.ffn // 4) > 0.5


@pytest.mark.parametrize("key", ["c2", "c3"])
def test_full_size_decode_step(key):
    cfg = CONFIGS[key]
    L = make_layer(cfg, layer=0, device=DEV)
    X = make_tokens(cfg, 3, device=DEV, layer=0)
    counts = _check_step(L, X, where=f"{key} decode step")
    frac = np.mean(counts) / cfg.ffn
    assert 0.5 * cfg.mean < frac < 1.6 * cfg.mean, frac


@pytest.mark.parametrize("kind,Bt", [("relu", 6), ("reglu", 20)])
def test_decode_step_batched(kind, Bt):
    """B >= 2: the batched predictor and the union path, bitwise those of the
    two calls, and within the oracle's tolerances per token."""
    cfg = custom_config(kind, 520, 1000, 72, mean=0.2, number=78 + Bt)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, Bt).to(DEV)
    y, idx, cnt = R.decode(L, X)
    idx2, cnt2 = R.predict(L, X)
    y2 = R.sparse(L, X, idx2, cnt2)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2)
    thr = O.logit_threshold(L["tau"])
    for t in range(Bt):
        c = int(cnt[t].item())
        gi = idx[t, :c].cpu().numpy()
        assert np.array_equal(gi, idx2[t, :c].cpu().numpy()), f"t={t}: list differs"
        assert torch.equal(y[t], y2[t]), f"t={t}: y differs from the two calls"
        xh = X[t].cpu()
        z = O.predictor_logits(xh, H["P1"], H.get("b1"), "relu", H["P2"], H.get("b2"))
        check_idx(gi, z, thr, where=f"batched t={t}")
        yo = O.sparse_ffn(H["kind"], xh, H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                          H["W_down"], gi)
        check_y(y[t].cpu().numpy(), yo, where=f"batched t={t}")


def test_decode_step_alternating_shapes_one_workspace():
    """Decode steps of three shapes in turn on one zero-filled workspace (the
    largest size asked for): the header stays where it is whatever the shape,
    so the single-token kernels' counters and epochs stay valid, and each data
    area is cleared when it finds another layout."""
    cfgs = [custom_config("relu", 1032, 2080, 136, mean=0.9, number=90),
            custom_config("relu", 64, 64, 8, mean=0.1, number=91),
            custom_config("reglu", 520, 1000, 72, mean=0.3, number=92)]
    Ls = [R.to_device(make_layer(c), DEV) for c in cfgs]
    Xs = [make_tokens(c, 2).to(DEV) for c in cfgs]
    wsb = max(B.pi_workspace_size(B.PI_OP_DECODE, 1, L["d"], L["r"], L["ffn"]) for L in Ls)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    for rnd, order in enumerate(([1, 0, 2], [0, 2, 1], [2, 1, 0])):
        for li in order:
            L, X = Ls[li], Xs[li]
            H = _host(L)
            ffn, d = L["ffn"], L["d"]
            for t in range(X.shape[0]):
                x = X[t:t + 1].contiguous()
                idx = torch.empty(1, ffn, dtype=torch.int32, device=DEV)
                cnt = torch.empty(1, dtype=torch.int32, device=DEV)
                y = torch.full((1, d), float("nan"), dtype=torch.float32, device=DEV)
                B.check(B.pi_ffn_decode(*_args(L, x, idx, cnt, y, ws, wsb)), "decode")
                torch.cuda.synchronize()
                c = int(cnt.item())
                gi = idx[0, :c].cpu().numpy()
                xh = X[t].cpu()
                where = f"round {rnd} shape {li} t={t}"
                z = O.predictor_logits(xh, H["P1"], H.get("b1"), "relu", H["P2"], H.get("b2"))
                check_idx(gi, z, O.logit_threshold(L["tau"]), where=where)
                yo = O.sparse_ffn(H["kind"], xh, H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                                  H["W_down"], gi)
                check_y(y[0].cpu().numpy(), yo, where=where)
