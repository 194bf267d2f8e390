"""pi_ffn_decode_hot on the GPU: a decode step on a hot-first layer whose
always-listed prefix has its FFN computed beside the predictor (single token).

The list and count must be bitwise those of pi_ffn_predict_hot (the extra
roles do not touch the prediction); y must meet the parity bar against the
oracle's FFN over that list (tests/parity.py); repeated calls and graph
replays are bitwise equal; several tokens are pi_ffn_predict_hot followed by
pi_ffn_sparse, bitwise.
"""

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


def _hot_first(cfg, L, ncal, layer=0):
    Xc = make_calibration(cfg, ncal, device=DEV, layer=layer)
    Wf = L["W_up"] if cfg.kind == "relu" else L["W_gate"]
    bf = L["b_up"] if cfg.kind == "relu" else L["b_gate"]
    counts = R.profile(Xc, Wf, bf).cpu().numpy()
    perm, _ = R.reorder(counts, 0.8)
    return R.permute_layer(L, torch.from_numpy(perm).to(DEV)), counts[perm]


def _check_step(P, x, n_hot, where, H=None):
    """One decode_hot step against predict_hot (list, bitwise) and the oracle (y)."""
    H = H or _host(P)
    y, idx, cnt = R.decode_hot(P, x, n_hot)
    i1, c1 = R.predict(P, x, n_hot=n_hot)
    torch.cuda.synchronize()
    c = int(cnt.cpu()[0])
    assert c == int(c1.cpu()[0]), f"{where}: count {c} vs pi_ffn_predict_hot {int(c1.cpu()[0])}"
    gi = idx[0, :c].cpu().numpy()
    assert np.array_equal(gi, i1[0, :c].cpu().numpy()), f"{where}: list differs from pi_ffn_predict_hot"
    assert np.array_equal(gi[:n_hot], np.arange(n_hot)), f"{where}: prefix not listed"
    xh = x[0].cpu()
    _, z = O.predict_hot(xh, H["P1"], H.get("b1"), "relu", H["P2"], H["b2"], P["tau"], n_hot)
    check_idx(gi, z, O.logit_threshold(P["tau"]), where=where)
    ref = O.sparse_ffn(H["kind"], xh, H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"), H["W_down"], gi)
    check_y(y[0].cpu().numpy(), ref, where=where)
    return y, c


@pytest.mark.parametrize("kind,n_hot", [("relu", 0), ("relu", 32), ("relu", 256), ("reglu", 64), ("reglu", 1024),
                                        ("swiglu", 128), ("relu", 2080), ("relu", 2048)])
def test_decode_hot_small(kind, n_hot):
    """d = 520 (a partial second 512-column tile), ffn = 2080; n_hot = 2080 is
    every neuron (no hidden rows, every tile in the prefix), 2048 needs more
    than 24 chunks of 64 rows (each hot W_down wave takes two batches)."""
    cfg = custom_config(kind, 520, 2080, 72, mean=0.2, exponent=1.3, number=120)
    L = R.to_device(make_layer(cfg), DEV)
    P, _ = _hot_first(cfg, L, 512)
    X = make_tokens(cfg, 3).to(DEV)
    H = _host(P)
    for t in range(3):
        _check_step(P, X[t:t + 1].contiguous(), n_hot, where=f"decode_hot {kind} n_hot={n_hot} t={t}", H=H)


def test_decode_hot_zero_prefix_equals_decode():
    """n_hot = 0: no extra roles, the same kernels as pi_ffn_decode: bitwise."""
    cfg = custom_config("reglu", 1032, 2080, 136, mean=0.2, number=121)
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, 2).to(DEV)
    for t in range(2):
        x = X[t:t + 1].contiguous()
        y0, i0, c0 = R.decode(L, x)
        y1, i1, c1 = R.decode_hot(L, x, 0)
        torch.cuda.synchronize()
        assert torch.equal(c0, c1) and torch.equal(i0[0, :int(c0[0])], i1[0, :int(c1[0])])
        assert torch.equal(y0, y1)


def test_decode_hot_repeatable_and_shapes_alternating():
    """Repeated calls are bitwise equal; calls alternating between two layer
    shapes and prefixes on the one runtime workspace stay correct (the library
    clears the tagged words when the layout changes; the hot epoch slots
    advance with the launches)."""
    c1 = custom_config("relu", 520, 2080, 72, mean=0.2, exponent=1.3, number=122)
    c2 = custom_config("relu", 2048, 4160, 256, mean=0.1, exponent=1.2, number=123)
    P1, _ = _hot_first(c1, R.to_device(make_layer(c1), DEV), 256)
    P2, _ = _hot_first(c2, R.to_device(make_layer(c2), DEV), 256)
    x1 = make_tokens(c1, 1).to(DEV)
    x2 = make_tokens(c2, 1).to(DEV)
    H1, H2 = _host(P1), _host(P2)
    first = {}
    for rep in range(3):
        for P, x, nh, H, key in ((P1, x1, 64, H1, "a"), (P2, x2, 512, H2, "b"), (P1, x1, 96, H1, "c")):
            y, _ = _check_step(P, x, nh, where=f"alternating {key} rep {rep}", H=H)
            if rep == 0:
                first[key] = y.clone()
            else:
                assert torch.equal(y, first[key]), f"{key}: repeat {rep} not bitwise equal"


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_decode_hot_graph_replay(kind):
    """A graph of decode_hot steps over several tokens, replayed four times with
    eager calls on the same workspace between replays: every replay bitwise
    equal to the eager results (the hot roles' epochs advance per launch)."""
    cfg = custom_config(kind, 520, 2080, 72, mean=0.2, exponent=1.3, number=124)
    P, _ = _hot_first(cfg, R.to_device(make_layer(cfg), DEV), 512)
    n_hot = 128
    X = make_tokens(cfg, 4).to(DEV)
    xs = [X[t:t + 1].contiguous() for t in range(4)]
    ys = [torch.empty(1, cfg.d, dtype=torch.float32, device=DEV) for _ in range(4)]
    idx = [torch.empty(1, cfg.ffn, dtype=torch.int32, device=DEV) for _ in range(4)]
    cnt = [torch.empty(1, dtype=torch.int32, device=DEV) for _ in range(4)]

    def run():
        for t in range(4):
            R.decode_hot(P, xs[t], n_hot, ys[t], idx[t], cnt[t])

    run()
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t in range(4):
            assert torch.equal(ys[t], ref[t]), f"replay {rep} token {t} differs"
        run()   # eager calls between replays
        torch.cuda.synchronize()
    H = _host(P)
    for t in range(4):
        c = int(cnt[t].cpu()[0])
        gi = idx[t][0, :c].cpu().numpy()
        r = O.sparse_ffn(H["kind"], xs[t][0].cpu(), H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                         H["W_down"], gi)
        check_y(ref[t][0].cpu().numpy(), r, where=f"graph {kind} t={t}")


def test_decode_hot_batched_is_predict_hot_then_sparse():
    cfg = custom_config("relu", 520, 2080, 72, mean=0.2, exponent=1.3, number=125)
    P, _ = _hot_first(cfg, R.to_device(make_layer(cfg), DEV), 512)
    X = make_tokens(cfg, 5).to(DEV)
    y, idx, cnt = R.decode_hot(P, X, 96)
    i1, c1 = R.predict(P, X, n_hot=96)
    y1 = R.sparse(P, X, i1, c1)
    torch.cuda.synchronize()
    assert torch.equal(cnt, c1)
    for t in range(5):
        c = int(cnt[t])
        assert torch.equal(idx[t, :c], i1[t, :c])
    assert torch.equal(y, y1)


def test_decode_hot_check_idx_flag():
    """PI_CHECK_IDX on a valid list leaves y unchanged."""
    cfg = custom_config("relu", 520, 2080, 72, mean=0.2, exponent=1.3, number=126)
    P, _ = _hot_first(cfg, R.to_device(make_layer(cfg), DEV), 256)
    x = make_tokens(cfg, 1).to(DEV)
    y0, _, _ = R.decode_hot(P, x, 64)
    y1, _, _ = R.decode_hot(P, x, 64, check_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("key,layer", [("c5", 0), ("c5", 41), ("c2", 0)])
def test_full_size_decode_hot(key, layer):
    """Hot-first layers of the OPT-66B-shaped stack (d 9216: x staged in two
    rounds by the hot up rows) and the OPT-30B-shaped layer, profiled on 4096
    calibration tokens; the prefix is the neurons that fired on >= 99 % of them."""
    cfg = CONFIGS[key]
    L = make_layer(cfg, layer=layer, device=DEV)
    P, pc = _hot_first(cfg, L, cfg.calib_tokens, layer=layer)
    del L
    n_hot = 32 * (int(np.count_nonzero(pc >= 0.99 * cfg.calib_tokens)) // 32)
    assert n_hot >= 512, n_hot
    X = make_tokens(cfg, 2, device=DEV, layer=layer)
    H = _host(P)
    for t in range(2):
        _check_step(P, X[t:t + 1].contiguous(), n_hot, where=f"{key} layer {layer} hot t={t}", H=H)


def test_decode_hot_begin_end_equal_one_call():
    """begin then end on one workspace (the runtime's, and one per layer) is
    bitwise the one-call result, for two layers interleaved by phase."""
    cfg = custom_config("reglu", 1032, 2080, 136, mean=0.2, exponent=1.3, number=127)
    Ps = [_hot_first(cfg, R.to_device(make_layer(cfg, layer=l), DEV), 256, layer=l)[0] for l in range(2)]
    X = make_tokens(cfg, 2).to(DEV)
    xs = [X[l:l + 1].contiguous() for l in range(2)]
    ref = [R.decode_hot(Ps[l], xs[l], 160)[0].clone() for l in range(2)]
    wss = [R.hot_workspace(Ps[l]) for l in range(2)]
    idx = [torch.empty(1, cfg.ffn, dtype=torch.int32, device=DEV) for _ in range(2)]
    cnt = [torch.empty(1, dtype=torch.int32, device=DEV) for _ in range(2)]
    ys = [torch.empty(1, cfg.d, dtype=torch.float32, device=DEV) for _ in range(2)]
    for rep in range(2):
        for l in range(2):
            R.decode_hot_begin(Ps[l], xs[l], 160, idx[l], cnt[l], ws=wss[l])
        for l in range(2):
            R.decode_hot_end(Ps[l], xs[l], 160, idx[l], cnt[l], ys[l], ws=wss[l])
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(ys[l], ref[l]), f"rep {rep} layer {l}"
    R.decode_hot_begin(Ps[0], xs[0], 160, idx[0], cnt[0])
    y = R.decode_hot_end(Ps[0], xs[0], 160, idx[0], cnt[0], ys[0])
    torch.cuda.synchronize()
    assert torch.equal(y, ref[0])

