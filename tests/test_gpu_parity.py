"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small ragged shapes span several tiles plus a tail on every axis (d vs the
512-column W_down tiles and 1024-element row steps, ffn vs the 32-neuron
logits tiles, r vs the 64-lane chunk columns).  Full-size layers are
checked on sampled tokens.  Rules (tests/parity.py): index lists bit-exact
outside a 1e-3 band around the logit threshold; y within rel-L2 1e-3 and
max-abs 2e-3 * ||y||_inf of the oracle evaluated on the GPU's own list.
"""

import numpy as np
import pytest
import torch

import oracle as O
from activation_sparse_predictor_amd import binding as B
from activation_sparse_predictor_amd import runtime as R
from synthetic import CONFIGS, custom_config, make_calibration, make_layer, make_tokens
from tests.parity import check_counts, check_idx, check_y

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(layer):
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}


def _oracle_y(H, x, idx):
    return O.sparse_ffn(H["kind"], x, H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                        H["W_down"], idx)


def _check_tokens(L, X, act="relu", where=""):
    """Predict + sparse one token at a time; full parity per token. Returns active counts."""
    H = _host(L)
    thr = O.logit_threshold(L["tau"])
    counts = []
    for t in range(X.shape[0]):
        x = X[t:t + 1].contiguous()
        idx, cnt = R.predict(L, x, act=act)
        y = R.sparse(L, x, idx, cnt)
        torch.cuda.synchronize()
        c = int(cnt.cpu()[0])
        assert 0 <= c <= L["ffn"], f"{where} t={t}: count {c}"
        gi = idx[0, :c].cpu().numpy()
        xh = X[t].cpu()
        z = O.predictor_logits(xh, H["P1"], H.get("b1"), act, H["P2"], H.get("b2"))
        check_idx(gi, z, thr, where=f"{where} t={t}")
        check_y(y[0].cpu().numpy(), _oracle_y(H, xh, gi), where=f"{where} t={t}")
        counts.append(c)
    return counts


SHAPES = [
    ("relu", 64, 64, 8, 0.10),
    ("relu", 256, 1024, 64, 0.10),
    ("relu", 520, 1000, 72, 0.10),
    ("relu", 1032, 2080, 136, 0.30),
    ("reglu", 520, 1000, 16, 0.20),
    ("reglu", 256, 1024, 64, 0.50),
    ("relu", 2048, 4160, 256, 0.05),
    ("swiglu", 520, 1000, 72, 0.50),     # SiLU gate: about half the neurons listed
    ("swiglu", 2048, 4160, 256, 0.30),
]


@pytest.mark.parametrize("kind,d,ffn,r,mean", SHAPES)
def test_decode_parity_small(kind, d, ffn, r, mean):
    cfg = custom_config(kind, d, ffn, r, mean=mean, number=40 + d % 37)
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, 6).to(DEV)
    counts = _check_tokens(L, X, where=f"{kind} d{d} ffn{ffn} r{r}")
    assert sum(counts) > 0


def test_decode_parity_tiny_config():
    cfg = CONFIGS["c1"]
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, cfg.tokens).to(DEV)
    counts = _check_tokens(L, X, where="c1")
    assert 0.03 * cfg.ffn < np.mean(counts) < 0.3 * cfg.ffn


@pytest.mark.parametrize("tau", [0.01, 0.3, 0.5, 0.99])
def test_tau_values(tau):
    cfg = custom_config("relu", 256, 1024, 64, mean=0.2, number=51)
    L = R.to_device(make_layer(cfg), DEV)
    L["tau"] = tau
    _check_tokens(L, make_tokens(cfg, 3).to(DEV), where=f"tau={tau}")


def test_linear_predictor_and_hidden_bias():
    cfg = custom_config("relu", 520, 1000, 72, number=52)
    L = R.to_device(make_layer(cfg), DEV)
    L["b1"] = torch.linspace(-0.5, 0.5, 72, device=DEV, dtype=torch.float32)
    X = make_tokens(cfg, 3).to(DEV)
    _check_tokens(L, X, act="none", where="act=none")
    _check_tokens(L, X, act="relu", where="act=relu b1")


def test_zero_token():
    cfg = custom_config("reglu", 256, 1000, 64, mean=0.3, number=53)
    L = R.to_device(make_layer(cfg), DEV)
    X = torch.zeros(1, 256, dtype=torch.float16, device=DEV)
    _check_tokens(L, X, where="x=0")


def _sparse_with(L, x, idx_list):
    ffn = L["ffn"]
    idx = torch.zeros(1, ffn, dtype=torch.int32, device=DEV)
    if len(idx_list):
        idx[0, :len(idx_list)] = torch.tensor(idx_list, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([len(idx_list)], dtype=torch.int32, device=DEV)
    y = R.sparse(L, x, idx, cnt)
    torch.cuda.synchronize()
    return y[0].cpu().numpy()


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_sparse_edge_lists(kind):
    cfg = custom_config(kind, 1032, 1000, 16, mean=0.3, number=54)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    x = make_tokens(cfg, 1).to(DEV)
    xh = x[0].cpu()
    y = _sparse_with(L, x, [])
    assert np.all(y == 0.0), "empty list must give exactly 0"
    for lst in ([cfg.ffn - 1], [0], list(range(cfg.ffn)), list(range(0, cfg.ffn, 7)),
                list(range(cfg.ffn - 9, cfg.ffn))):
        check_y(_sparse_with(L, x, lst), _oracle_y(H, xh, lst), where=f"{kind} list len {len(lst)}")


@pytest.mark.parametrize("n", [127, 128, 129, 6143, 6144, 6145, 16000])
def test_sparse_list_lengths_around_chunking(n):
    """The single-token FFN uses ceil(n / 128) list chunks per column tile (at
    most 48): lengths at the chunk-count steps, and past 48 x 128 where each
    row group takes several batches of 16 rows in turn."""
    cfg = custom_config("relu", 520, 16384, 16, mean=0.3, number=59)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    x = make_tokens(cfg, 1).to(DEV)
    rng = np.random.default_rng(n)
    lst = np.sort(rng.choice(cfg.ffn, size=n, replace=False)).tolist()
    check_y(_sparse_with(L, x, lst), _oracle_y(H, x[0].cpu(), lst), where=f"list len {n}")


@pytest.mark.parametrize("kind", ["relu", "reglu", "swiglu"])
def test_dense_flag(kind):
    cfg = custom_config(kind, 520, 2080, 16, number=55)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, 3).to(DEV)
    Y = R.sparse(L, X, None, None, dense=True)
    torch.cuda.synchronize()
    for t in range(3):
        xh = X[t].cpu()
        ref = O.dense_ffn(kind, xh, H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"), H["W_down"])
        check_y(Y[t].cpu().numpy(), ref, where=f"dense t={t}")


@pytest.mark.parametrize("kind,Bt", [("relu", 1), ("relu", 2), ("relu", 4), ("relu", 9), ("relu", 15),
                                     ("relu", 16), ("relu", 17), ("relu", 32), ("relu", 33), ("reglu", 8),
                                     ("reglu", 12), ("reglu", 20), ("reglu", 32), ("reglu", 64), ("relu", 65),
                                     ("relu", 100), ("reglu", 128), ("relu", 131), ("swiglu", 4),
                                     ("swiglu", 20), ("swiglu", 64), ("swiglu", 128)])
def test_batched_union_path(kind, Bt):
    """Batch of Bt tokens.  The batched predictor (matrix cores) must satisfy the
    index rule per token, and agree with the single-token predictor except
    inside the threshold band; y of the union path matches the oracle on each
    token's own list; the per-token sparse path is bitwise equal to a
    single-token call on the same list."""
    cfg = custom_config(kind, 520, 1000, 72, mean=0.15, number=56)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, Bt).to(DEV)
    idx, cnt = R.predict(L, X)
    Y = R.sparse(L, X, idx, cnt)
    Yp = R.sparse(L, X, idx, cnt, per_token=True)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    cnt_h, idx_h, Y_h, Yp_h = cnt.cpu().numpy(), idx.cpu().numpy(), Y.cpu().numpy(), Yp.cpu().numpy()
    for t in sorted(set([0, Bt // 2, Bt - 1] + list(range(0, Bt, max(1, Bt // 8))))):
        x1 = X[t:t + 1].contiguous()
        c = int(cnt_h[t])
        mine = idx_h[t, :c]
        i1, c1 = R.predict(L, x1)
        one = torch.from_numpy(idx_h[t:t + 1].copy()).to(DEV)
        y1 = R.sparse(L, x1, one, cnt[t:t + 1].clone())
        torch.cuda.synchronize()
        xh = X[t].cpu()
        z = O.predictor_logits(xh, H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(mine, z, thr, where=f"batched predict B={Bt} t={t}")
        single = i1[0, :int(c1.cpu()[0])].cpu().numpy()
        diff = set(mine.tolist()) ^ set(single.tolist())
        assert all(abs(z[j] - thr) <= 1e-3 for j in diff), f"B={Bt} t={t}: lists differ outside the band"
        assert np.array_equal(Yp_h[t], y1[0].cpu().numpy()), "per-token path differs from single token"
        ref = _oracle_y(H, xh, mine)
        check_y(Y_h[t], ref, where=f"union B={Bt} t={t}")
        check_y(Yp_h[t], ref, where=f"per-token B={Bt} t={t}")


@pytest.mark.parametrize("kind,ffn", [("relu", 24576), ("relu", 24448), ("reglu", 24576)])
def test_union_whole_row_block_threshold(kind, ffn):
    """128 tokens whose union is every neuron: 192 row blocks of 128 (3/4 of
    the 256 resident up-GEMM workgroups: one whole row block each) and 191
    (below the threshold: the even split with pieces and last arrivers), with
    a ragged K (d = 520).  y of sampled tokens against the oracle."""
    cfg = custom_config(kind, 520, ffn, 32, mean=0.7, exponent=0.3, number=66)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, 128).to(DEV)
    idx, cnt = R.predict(L, X)
    Y = R.sparse(L, X, idx, cnt)
    torch.cuda.synchronize()
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    union = np.zeros(ffn, dtype=bool)
    for t in range(128):
        union[idx_h[t, :cnt_h[t]]] = True
    assert union.all(), f"union {union.sum()} of {ffn}: the row-block count this test needs is not reached"
    for t in (0, 77, 127):
        mine = idx_h[t, :cnt_h[t]]
        check_y(Y[t].cpu().numpy(), _oracle_y(H, X[t].cpu(), mine), where=f"{kind} ffn={ffn} t={t}")


@pytest.mark.parametrize("Bt,d", [(3, 520), (5, 520), (3, 8200), (7, 9216), (6, 9224), (8, 16384)])
def test_batched_predictor_hidden_paths(Bt, d):
    """Groups of up to 8 tokens take the hidden layer on the vector units when
    their x fits in LDS (B <= 4: d <= 16384; B <= 8: d <= 9216), else on the
    matrix cores: padding tokens, rows longer than 8192, both sides of the
    size limit.  The index rule per token against the oracle, and agreement
    with the single-token predictor outside the threshold band."""
    cfg = custom_config("relu", d, 1000, 72, mean=0.15, number=58)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, Bt).to(DEV)
    idx, cnt = R.predict(L, X)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    for t in range(Bt):
        c = int(cnt[t].item())
        mine = idx[t, :c].cpu().numpy()
        z = O.predictor_logits(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(mine, z, thr, where=f"B={Bt} d={d} t={t}")
        i1, c1 = R.predict(L, X[t:t + 1].contiguous())
        torch.cuda.synchronize()
        single = i1[0, :int(c1.item())].cpu().numpy()
        diff = set(mine.tolist()) ^ set(single.tolist())
        assert all(abs(z[j] - thr) <= 1e-3 for j in diff), f"B={Bt} d={d} t={t}: lists differ outside the band"


@pytest.mark.parametrize("r,Bt,n_hot", [(256, 33, 0), (512, 64, 0), (1024, 100, 0), (1024, 128, 64),
                                         (256, 131, 32), (1024, 40, 992), (512, 96, 960)])
def test_batched_logits_h_in_registers(r, Bt, n_hot):
    """More than 32 tokens with r = 256, 512 or 1024 take the logits kernel
    that holds h in registers (32-token groups, whole 32-row blocks of P2, no
    K split).  ffn = 1000 leaves a partial last 32-row block; the hot prefix
    shifts the rows (n_hot = 992: one partial block left).  The
    index rule per token against the oracle, and agreement with the
    single-token predictor outside the threshold band."""
    cfg = custom_config("relu", 264, 1000, r, mean=0.15, number=64)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    X = make_tokens(cfg, Bt).to(DEV)
    idx, cnt = R.predict(L, X, n_hot=n_hot)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    for t in sorted(set([0, 31, 32, Bt - 1] + list(range(0, Bt, 7)))):
        c = int(cnt_h[t])
        mine = idx_h[t, :c]
        _, z = O.predict_hot(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"], L["tau"], n_hot)
        check_idx(mine, z, thr, where=f"r={r} B={Bt} n_hot={n_hot} t={t}")
        assert np.array_equal(mine[:n_hot], np.arange(n_hot)), "prefix not listed"
        i1, c1 = R.predict(L, X[t:t + 1].contiguous(), n_hot=n_hot)
        torch.cuda.synchronize()
        single = i1[0, :int(c1.cpu()[0])].cpu().numpy()
        diff = set(mine.tolist()) ^ set(single.tolist())
        assert all(abs(z[j] - thr) <= 1e-3 for j in diff), f"r={r} B={Bt} t={t}: lists differ outside the band"


def test_union_path_edge_lists():
    """Empty lists, disjoint lists, identical lists, one full list, a list whose
    32-neuron words run across the 64-entry waves that build the token
    bitmaps, and one with a long gap, in one batch."""
    cfg = custom_config("reglu", 1032, 1000, 16, mean=0.3, number=60)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    ffn = cfg.ffn
    lists = [[], list(range(0, ffn, 2)), list(range(1, ffn, 2)), list(range(0, ffn, 2)), list(range(ffn)), [ffn - 1],
             list(range(0, 41)) + list(range(100, 300)) + list(range(500, 503)), [3, 600, 601, ffn - 2]]
    Bt = len(lists)
    X = make_tokens(cfg, Bt).to(DEV)
    idx = torch.zeros(Bt, ffn, dtype=torch.int32, device=DEV)
    for t, l in enumerate(lists):
        if l:
            idx[t, :len(l)] = torch.tensor(l, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([len(l) for l in lists], dtype=torch.int32, device=DEV)
    Y = R.sparse(L, X, idx, cnt)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    assert np.all(Yh[0] == 0.0)
    for t in range(1, Bt):
        check_y(Yh[t], _oracle_y(H, X[t].cpu(), lists[t]), where=f"edge list t={t}")


def test_union_bitmap_runs_across_waves():
    """The token bitmaps are built 64 list entries a wave; a 32-neuron word's
    run that crosses a wave's end is completed from the (at most 31) entries
    after it.  Lists whose run there goes on for 31 entries (the most), for 1,
    for none (a word boundary at the wave's end), one that ends inside those
    31, and dense lists long enough that every wave takes several rounds."""
    cfg = custom_config("relu", 1032, 1000, 16, mean=0.3, number=63)
    L = R.to_device(make_layer(cfg), DEV)
    H = _host(L)
    ffn = cfg.ffn
    lists = [list(range(1, ffn)),                              # entry 63 = neuron 64: 31 more of word 2
             list(range(31, ffn)),                             # entry 63 = neuron 94: 1 more of word 2
             list(range(32, ffn)),                             # entry 63 = neuron 95: word 2 ends there
             list(range(0, 63)) + list(range(96, 128)) + list(range(700, 990, 3)),
             list(range(0, 63)) + list(range(96, 110)),        # the list ends inside the run
             list(range(5, 69)) + list(range(70, 80))]         # a run of word 2 split 5 / 10 by the wave's end
    Bt = len(lists)
    X = make_tokens(cfg, Bt).to(DEV)
    idx = torch.zeros(Bt, ffn, dtype=torch.int32, device=DEV)
    for t, l in enumerate(lists):
        idx[t, :len(l)] = torch.tensor(l, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([len(l) for l in lists], dtype=torch.int32, device=DEV)
    Y = R.sparse(L, X, idx, cnt)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    for t in range(Bt):
        check_y(Yh[t], _oracle_y(H, X[t].cpu(), lists[t]), where=f"run list t={t}")


@pytest.mark.parametrize("per_token", [False, True])
def test_check_idx_flag(per_token):
    """PI_CHECK_IDX: tokens whose lists break the contract (an id out of range,
    out of order, repeated, a count above ffn or below 0) get y = NaN; valid
    tokens are bitwise equal to the call without the flag.  The batched path
    (per_token=False) and the single-token kernel (per_token=True) both."""
    cfg = custom_config("relu", 264, 600, 16, mean=0.2, number=62)
    L = R.to_device(make_layer(cfg), DEV)
    ffn = cfg.ffn
    good = [list(range(3, ffn, 7)), [], [0, ffn - 1]]
    bad = [[5, ffn, 9], [1, 8, 4], [2, 2, 3], [-1, 4]]
    lists = good + bad
    Bt = len(lists)
    X = make_tokens(cfg, Bt).to(DEV)
    idx = torch.zeros(Bt, ffn, dtype=torch.int32, device=DEV)
    for t, l in enumerate(lists):
        if l:
            idx[t, :len(l)] = torch.tensor(l, dtype=torch.int32, device=DEV)
    counts = [len(l) for l in lists]
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    cnt_over = cnt.clone()
    cnt_over[1] = ffn + 1     # a count above ffn on an otherwise empty list
    cnt_neg = cnt.clone()
    cnt_neg[1] = -3
    Y0 = R.sparse(L, X, idx, cnt, per_token=per_token).cpu().numpy()
    Y1 = R.sparse(L, X, idx, cnt, per_token=per_token, check_idx=True).cpu().numpy()
    Y2 = R.sparse(L, X, idx, cnt_over, per_token=per_token, check_idx=True).cpu().numpy()
    Y3 = R.sparse(L, X, idx, cnt_neg, per_token=per_token, check_idx=True).cpu().numpy()
    for t in range(len(good)):
        assert np.array_equal(Y1[t], Y0[t]), f"valid token {t} changed by the check"
    for t in range(len(good), Bt):
        assert np.all(np.isnan(Y1[t])), f"broken list {t} not flagged"
    assert np.all(np.isnan(Y2[1])) and np.all(np.isnan(Y3[1])), "count outside [0, ffn] not flagged"
    assert np.array_equal(Y2[0], Y0[0]) and np.array_equal(Y3[2], Y0[2])


def test_negative_count_gives_nan():
    """count = -1 is the predictor's report of an overrun wait.  Without
    PI_CHECK_IDX every FFN path answers it with y_t = NaN (the single-token
    kernel, PI_PER_TOKEN, the union path, both INT4 paths), while the other
    tokens of the call keep the results they get when that token's list is
    empty (bitwise: the union, and so its chunking, is then the same)."""
    cfg = custom_config("relu", 520, 1000, 64, mean=0.2, number=64)
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, 3).to(DEV)
    idx, cnt = R.predict(L, X)
    bad, empty = cnt.clone(), cnt.clone()
    bad[1], empty[1] = -1, 0
    for Bt, per_token in ((1, False), (3, True), (3, False)):
        c_ok, c_bad = empty[:Bt].contiguous(), bad[:Bt].contiguous()
        if Bt == 1:
            c_bad = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        Y0 = R.sparse(L, X[:Bt].contiguous(), idx[:Bt].contiguous(), c_ok, per_token=per_token).cpu().numpy()
        Y1 = R.sparse(L, X[:Bt].contiguous(), idx[:Bt].contiguous(), c_bad, per_token=per_token).cpu().numpy()
        nan_t = 0 if Bt == 1 else 1
        assert np.all(np.isnan(Y1[nan_t])), f"B={Bt} per_token={per_token}: count -1 did not give NaN"
        for t in range(Bt):
            if t != nan_t:
                assert np.array_equal(Y1[t], Y0[t]), f"B={Bt} per_token={per_token}: token {t} changed"


def test_negative_count_gives_nan_q4():
    cfg = custom_config("reglu", 512, 1000, 64, mean=0.2, number=65)
    L = R.to_device(make_layer(cfg), DEV)
    Q = R.quantize_layer(L)
    X = make_tokens(cfg, 3).to(DEV)
    idx, cnt = R.predict(L, X)
    bad, empty = cnt.clone(), cnt.clone()
    bad[1], empty[1] = -1, 0
    for Bt in (1, 3):
        c_ok = empty[:Bt].contiguous()
        c_bad = bad[:Bt].contiguous() if Bt > 1 else torch.full((1,), -1, dtype=torch.int32, device=DEV)
        Y0 = R.sparse_q4(Q, X[:Bt].contiguous(), idx[:Bt].contiguous(), c_ok).cpu().numpy()
        Y1 = R.sparse_q4(Q, X[:Bt].contiguous(), idx[:Bt].contiguous(), c_bad).cpu().numpy()
        nan_t = 0 if Bt == 1 else 1
        assert np.all(np.isnan(Y1[nan_t])), f"INT4 B={Bt}: count -1 did not give NaN"
        for t in range(Bt):
            if t != nan_t:
                assert np.array_equal(Y1[t], Y0[t]), f"INT4 B={Bt}: token {t} changed"


def test_deterministic_repeats():
    cfg = custom_config("reglu", 1032, 2080, 136, mean=0.3, number=57)
    L = R.to_device(make_layer(cfg), DEV)
    x = make_tokens(cfg, 1).to(DEV)
    outs = []
    for _ in range(3):
        idx, cnt = R.predict(L, x)
        y = R.sparse(L, x, idx, cnt)
        torch.cuda.synchronize()
        c = int(cnt.cpu()[0])
        outs.append((c, idx[0, :c].cpu().numpy().copy(), y.cpu().numpy().copy()))
    for c, i, y in outs[1:]:
        assert c == outs[0][0] and np.array_equal(i, outs[0][1]) and np.array_equal(y, outs[0][2])


def _decode_args(L, x, idx, cnt, y, ws, ws_bytes):
    kind = B.KINDS[L["kind"]]
    p = (x, x.shape[0], L["d"], L["P1"], L.get("b1"), B.PI_ACT_RELU, L["P2"], L.get("b2"), L["r"], L["ffn"],
         float(L["tau"]), idx, cnt, ws, ws_bytes)
    q = (kind, x, x.shape[0], L["d"], L["ffn"], L["W_up"], L.get("b_up"), L.get("W_gate"), L.get("b_gate"),
         L["W_down"], idx, cnt, y, 0, ws, ws_bytes)
    return p, q


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_graph_replay(kind):
    """Single-token predict + sparse captured in a HIP graph and replayed several
    times, with eager calls on the same workspaces (other tokens) between the
    replays: every replay must equal the eager result bitwise (the kernels take
    their launch epoch from the workspace, not from the captured arguments)."""
    cfg = custom_config(kind, 520, 1000, 72, mean=0.2, number=60)
    L = R.to_device(make_layer(cfg), DEV)
    X = make_tokens(cfg, 6).to(DEV)
    ffn, d = L["ffn"], L["d"]
    wsb = max(B.pi_workspace_size(B.PI_OP_PREDICT, 1, d, L["r"], ffn),
              B.pi_workspace_size(B.PI_OP_SPARSE, 1, d, L["r"], ffn))
    ws_p = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    ws_s = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    bufs = [(torch.empty(1, ffn, dtype=torch.int32, device=DEV), torch.empty(1, dtype=torch.int32, device=DEV),
             torch.empty(1, d, dtype=torch.float32, device=DEV)) for _ in range(3)]

    def run(t, b):
        p, _ = _decode_args(L, X[t:t + 1], b[0], b[1], b[2], ws_p, wsb)
        _, q = _decode_args(L, X[t:t + 1], b[0], b[1], b[2], ws_s, wsb)
        B.check(B.pi_ffn_predict(*p), "predict")
        B.check(B.pi_ffn_sparse(*q), "sparse")

    for t in range(3):   # eager reference (also settles the workspaces' layouts)
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
        run(3 + rep % 3, scratch)   # eager work on the same workspaces between replays
        torch.cuda.synchronize()
    H = _host(L)
    for t in range(3):
        check_y(ref[t][2][0].numpy(), _oracle_y(H, X[t].cpu(), ref[t][1].numpy()), where=f"graph t={t}")


def test_one_workspace_for_everything():
    """One zero-filled workspace shared by every operation and two shapes, in
    an order that makes each single-token call find a different layout than it
    left: results must match the oracle throughout."""
    cfgs = [custom_config("relu", 520, 1000, 72, mean=0.2, number=61),
            custom_config("reglu", 264, 2080, 136, mean=0.3, number=62)]
    Ls = [R.to_device(make_layer(c), DEV) for c in cfgs]
    Xs = [make_tokens(c, 5).to(DEV) for c in cfgs]
    wsb = 0
    for L in Ls:
        for op in (B.PI_OP_PREDICT, B.PI_OP_SPARSE):
            for Bt in (1, 5):
                wsb = max(wsb, B.pi_workspace_size(op, Bt, L["d"], L["r"], L["ffn"]))
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    thr = O.logit_threshold(0.5)
    for rnd in range(3):
        for li, (L, X) in enumerate(zip(Ls, Xs)):
            H = _host(L)
            ffn, d = L["ffn"], L["d"]
            for Bt in ((1, 5) if rnd % 2 == 0 else (5, 1)):
                x = X[:Bt].contiguous()
                idx = torch.empty(Bt, ffn, dtype=torch.int32, device=DEV)
                cnt = torch.empty(Bt, dtype=torch.int32, device=DEV)
                y = torch.empty(Bt, d, dtype=torch.float32, device=DEV)
                p, q = _decode_args(L, x, idx, cnt, y, ws, wsb)
                B.check(B.pi_ffn_predict(*p), "predict")
                B.check(B.pi_ffn_sparse(*q), "sparse")
                torch.cuda.synchronize()
                for t in range(Bt):
                    c = int(cnt[t].item())
                    gi = idx[t, :c].cpu().numpy()
                    xh = X[t].cpu()
                    z = O.predictor_logits(xh, H["P1"], None, "relu", H["P2"], H["b2"])
                    where = f"round {rnd} layer {li} B={Bt} t={t}"
                    check_idx(gi, z, thr, where=where)
                    check_y(y[t].cpu().numpy(), _oracle_y(H, xh, gi), where=where)


@pytest.mark.parametrize("kind,d,ffn,n", [("relu", 64, 96, 40), ("relu", 520, 1000, 300),
                                          ("reglu", 256, 1024, 129), ("relu", 1032, 2080, 1024)])
def test_profile_parity(kind, d, ffn, n):
    cfg = custom_config(kind, d, ffn, 8, mean=0.2, number=58)
    L = R.to_device(make_layer(cfg, predictor=False), DEV)
    Xc = make_calibration(cfg, n).to(DEV)
    Wf = L["W_up"] if kind == "relu" else L["W_gate"]
    bf = L["b_up"] if kind == "relu" else L["b_gate"]
    counts = R.profile(Xc, Wf, bf)
    torch.cuda.synchronize()
    pre = O.profile_preactivations(Xc.cpu(), Wf.cpu(), bf.cpu())
    check_counts(counts.cpu().numpy(), pre, where=f"profile {kind} d{d} ffn{ffn} n{n}")
    # counts accumulate across calls
    R.profile(Xc, Wf, bf, counts)
    torch.cuda.synchronize()
    lo, hi = (pre > 1e-3).sum(0), (pre > -1e-3).sum(0)
    c2 = counts.cpu().numpy().astype(np.int64)
    assert np.all((c2 >= 2 * lo) & (c2 <= 2 * hi))


@pytest.mark.parametrize("rows,cols,dtype", [(1000, 520, torch.float16), (4160, 1, torch.float32),
                                              (7, 3, torch.float32), (64, 4096, torch.float16)])
def test_permute_rows_bit_exact(rows, cols, dtype):
    g = torch.Generator(device="cpu").manual_seed(rows)
    src = torch.randn(rows, cols, generator=g).to(dtype).to(DEV)
    if cols == 1:
        src = src[:, 0].contiguous()
    perm = torch.randperm(rows, generator=g).to(torch.int32)
    out = R.permute_rows(src, perm.to(DEV))
    ident = R.permute_rows(src, torch.arange(rows, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    want = O.permute_rows(src.cpu().numpy(), perm.numpy())
    assert np.array_equal(out.cpu().numpy(), want)
    assert torch.equal(ident, src)


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_profile_reorder_invariance(kind):
    """Profile -> host plan -> permuted layer: the same y, and idx' = sort(perm^-1[idx])."""
    cfg = custom_config(kind, 520, 2080, 72, mean=0.15, exponent=1.3, number=59)
    L = R.to_device(make_layer(cfg), DEV)
    Xc = make_calibration(cfg, 512).to(DEV)
    Wf = L["W_up"] if kind == "relu" else L["W_gate"]
    bf = L["b_up"] if kind == "relu" else L["b_gate"]
    counts = R.profile(Xc, Wf, bf).cpu().numpy()
    perm, hot = R.reorder(counts, 0.8)
    operm, ohot = O.reorder_plan(counts.astype(np.int64), 0.8)
    assert np.array_equal(perm, operm) and hot == ohot
    P = R.permute_layer(L, torch.from_numpy(perm).to(DEV))
    inv = np.argsort(perm)
    H = _host(L)
    thr = O.logit_threshold(L["tau"])
    X = make_tokens(cfg, 4).to(DEV)
    for t in range(4):
        x = X[t:t + 1].contiguous()
        i0, c0 = R.predict(L, x)
        i1, c1 = R.predict(P, x)
        y0 = R.sparse(L, x, i0, c0)
        y1 = R.sparse(P, x, i1, c1)
        torch.cuda.synchronize()
        a0 = i0[0, :int(c0.cpu()[0])].cpu().numpy()
        a1 = i1[0, :int(c1.cpu()[0])].cpu().numpy()
        z = O.predictor_logits(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"])
        diff = set(a1.tolist()) ^ set(inv[a0].tolist())
        assert all(abs(z[perm[j]] - thr) <= 1e-3 for j in diff)
        check_y(y1[0].cpu().numpy(), _oracle_y(H, X[t].cpu(), np.sort(perm[a1])), where=f"reordered t={t}")
    # hot prefix holds the most active neurons
    pc = counts[perm]
    assert np.all(np.diff(pc.astype(np.int64)) <= 0)


# ---------------------------------------------------------------- full-size layers
def _full(key, layer=0, ntok=3):
    cfg = CONFIGS[key]
    L = make_layer(cfg, layer=layer, device=DEV)
    X = make_tokens(cfg, ntok, device=DEV, layer=layer)
    return cfg, L, X


def test_union_down_id_windows():
    """A union larger than one LDS window of ids per down chunk (d = 8192 gives
    8 chunks per column tile, so |U| = 40960 means 5120 entries per chunk: the
    down GEMM reloads its ids mid-chunk).  Lists: token t takes every neuron
    i with (i + t) % 3 != 0, so the union is every neuron."""
    cfg = custom_config("relu", 8192, 40960, 64, mean=0.1, number=63)
    L = make_layer(cfg, device=DEV)
    H = _host(L)
    Bt, ffn = 6, cfg.ffn
    X = make_tokens(cfg, Bt, device=DEV)
    lists = [[i for i in range(ffn) if (i + t) % 3 != 0] for t in range(Bt)]
    idx = torch.zeros(Bt, ffn, dtype=torch.int32, device=DEV)
    for t, l in enumerate(lists):
        idx[t, :len(l)] = torch.tensor(l, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([len(l) for l in lists], dtype=torch.int32, device=DEV)
    Y = R.sparse(L, X, idx, cnt).cpu().numpy()
    for t in (0, Bt - 1):
        check_y(Y[t], _oracle_y(H, X[t].cpu(), lists[t]), where=f"union windows t={t}")


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c3s"])
def test_full_size_decode(key):
    cfg, L, X = _full(key)
    counts = _check_tokens(L, X, where=key)
    frac = np.mean(counts) / cfg.ffn
    assert 0.5 * cfg.mean < frac < 1.6 * cfg.mean, frac


def test_full_size_stack_layer_and_profile():
    """One sampled layer of the 64-layer stack shape, plus its profile on 256 calibration tokens."""
    cfg, L, X = _full("c5", layer=17, ntok=2)
    _check_tokens(L, X, where="c5 layer 17")
    Xc = make_calibration(cfg, 256, device=DEV, layer=17)
    counts = R.profile(Xc, L["W_up"], L["b_up"])
    torch.cuda.synchronize()
    pre = O.profile_preactivations(Xc.cpu(), L["W_up"].cpu(), L["b_up"].cpu())
    check_counts(counts.cpu().numpy(), pre, where="c5 profile")


@pytest.mark.parametrize("Bt", [4, 16, 32, 64, 128])
def test_full_size_batched(Bt):
    cfg, L, X = _full("c4", ntok=Bt)
    H = _host(L)
    idx, cnt = R.predict(L, X)
    Y = R.sparse(L, X, idx, cnt)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    for t in (0, Bt - 1):
        c = int(cnt[t].cpu())
        gi = idx[t, :c].cpu().numpy()
        z = O.predictor_logits(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(gi, z, thr, where=f"c4 B={Bt} t={t}")
        check_y(Y[t].cpu().numpy(), _oracle_y(H, X[t].cpu(), gi), where=f"c4 B={Bt} t={t}")


def test_full_size_swiglu_batched():
    """The LLaMA2-70B-shaped SiLU-gated layer through the union path (16 tokens,
    about half the neurons each, so the union covers nearly every row)."""
    cfg, L, X = _full("c3s", ntok=16)
    H = _host(L)
    idx, cnt = R.predict(L, X)
    Y = R.sparse(L, X, idx, cnt)
    torch.cuda.synchronize()
    thr = O.logit_threshold(L["tau"])
    for t in (0, 15):
        c = int(cnt[t].cpu())
        gi = idx[t, :c].cpu().numpy()
        z = O.predictor_logits(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(gi, z, thr, where=f"c3s B=16 t={t}")
        check_y(Y[t].cpu().numpy(), _oracle_y(H, X[t].cpu(), gi), where=f"c3s B=16 t={t}")


# ---------------------------------------------------------------- hot prefix (pi_ffn_predict_hot)
def _hot_first(cfg, L, ncal):
    """Profile on calibration tokens, plan the hot-first order, permute the layer;
    returns the permuted layer and its counts in the new order."""
    Xc = make_calibration(cfg, ncal).to(DEV)
    Wf = L["W_up"] if cfg.kind == "relu" else L["W_gate"]
    bf = L["b_up"] if cfg.kind == "relu" else L["b_gate"]
    counts = R.profile(Xc, Wf, bf).cpu().numpy()
    perm, _ = R.reorder(counts, 0.8)
    return R.permute_layer(L, torch.from_numpy(perm).to(DEV)), counts[perm]


def _check_hot(P, X, n_hot, where):
    H = _host(P)
    thr = O.logit_threshold(P["tau"])
    idx, cnt = R.predict(P, X, n_hot=n_hot)
    Y = R.sparse(P, X, idx, cnt)
    torch.cuda.synchronize()
    for t in sorted({0, X.shape[0] // 2, X.shape[0] - 1}):
        c = int(cnt[t].cpu())
        gi = idx[t, :c].cpu().numpy()
        assert np.array_equal(gi[:n_hot], np.arange(n_hot)), f"{where} t={t}: hot prefix not listed"
        _, z = O.predict_hot(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"], P["tau"], n_hot)
        check_idx(gi, z, thr, where=f"{where} t={t}")
        check_y(Y[t].cpu().numpy(), _oracle_y(H, X[t].cpu(), gi), where=f"{where} t={t}")


@pytest.mark.parametrize("kind,Bt,n_hot", [("relu", 1, 64), ("reglu", 1, 256), ("relu", 4, 96),
                                           ("relu", 20, 64), ("swiglu", 16, 128), ("relu", 1, 2048)])
def test_hot_prefix(kind, Bt, n_hot):
    """Neurons [0, n_hot) of a hot-first layer are listed for every token without
    the predictor; the others follow the oracle's prediction from rows n_hot.."""
    cfg = custom_config(kind, 520, 2080, 72, mean=0.2, exponent=1.3, number=97)
    L = R.to_device(make_layer(cfg), DEV)
    P, _ = _hot_first(cfg, L, 512)
    X = make_tokens(cfg, Bt).to(DEV)
    _check_hot(P, X, n_hot, where=f"hot {kind} B={Bt} n_hot={n_hot}")


@pytest.mark.parametrize("ffn,n_hot", [(8192, 0), (8224, 0), (9000, 64), (16416, 96), (24608, 7200)])
def test_compaction_rounds(ffn, n_hot):
    """The single-token compaction goes through the tiles past the prefix in
    rounds of 256: exactly one round (256 tiles), a one-tile last round (257),
    a ragged last tile (9000 = 281 x 32 + 8), a prefix that shifts the rounds
    and leaves a ragged last round (513 tiles from tile 3), and a long prefix
    (tile 225 of 769) on a hot-first layer."""
    cfg = custom_config("relu", 64, ffn, 16, mean=0.15, exponent=1.3, number=131)
    L = R.to_device(make_layer(cfg), DEV)
    P = _hot_first(cfg, L, 256)[0] if n_hot >= 1024 else L
    _check_hot(P, make_tokens(cfg, 1).to(DEV), n_hot, where=f"compaction ffn={ffn} n_hot={n_hot}")
    # pi_ffn_decode_hot's predictor launch (the same compaction, with the prefix's FFN beside it)
    x = make_tokens(cfg, 2).to(DEV)[1:2].contiguous()
    y, i1, c1 = R.decode_hot(P, x, n_hot)
    i0, c0 = R.predict(P, x, n_hot=n_hot)
    torch.cuda.synchronize()
    c = int(c0.cpu()[0])
    assert int(c1.cpu()[0]) == c and torch.equal(i1[0, :c], i0[0, :c])


def test_hot_prefix_zero_and_whole():
    """n_hot = 0 is pi_ffn_predict (bitwise); n_hot = ffn lists every neuron."""
    cfg = custom_config("relu", 256, 1024, 64, mean=0.1, number=98)
    L = R.to_device(make_layer(cfg), DEV)
    for Bt in (1, 5):
        X = make_tokens(cfg, Bt).to(DEV)
        i0, c0 = R.predict(L, X)
        ws = torch.zeros(B.pi_workspace_size(B.PI_OP_PREDICT, Bt, 256, 64, 1024), dtype=torch.uint8, device=DEV)
        i1 = torch.empty_like(i0)
        c1 = torch.empty_like(c0)
        B.check(B.pi_ffn_predict_hot(X, Bt, 256, L["P1"], None, B.PI_ACT_RELU, L["P2"], L["b2"], 64, 1024, 0,
                                     float(L["tau"]), i1, c1, ws, ws.numel()), "predict_hot 0")
        i2, c2 = R.predict(L, X, n_hot=1024)
        torch.cuda.synchronize()
        assert torch.equal(c0, c1)
        for t in range(Bt):
            c = int(c0[t])
            assert torch.equal(i0[t, :c], i1[t, :c])
            assert int(c2[t]) == 1024 and torch.equal(i2[t].cpu(), torch.arange(1024, dtype=torch.int32))


def test_full_size_hot_prefix():
    """The OPT-30B-shaped layer profiled on 4096 calibration tokens and reordered;
    the neurons that fired on at least 99 % of them (rounded down to whole mask
    words) are the always-listed prefix."""
    cfg, L, X = _full("c2", ntok=4)
    P, pc = _hot_first(cfg, L, 4096)
    n_hot = 32 * (int(np.count_nonzero(pc >= 0.99 * 4096)) // 32)
    assert n_hot >= 512, n_hot   # about 1157 neurons fire with probability 0.999 by construction
    del L
    _check_hot(P, X[:1].contiguous(), n_hot, where="c2 hot B=1")
    _check_hot(P, X, n_hot, where="c2 hot B=4")


# ---------------------------------------------------------------- OPT-66B-shaped stack (d 9216, ffn 36864)
def test_full_size_stack_prompt_batch():
    """The 128-token prompt of the OPT-66B-shaped stack in one call per entry
    point (d 9216, ffn 36864, B = 128: the union covers most rows), the batch
    the prompt-phase measurement times; sampled tokens against the oracle."""
    cfg = CONFIGS["c5"]
    L = make_layer(cfg, layer=3, device=DEV)
    X = make_tokens(cfg, cfg.prompt_tokens, device=DEV, layer=3, stream="prompt")
    idx, cnt = R.predict(L, X)
    Y = R.sparse(L, X, idx, cnt)
    torch.cuda.synchronize()
    H = _host(L)
    del L
    thr = O.logit_threshold(H["tau"])
    cnt_h = cnt.cpu().numpy()
    assert np.all((cnt_h >= 0) & (cnt_h <= cfg.ffn))
    for t in (0, 41, 85, cfg.prompt_tokens - 1):
        c = int(cnt_h[t])
        gi = idx[t, :c].cpu().numpy()
        xh = X[t].cpu()
        z = O.predictor_logits(xh, H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(gi, z, thr, where=f"c5 prompt t={t}")
        check_y(Y[t].cpu().numpy(), _oracle_y(H, xh, gi), where=f"c5 prompt t={t}")


def _stack_layer_hot_first(cfg, layer):
    """One layer of the stack as the stack measurement builds it: profiled on
    its 4096 calibration tokens, reordered hot-first, rows permuted; n_hot is
    the neurons that fired on >= 99 % of those tokens, in whole mask words."""
    L = make_layer(cfg, layer=layer, device=DEV)
    counts = R.profile(make_calibration(cfg, device=DEV, layer=layer), L["W_up"], L["b_up"]).cpu().numpy()
    perm, hot = R.reorder(counts, 0.8)
    P = R.permute_layer(L, torch.from_numpy(perm).to(DEV))
    del L
    n_hot = 32 * (int(np.count_nonzero(counts[perm] >= 0.99 * cfg.calib_tokens)) // 32)
    return P, n_hot, hot


@pytest.mark.parametrize("layer", [0, 41])
def test_full_size_stack_layers_hot_first(layer):
    """Layers of the 64-layer stack, profiled and reordered hot-first, decoded
    at B = 1 with the plain predictor (n_hot = 0) and with the always-listed
    prefix (n_hot > 0), each against the oracle."""
    cfg = CONFIGS["c5"]
    P, n_hot, hot = _stack_layer_hot_first(cfg, layer)
    assert 512 <= n_hot <= hot, (n_hot, hot)
    X = make_tokens(cfg, 2, device=DEV, layer=layer)
    H = _host(P)
    thr = O.logit_threshold(P["tau"])
    for nh in (0, n_hot):
        for t in range(X.shape[0]):
            x = X[t:t + 1].contiguous()
            idx, cnt = R.predict(P, x, n_hot=nh)
            y = R.sparse(P, x, idx, cnt)
            torch.cuda.synchronize()
            c = int(cnt.cpu()[0])
            gi = idx[0, :c].cpu().numpy()
            assert np.array_equal(gi[:nh], np.arange(nh))
            _, z = O.predict_hot(X[t].cpu(), H["P1"], None, "relu", H["P2"], H["b2"], P["tau"], nh)
            check_idx(gi, z, thr, where=f"c5 layer {layer} n_hot={nh} t={t}")
            check_y(y[0].cpu().numpy(), _oracle_y(H, X[t].cpu(), gi), where=f"c5 layer {layer} n_hot={nh} t={t}")
