"""Pins for the CPU oracle (run without a GPU).

The oracle is trusted only after it agrees with things other than itself:
  * hand-worked fixtures (tests/golden/*.json, derivations written out);
  * exact rational brute force on tiny dyadic inputs (fractions.Fraction);
  * closed forms on structured (identity / one-hot, non-square) weights;
  * invariants: all-ones mask = dense, empty mask = 0, superset-of-support
    mask = dense, batch invariance, reorder invariance;
  * the float64 error bound against exact arithmetic on general inputs;
  * the binomial law of the profile counts on the synthetic generator;
  * equivalence of the logit threshold with sigmoid(z) > tau.
`test_planted_mistakes_are_caught` plants plausible mistakes in the oracle
(on the CPU) and checks that at least one pin fails for each.
"""

import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import ffn as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------- exact helpers
def _frm(a):
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == 1:
        return [Fr(float(v)) for v in a]
    return [[Fr(float(v)) for v in row] for row in a]


def _dot(row, x):
    s = Fr(0)
    for a, b in zip(row, x):
        s += a * b
    return s


def _bf_logits(x, P1, b1, act, P2, b2):
    x, P1, P2 = _frm(x), _frm(P1), _frm(P2)
    b1 = _frm(b1) if b1 is not None else [Fr(0)] * len(P1)
    b2 = _frm(b2) if b2 is not None else [Fr(0)] * len(P2)
    s = [_dot(P1[j], x) + b1[j] for j in range(len(P1))]
    h = [max(v, Fr(0)) for v in s] if act == "relu" else s
    return [_dot(P2[i], h) + b2[i] for i in range(len(P2))]


def _bf_ffn(kind, x, W_up, b_up, W_gate, b_gate, W_down, idx):
    x, Wu, Wd = _frm(x), _frm(W_up), _frm(W_down)
    d_out = len(Wd[0])
    y = [Fr(0)] * d_out
    for i in idx:
        u = _dot(Wu[i], x) + (Fr(float(b_up[i])) if b_up is not None else Fr(0))
        if kind == "relu":
            a = max(u, Fr(0))
        else:
            Wg = _frm(W_gate)
            g = _dot(Wg[i], x) + (Fr(float(b_gate[i])) if b_gate is not None else Fr(0))
            a = max(g, Fr(0)) * u
        for j in range(d_out):
            y[j] += a * Wd[i][j]
    return y


def _dyadic(rng, *shape):
    # multiples of 1/8 in [-2, 2]: exact in fp16, and every product/sum below is exact in fp64
    return rng.integers(-16, 17, size=shape).astype(np.float64) / 8.0


def _as_f16(a):
    return np.asarray(a, dtype=np.float16)


# ---------------------------------------------------------------- pins
def pin_golden_ffn():
    g = _load("tiny_layer.json")
    e = g["expected"]
    x = _as_f16(g["x"])
    Wu, b, Wd = _as_f16(g["W_up_relu"]), np.float32(g["b_fire"]), _as_f16(g["W_down"])
    a = O.neuron_activations("relu", x, Wu, b, None, None, np.arange(4))
    assert np.array_equal(a, e["relu_a"]), a
    assert np.array_equal(O.dense_ffn("relu", x, Wu, b, None, None, Wd), e["relu_dense_y"])
    assert np.array_equal(O.sparse_ffn("relu", x, Wu, b, None, None, Wd, [0, 2]), e["relu_y_idx_0_2"])
    assert np.array_equal(O.sparse_ffn("relu", x, Wu, b, None, None, Wd, [1, 3]), e["relu_y_idx_1_3"])
    assert np.array_equal(O.sparse_ffn("relu", x, Wu, b, None, None, Wd, []), [0.0, 0.0, 0.0])
    WuR = _as_f16(g["W_up_reglu"])
    a = O.neuron_activations("reglu", x, WuR, None, Wu, b, np.arange(4))
    assert np.array_equal(a, e["reglu_a"]), a
    assert np.array_equal(O.dense_ffn("reglu", x, WuR, None, Wu, b, Wd), e["reglu_dense_y"])


def pin_golden_predictor():
    g = _load("tiny_layer.json")
    e = g["expected"]
    x = _as_f16(g["x"])
    P1, b1, P2, b2 = _as_f16(g["P1"]), np.float32(g["b1"]), _as_f16(g["P2"]), np.float32(g["b2"])
    z = O.predictor_logits(x, P1, b1, "relu", P2, b2)
    assert np.array_equal(z, e["z_relu_hidden"]), z
    for tau, key in ((0.5, "idx_tau_0.5"), (0.7, "idx_tau_0.7"), (0.25, "idx_tau_0.25")):
        idx, _ = O.predict(x, P1, b1, "relu", P2, b2, tau)
        assert list(idx) == e[key], (tau, idx)
    z = O.predictor_logits(x, P1, b1, "none", P2, b2)
    assert np.array_equal(z, e["z_no_hidden_act"]), z
    idx, _ = O.predict(x, P1, b1, "none", P2, b2, 0.5)
    assert list(idx) == e["idx_no_hidden_act_tau_0.5"]
    layer = dict(kind="relu", W_up=_as_f16(g["W_up_relu"]), b_up=np.float32(g["b_fire"]),
                 W_gate=None, b_gate=None, W_down=_as_f16(g["W_down"]), P1=P1, b1=b1,
                 P2=P2, b2=b2, tau=0.5)
    y, idx, _ = O.decode_step(layer, x)
    assert list(idx) == e["idx_tau_0.5"] and np.array_equal(y, e["decode_y_tau_0.5"])


def pin_golden_profile_reorder():
    g = _load("tiny_layer.json")
    e = g["expected"]
    counts = O.profile_counts("relu", _as_f16(e["calib_X"]), _as_f16(g["W_up_relu"]),
                              np.float32(g["b_fire"]))
    assert list(counts) == e["profile_counts"], counts
    perm, hot = O.reorder_plan(counts, 0.8)
    assert list(perm) == e["reorder_perm"] and hot == e["reorder_hot_count"], (perm, hot)
    for case in _load("reorder_cases.json")["cases"]:
        perm, hot = O.reorder_plan(case["counts"], case["hot_share"])
        assert list(perm) == case["perm"] and hot == case["hot_count"], (case, perm, hot)


def pin_exact_predictor():
    rng = np.random.default_rng(11)
    for (d, r, ffn) in ((5, 3, 7), (9, 4, 2), (1, 1, 3), (6, 8, 5)):
        for act in ("relu", "none"):
            x, P1, b1 = _dyadic(rng, d), _dyadic(rng, r, d), _dyadic(rng, r)
            P2, b2 = _dyadic(rng, ffn, r), _dyadic(rng, ffn)
            z = O.predictor_logits(_as_f16(x), _as_f16(P1), b1, act, _as_f16(P2), b2)
            zx = _bf_logits(x, P1, b1, act, P2, b2)
            assert [Fr(float(v)) for v in z] == zx, (d, r, ffn, act)
            idx, _ = O.predict(_as_f16(x), _as_f16(P1), b1, act, _as_f16(P2), b2, 0.5)
            assert list(idx) == [i for i in range(ffn) if zx[i] > 0]


def pin_exact_ffn():
    rng = np.random.default_rng(12)
    for (d, ffn) in ((5, 7), (3, 11), (8, 4), (1, 2)):
        for kind in ("relu", "reglu"):
            x = _dyadic(rng, d)
            Wu, Wg, Wd = _dyadic(rng, ffn, d), _dyadic(rng, ffn, d), _dyadic(rng, ffn, d + 1)
            bu, bg = _dyadic(rng, ffn), _dyadic(rng, ffn)
            if kind == "relu":
                Wg_, bg_ = None, None
            else:
                Wg_, bg_ = Wg, bg
            for idx in (list(range(ffn)), sorted(rng.choice(ffn, size=max(1, ffn // 2), replace=False).tolist()), []):
                y = O.sparse_ffn(kind, _as_f16(x), _as_f16(Wu), bu,
                                 None if Wg_ is None else _as_f16(Wg_), bg_, _as_f16(Wd), idx)
                yx = _bf_ffn(kind, x, Wu, bu, Wg_, bg_, Wd, idx)
                assert [Fr(float(v)) for v in y] == yx, (kind, d, ffn, idx)


def pin_float64_error_bound():
    """Oracle on general fp16 inputs vs exact arithmetic, within the fp64 bound."""
    rng = np.random.default_rng(13)
    u = 2.0 ** -53
    for kind in ("relu", "reglu"):
        d, ffn = 24, 17
        x = _as_f16(rng.standard_normal(d))
        Wu = _as_f16(rng.standard_normal((ffn, d)) / math.sqrt(d))
        Wg = _as_f16(rng.standard_normal((ffn, d)) / math.sqrt(d))
        Wd = _as_f16(rng.standard_normal((ffn, d)) / math.sqrt(d))
        b = rng.standard_normal(ffn).astype(np.float32)
        idx = list(range(ffn))
        if kind == "relu":
            y = O.sparse_ffn(kind, x, Wu, b, None, None, Wd, idx)
            yx = _bf_ffn(kind, x, Wu, b, None, None, Wd, idx)
        else:
            y = O.sparse_ffn(kind, x, Wu, None, Wg, b, Wd, idx)
            yx = _bf_ffn(kind, x, Wu, None, Wg, b, Wd, idx)
        # |a_hat - a| and |y_hat - y| are bounded by gamma_n times the absolute-value problem
        n = 2 * d + ffn + 4
        gamma = n * u / (1 - n * u)
        xa, Wua, Wga, Wda = (np.abs(np.float64(v)) for v in (x, Wu, Wg, Wd))
        su = Wua @ xa + (np.abs(b) if kind == "relu" else 0)
        sg = Wga @ xa + np.abs(b)
        mag = su if kind == "relu" else su * sg
        bound = 4 * gamma * (mag @ Wda) + 1e-300
        err = np.abs(np.array([float(v) for v in yx]) - y)
        assert np.all(err <= bound), (kind, err.max(), bound.min())


def pin_closed_forms():
    rng = np.random.default_rng(14)
    # identity FFN: y = relu(x + b)
    d = 6
    x = _as_f16(rng.standard_normal(d))
    b = rng.standard_normal(d).astype(np.float32)
    I = np.eye(d, dtype=np.float16)
    y = O.dense_ffn("relu", x, I, b, None, None, I)
    assert np.array_equal(y, np.maximum(np.float64(x) + np.float64(b), 0.0))
    # one-hot rows, non-square: u_i = x[sig(i)] + b_i ; y[pi(i)] += c_i * relu(u_i)
    d, ffn = 4, 6
    sig, pi = [2, 0, 3, 1, 2, 0], [1, 3, 0, 2, 1, 3]
    c = [1.0, -2.0, 0.5, 4.0, -1.0, 0.25]
    x = np.float16([1.5, -0.5, 2.0, -3.0])
    b = np.float32([0.5, 1.0, 1.0, 2.5, -2.5, 0.0])
    Wu = np.zeros((ffn, d), np.float16)
    Wd = np.zeros((ffn, d), np.float16)
    for i in range(ffn):
        Wu[i, sig[i]] = 1.0
        Wd[i, pi[i]] = c[i]
    expect = [0.0] * d
    for i in range(ffn):
        expect[pi[i]] += c[i] * max(float(x[sig[i]]) + float(b[i]), 0.0)
    assert np.array_equal(O.dense_ffn("relu", x, Wu, b, None, None, Wd), expect)
    # ReGLU with gate == up and no biases: a = relu(u) * u = relu(u)^2
    Wr = _as_f16(rng.standard_normal((ffn, d)))
    a = O.neuron_activations("reglu", x, Wr, None, Wr, None, np.arange(ffn))
    uu = np.float64(Wr) @ np.float64(x)
    assert np.array_equal(a, np.maximum(uu, 0.0) ** 2)
    # ReGLU: gate selects coordinate sig(i), up selects pi(i): a_i = relu(x[sig]+b) * x[pi]
    Wg1 = Wu
    Wu1 = np.zeros((ffn, d), np.float16)
    for i in range(ffn):
        Wu1[i, pi[i]] = 1.0
    a = O.neuron_activations("reglu", x, Wu1, None, Wg1, b, np.arange(ffn))
    assert np.array_equal(a, [max(float(x[sig[i]]) + float(b[i]), 0.0) * float(x[pi[i]]) for i in range(ffn)])
    # predictor with a basis token e_k: s = P1[:, k] + b1
    r, d2, k = 3, 5, 2
    P1 = _as_f16(rng.standard_normal((r, d2)))
    P2 = np.eye(r, dtype=np.float16)[[2, 0, 1, 2]]     # z picks hidden units 2,0,1,2
    b1 = np.float32([0.25, -0.5, 0.0])
    e = np.zeros(d2, np.float16)
    e[k] = 1.0
    z = O.predictor_logits(e, P1, b1, "relu", P2, None)
    h = np.maximum(np.float64(P1[:, k]) + np.float64(b1), 0.0)
    assert np.array_equal(z, h[[2, 0, 1, 2]])


def pin_sigmoid_threshold():
    rng = np.random.default_rng(15)
    z = rng.standard_normal(4000) * 3
    P2 = np.eye(1, dtype=np.float16).repeat(4000, axis=0)
    for tau in (0.05, 0.3, 0.5, 0.7, 0.95):
        # one hidden unit h = 1 (P1 = [1], x = [1]); z_i = 1 + (z_i - 1) via the bias
        idx, zz = O.predict(np.float16([1.0]), np.float16([[1.0]]), None, "relu", P2, z - 1.0, tau)
        sig = 1.0 / (1.0 + np.exp(-zz))
        far = np.abs(sig - tau) > 1e-12
        mask = np.zeros(4000, bool)
        mask[idx] = True
        assert np.array_equal(mask[far], (sig > tau)[far]), tau
        assert np.all(np.diff(idx) > 0)


def _random_layer(rng, kind, d, ffn, r):
    Wu = _as_f16(rng.standard_normal((ffn, d)) / math.sqrt(d))
    Wg = _as_f16(rng.standard_normal((ffn, d)) / math.sqrt(d)) if kind == "reglu" else None
    Wd = _as_f16(rng.standard_normal((ffn, d)) / math.sqrt(d))
    b = (rng.standard_normal(ffn) - 1.0).astype(np.float32)
    P1 = _as_f16(rng.standard_normal((r, d)) / math.sqrt(d))
    P2 = _as_f16(rng.standard_normal((ffn, r)) / math.sqrt(r))
    b2 = (rng.standard_normal(ffn) - 0.5).astype(np.float32)
    L = dict(kind=kind, W_up=Wu, W_gate=Wg, W_down=Wd, P1=P1, b1=None, P2=P2, b2=b2, tau=0.5)
    if kind == "relu":
        L.update(b_up=b, b_gate=None)
    else:
        L.update(b_up=None, b_gate=b)
    return L


def pin_invariants():
    rng = np.random.default_rng(16)
    for kind in ("relu", "reglu"):
        L = _random_layer(rng, kind, 40, 96, 16)
        args = (L["W_up"], L["b_up"], L["W_gate"], L["b_gate"], L["W_down"])
        for _ in range(3):
            x = _as_f16(rng.standard_normal(40))
            dense = O.dense_ffn(kind, x, *args)
            # all-ones mask == dense (bitwise)
            assert np.array_equal(O.sparse_ffn(kind, x, *args[:4], args[4], np.arange(96)), dense)
            # empty mask == 0 exactly
            assert np.array_equal(O.sparse_ffn(kind, x, *args[:4], args[4], []), np.zeros(40))
            # superset of the nonzero-activation set == dense (bitwise: skipped terms are +-0)
            a = O.neuron_activations(kind, x, *args[:4], np.arange(96))
            support = set(np.flatnonzero(a != 0).tolist())
            extra = set(rng.choice(96, size=10, replace=False).tolist())
            assert np.array_equal(O.sparse_ffn(kind, x, *args[:4], args[4], sorted(support | extra)), dense)
            # a strict subset that drops a nonzero activation differs
            if support:
                drop = sorted(support)[0]
                y = O.sparse_ffn(kind, x, *args[:4], args[4], sorted(support - {drop}))
                assert not np.array_equal(y, dense)
        # batch invariance and union
        X = _as_f16(rng.standard_normal((5, 40)))
        lists = [O.predict(X[t], L["P1"], None, "relu", L["P2"], L["b2"], 0.5)[0] for t in range(5)]
        Y = O.batched_sparse_ffn(kind, X, *args, lists)
        for t in range(5):
            assert np.array_equal(Y[t], O.sparse_ffn(kind, X[t], *args, lists[t]))
        U = O.union_rows(lists)
        m = np.zeros(96, bool)
        for l in lists:
            m[l] = True
        assert np.array_equal(U, np.flatnonzero(m))


def pin_reorder_invariance():
    rng = np.random.default_rng(17)
    for kind in ("relu", "reglu"):
        L = _random_layer(rng, kind, 32, 64, 8)
        X = _as_f16(rng.standard_normal((64, 32)))
        Wf = L["W_up"] if kind == "relu" else L["W_gate"]
        bf = L["b_up"] if kind == "relu" else L["b_gate"]
        counts = O.profile_counts(kind, X, Wf, bf)
        perm, hot = O.reorder_plan(counts, 0.8)
        P = {k: (O.permute_rows(v, perm) if (v is not None and k in
             ("W_up", "W_gate", "W_down", "P2", "b2", "b_up", "b_gate")) else v) for k, v in L.items()}
        inv = np.argsort(perm)
        # permuted counts are the sorted counts, and the hot prefix is the same neurons
        c2 = O.profile_counts(kind, X, P["W_up"] if kind == "relu" else P["W_gate"],
                              P["b_up"] if kind == "relu" else P["b_gate"])
        assert np.array_equal(c2, counts[perm]) and np.all(np.diff(c2) <= 0)
        for t in range(4):
            x = X[t]
            y, idx, z = O.decode_step(L, x)
            y2, idx2, z2 = O.decode_step(P, x)
            np.testing.assert_allclose(z2, z[perm], rtol=0, atol=1e-12)
            # idx' = sort(perm^-1[idx]); only a logit within rounding of the threshold may differ
            diff = set(idx2.tolist()) ^ set(inv[idx].tolist())
            assert all(abs(z2[j]) <= 1e-9 for j in diff), diff
            assert np.all(np.diff(idx2) > 0)
            np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)


def pin_reorder_properties():
    rng = np.random.default_rng(18)
    for n in (1, 2, 7, 100, 1000):
        for share in (0.5, 0.8, 0.999, 1.0):
            counts = rng.integers(0, 6, size=n) * rng.integers(0, 2, size=n)
            perm, hot = O.reorder_plan(counts, share)
            assert sorted(perm.tolist()) == list(range(n))
            cs = counts[perm]
            assert np.all(np.diff(cs) <= 0)
            for j in range(n - 1):       # ties keep the original order
                if cs[j] == cs[j + 1]:
                    assert perm[j] < perm[j + 1]
            total = counts.sum()
            if total == 0:
                assert hot == 0
                continue
            pre = np.concatenate([[0], np.cumsum(cs)])
            assert pre[hot] >= share * total and (hot == 0 or pre[hot - 1] < share * total)


def pin_profile_exact():
    rng = np.random.default_rng(19)
    for kind in ("relu", "reglu"):
        X, W, b = _dyadic(rng, 9, 5), _dyadic(rng, 6, 5), _dyadic(rng, 6)
        counts = O.profile_counts(kind, _as_f16(X), _as_f16(W), b)
        Xf, Wf, bf = _frm(X), _frm(W), _frm(b)
        want = [sum(1 for t in range(9) if _dot(Wf[i], Xf[t]) + bf[i] > 0) for i in range(6)]
        assert list(counts) == want


def pin_profile_binomial():
    """Unit-norm rows and x ~ N(0, I): w.x ~ N(0,1), so counts_i ~ Binomial(n, f_i) with b_i = Phi^-1(f_i)."""
    from synthetic import custom_config, make_layer, make_calibration
    cfg = custom_config("relu", d=128, ffn=384, r=16, mean=0.2, exponent=0.8, number=77)
    L = make_layer(cfg, predictor=False)
    n = 3000
    X = make_calibration(cfg, n)
    counts = O.profile_counts("relu", X, L["W_up"], L["b_up"])
    f = L["f"]
    sd = np.sqrt(n * f * (1 - f))
    assert np.all(np.abs(counts - n * f) <= 5 * sd + 2), np.max(np.abs(counts - n * f) / (sd + 1))


def pin_swiglu():
    """SiLU and the SiLU-gated FFN against forms that share no code with the oracle.

    SiLU(v) = v * sigmoid(v) = (v / 2) * (1 + tanh(v / 2)), and SiLU(v) - SiLU(-v) = v
    (sigmoid(v) + sigmoid(-v) = 1).  The FFN is then written out row by row with
    the tanh form: y = sum_i SiLU(W_gate[i] x + b_gate_i) (W_up[i] x + b_up_i) W_down[i].
    """
    v = np.linspace(-30.0, 30.0, 601)
    s = O.silu(v)
    assert np.allclose(s - O.silu(-v), v, rtol=0, atol=1e-13)
    # (1 + tanh(v / 2) cancels for v << 0: an absolute bound there)
    assert np.allclose(s, 0.5 * v * (1.0 + np.tanh(0.5 * v)), rtol=1e-13, atol=1e-13)
    assert O.silu(0.0) == 0.0 and O.silu(800.0) == 800.0 and O.silu(-800.0) == 0.0
    rng = np.random.default_rng(21)
    for (d, ffn) in ((6, 9), (16, 5), (1, 3)):
        x = rng.standard_normal(d).astype(np.float16)
        Wu = rng.standard_normal((ffn, d)).astype(np.float16)
        Wg = rng.standard_normal((ffn, d)).astype(np.float16)
        Wd = rng.standard_normal((ffn, d)).astype(np.float16)
        bu = rng.standard_normal(ffn).astype(np.float32)
        bg = rng.standard_normal(ffn).astype(np.float32)
        idx = np.sort(rng.choice(ffn, size=max(1, ffn // 2), replace=False))
        want = [0.0] * d
        for i in idx:
            u = float(bu[i]) + sum(float(Wu[i, k]) * float(x[k]) for k in range(d))
            g = float(bg[i]) + sum(float(Wg[i, k]) * float(x[k]) for k in range(d))
            a = 0.5 * g * (1.0 + math.tanh(0.5 * g)) * u
            for k in range(d):
                want[k] += a * float(Wd[i, k])
        got = O.sparse_ffn("swiglu", x, Wu, bu, Wg, bg, Wd, idx)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (d, ffn)
        # every neuron listed is the dense FFN; an empty list gives 0
        assert np.array_equal(O.sparse_ffn("swiglu", x, Wu, bu, Wg, bg, Wd, np.arange(ffn)),
                              O.dense_ffn("swiglu", x, Wu, bu, Wg, bg, Wd))
        assert not np.any(O.sparse_ffn("swiglu", x, Wu, bu, Wg, bg, Wd, []))


def pin_hot_prefix():
    """The hot-prefix list: no prefix is the plain prediction; a whole prefix is
    every neuron; otherwise the prefix, then exactly the plain prediction's
    neurons past it (the predictor's row i depends on row i of P2 and b2 only)."""
    rng = np.random.default_rng(22)
    d, r, ffn = 24, 8, 160
    x = rng.standard_normal(d).astype(np.float16)
    P1 = rng.standard_normal((r, d)).astype(np.float16)
    P2 = rng.standard_normal((ffn, r)).astype(np.float16)
    b2 = (rng.standard_normal(ffn) * 0.5).astype(np.float32)
    full, zf = O.predict(x, P1, None, "relu", P2, b2, 0.5)
    idx0, z0 = O.predict_hot(x, P1, None, "relu", P2, b2, 0.5, 0)
    assert np.array_equal(idx0, full) and np.array_equal(z0, zf)
    idxa, za = O.predict_hot(x, P1, None, "relu", P2, b2, 0.5, ffn)
    assert np.array_equal(idxa, np.arange(ffn)) and np.all(np.isinf(za))
    for n_hot in (32, 64, 96):
        idx, z = O.predict_hot(x, P1, None, "relu", P2, b2, 0.5, n_hot)
        want = np.concatenate([np.arange(n_hot), full[full >= n_hot]])
        assert np.array_equal(idx, want), n_hot
        assert np.array_equal(z[n_hot:], zf[n_hot:])
        assert np.all(np.diff(idx) > 0)


def pin_int4_rows():
    """INT4 rows against values fixed by the format's definition.

    A group whose largest magnitude is 7 * 2^e and whose weights are k * 2^e
    (|k| <= 7) has scale 2^e and codes k + 8 exactly; halves round to even
    (w / s = 2.5 -> 2, 3.5 -> 4, -2.5 -> -2); an all-zero group has scale 0 and
    code 8; weight 0 of a row is the low nibble of byte 0, weight 1 its high
    nibble.  On random rows the dequantised weight is within s / 2 of w.
    """
    e = 2.0 ** -3
    ks = np.array([7, -7, 0, 1, -1, 3, -5, 2] * 8, dtype=np.int64)
    row = np.concatenate([(ks * e).astype(np.float16), np.zeros(64, np.float16)])
    halves = np.zeros(64, np.float16)
    halves[:5] = [7.0, 2.5, 3.5, -2.5, -7.0]     # scale 1: codes 15, 10, 12, 6, 1
    W = np.stack([row, np.concatenate([halves, np.zeros(64, np.float16)])])
    q, sc = O.quantize_rows(W)
    assert sc.dtype == np.float16 and sc.shape == (2, 2) and q.shape == (2, 64)
    assert sc[0, 0] == np.float16(e) and sc[0, 1] == 0 and sc[1, 0] == 1
    codes0 = np.empty(128, np.int64)
    codes0[0::2], codes0[1::2] = q[0] & 0xF, q[0] >> 4
    assert np.array_equal(codes0[:64], ks + 8) and np.all(codes0[64:] == 8)
    assert q[0, 0] == (7 + 8) | ((-7 + 8) << 4)            # low nibble = weight 0
    assert list((q[1, :3] & 0xF)) == [15, 12, 1] and list(q[1, :2] >> 4) == [10, 6]
    assert np.array_equal(O.dequantize_rows(q, sc, 128)[0], row.astype(np.float64))
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((5, 192)) * np.exp(rng.standard_normal((5, 1)))).astype(np.float16)
    q, sc = O.quantize_rows(W)
    back = O.dequantize_rows(q, sc, 192)
    half = np.repeat(sc.astype(np.float64), 64, axis=1) / 2
    assert np.all(np.abs(back - W.astype(np.float64)) <= half * (1 + 1e-6))


PINS = [pin_golden_ffn, pin_golden_predictor, pin_golden_profile_reorder, pin_exact_predictor,
        pin_exact_ffn, pin_float64_error_bound, pin_closed_forms, pin_sigmoid_threshold,
        pin_invariants, pin_reorder_invariance, pin_reorder_properties, pin_profile_exact,
        pin_profile_binomial, pin_swiglu, pin_hot_prefix, pin_int4_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes
def _mutants():
    orig = {k: getattr(O, k) for k in ("neuron_preactivations", "neuron_activations", "predictor_hidden",
                                       "predict", "profile_counts", "reorder_plan", "sparse_ffn",
                                       "logit_threshold", "predictor_logits", "predict_hot",
                                       "quantize_rows")}

    def pre_no_bias(kind, x, W_up, b_up, W_gate, b_gate, rows):
        return orig["neuron_preactivations"](kind, x, W_up, None, W_gate, None, rows)

    def pre_neg_bias(kind, x, W_up, b_up, W_gate, b_gate, rows):
        nb = lambda b: None if b is None else -O.widen(b)
        return orig["neuron_preactivations"](kind, x, W_up, nb(b_up), W_gate, nb(b_gate), rows)

    def act_gate_no_relu(kind, x, W_up, b_up, W_gate, b_gate, rows):
        u, g = O.neuron_preactivations(kind, x, W_up, b_up, W_gate, b_gate, rows)
        return np.maximum(u, 0.0) if kind == "relu" else g * u

    def act_relu_on_up(kind, x, W_up, b_up, W_gate, b_gate, rows):
        u, g = O.neuron_preactivations(kind, x, W_up, b_up, W_gate, b_gate, rows)
        return np.maximum(u, 0.0) if kind == "relu" else g * np.maximum(u, 0.0)

    def hidden_no_relu(x, P1, b1=None, act="relu"):
        return orig["predictor_hidden"](x, P1, b1, "none")

    def hidden_no_bias(x, P1, b1=None, act="relu"):
        return orig["predictor_hidden"](x, P1, None, act)

    def predict_ge(x, P1, b1, act, P2, b2, tau):
        z = O.predictor_logits(x, P1, b1, act, P2, b2)
        return np.flatnonzero(z >= O.logit_threshold(tau)), z

    def predict_descending(x, P1, b1, act, P2, b2, tau):
        idx, z = orig["predict"](x, P1, b1, act, P2, b2, tau)
        return idx[::-1].copy(), z

    def thr_ignores_tau(tau):
        return 0.0

    def thr_inverted(tau):
        return math.log((1 - tau) / tau)

    def logits_no_b2(x, P1, b1, act, P2, b2):
        return orig["predictor_logits"](x, P1, b1, act, P2, None)

    def profile_ge(kind, X, W_fire, b_fire):
        pre = O.widen(X) @ O.widen(W_fire).T + O.widen(b_fire)[None, :]
        return (pre >= 0).sum(axis=0)

    def profile_transposed(kind, X, W_fire, b_fire):
        pre = O.widen(X) @ O.widen(W_fire).T + O.widen(b_fire)[None, :]
        return (pre > 0).sum(axis=1)

    def reorder_unstable(counts, hot_share=0.8):
        counts = np.asarray(counts, dtype=np.int64)
        perm = np.argsort(-counts[::-1], kind="stable")
        perm = (len(counts) - 1 - perm)
        _, hot = orig["reorder_plan"](counts, hot_share)
        return perm, hot

    def reorder_strict(counts, hot_share=0.8):
        perm, _ = orig["reorder_plan"](counts, hot_share)
        c = np.asarray(counts)[perm]
        total = c.sum()
        if total == 0:
            return perm, 0
        k = int(np.argmax(np.cumsum(c) > hot_share * total)) + 1
        return perm, k

    def sparse_f32(kind, x, W_up, b_up, W_gate, b_gate, W_down, idx):
        idx = np.asarray(idx, dtype=np.int64)
        Wd = np.asarray(O.widen(W_down), np.float32)
        y = np.zeros(Wd.shape[1], np.float32)
        if idx.size:
            a = O.neuron_activations(kind, x, W_up, b_up, W_gate, b_gate, idx).astype(np.float32)
            for ai, i in zip(a, idx):
                y += ai * Wd[i]
        return y.astype(np.float64)

    def sparse_wrong_row(kind, x, W_up, b_up, W_gate, b_gate, W_down, idx):
        idx = np.asarray(idx, dtype=np.int64)
        Wd = O.widen(W_down)
        y = np.zeros(Wd.shape[1])
        if idx.size:
            a = O.neuron_activations(kind, x, W_up, b_up, W_gate, b_gate, idx)
            for j, (ai, i) in enumerate(zip(a, idx)):
                y += ai * Wd[j]          # position instead of neuron id
        return y

    def sparse_transposed(kind, x, W_up, b_up, W_gate, b_gate, W_down, idx):
        idx = np.asarray(idx, dtype=np.int64)
        Wd = O.widen(W_down)
        a_full = np.zeros(Wd.shape[0])
        if idx.size:
            a_full[idx] = O.neuron_activations(kind, x, W_up, b_up, W_gate, b_gate, idx)
        return Wd @ a_full            # W_down read as d x ffn

    def pre_bias_on_up(kind, x, W_up, b_up, W_gate, b_gate, rows):
        if kind == "relu":
            return orig["neuron_preactivations"](kind, x, W_up, b_up, W_gate, b_gate, rows)
        return orig["neuron_preactivations"](kind, x, W_up, b_gate, W_gate, b_up, rows)

    def act_swiglu_on_up(kind, x, W_up, b_up, W_gate, b_gate, rows):
        if kind != "swiglu":
            return orig["neuron_activations"](kind, x, W_up, b_up, W_gate, b_gate, rows)
        u, g = O.neuron_preactivations(kind, x, W_up, b_up, W_gate, b_gate, rows)
        return O.silu(u) * g

    def act_swiglu_sigmoid(kind, x, W_up, b_up, W_gate, b_gate, rows):
        if kind != "swiglu":
            return orig["neuron_activations"](kind, x, W_up, b_up, W_gate, b_gate, rows)
        u, g = O.neuron_preactivations(kind, x, W_up, b_up, W_gate, b_gate, rows)
        return u / (1.0 + np.exp(-g))

    def pre_swiglu_no_gate_bias(kind, x, W_up, b_up, W_gate, b_gate, rows):
        if kind != "swiglu":
            return orig["neuron_preactivations"](kind, x, W_up, b_up, W_gate, b_gate, rows)
        return orig["neuron_preactivations"](kind, x, W_up, b_up, W_gate, None, rows)

    def hot_not_shifted(x, P1, b1, act, P2, b2, tau, n_hot):
        idx, z = orig["predict_hot"](x, P1, b1, act, P2, b2, tau, n_hot)
        return np.concatenate([idx[:n_hot], idx[n_hot:] - n_hot]), z

    def hot_prefix_not_listed(x, P1, b1, act, P2, b2, tau, n_hot):
        idx, z = orig["predict_hot"](x, P1, b1, act, P2, b2, tau, n_hot)
        return idx[n_hot:], z

    def q4_nibbles_swapped(W):
        q, sc = orig["quantize_rows"](W)
        return ((q >> 4) | (q << 4)).astype(np.uint8), sc

    def q4_scale_over_8(W):
        W32 = np.asarray(W, dtype=np.float16).astype(np.float32)
        q, _ = orig["quantize_rows"](W)
        amax = np.abs(W32.reshape(W32.shape[0], -1, 64)).max(axis=2)
        return q, (amax / np.float32(8.0)).astype(np.float16)

    def q4_floor(W):
        W32 = np.asarray(W, dtype=np.float16).astype(np.float32)
        rows, d = W32.shape
        G = W32.reshape(rows, d // 64, 64)
        s16 = (np.abs(G).max(axis=2) / np.float32(7)).astype(np.float16)
        with np.errstate(divide="ignore", invalid="ignore"):
            c = np.where(s16[..., None] == 0, 0, np.clip(np.floor(G / s16.astype(np.float32)[..., None]), -8, 7))
        codes = (c.astype(np.int64) + 8).reshape(rows, d)
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), s16

    return {
        "INT4 nibbles swapped": ("quantize_rows", q4_nibbles_swapped),
        "INT4 scale max/8": ("quantize_rows", q4_scale_over_8),
        "INT4 floor instead of rint": ("quantize_rows", q4_floor),
        "hot prefix: rest not shifted by n_hot": ("predict_hot", hot_not_shifted),
        "hot prefix not listed": ("predict_hot", hot_prefix_not_listed),
        "SwiGLU with SiLU on up": ("neuron_activations", act_swiglu_on_up),
        "SwiGLU with sigmoid for SiLU": ("neuron_activations", act_swiglu_sigmoid),
        "SwiGLU gate bias dropped": ("neuron_preactivations", pre_swiglu_no_gate_bias),
        "bias dropped": ("neuron_preactivations", pre_no_bias),
        "bias sign flipped": ("neuron_preactivations", pre_neg_bias),
        "ReGLU without ReLU on the gate": ("neuron_activations", act_gate_no_relu),
        "ReGLU with ReLU on up": ("neuron_activations", act_relu_on_up),
        "predictor hidden ReLU dropped": ("predictor_hidden", hidden_no_relu),
        "predictor b1 dropped": ("predictor_hidden", hidden_no_bias),
        "threshold not strict": ("predict", predict_ge),
        "index list descending": ("predict", predict_descending),
        "threshold ignores tau": ("logit_threshold", thr_ignores_tau),
        "threshold inverted": ("logit_threshold", thr_inverted),
        "predictor b2 dropped": ("predictor_logits", logits_no_b2),
        "profile counts >= 0": ("profile_counts", profile_ge),
        "profile summed over the wrong axis": ("profile_counts", profile_transposed),
        "reorder ties reversed": ("reorder_plan", reorder_unstable),
        "hot set uses > instead of >=": ("reorder_plan", reorder_strict),
        "y accumulated in float32": ("sparse_ffn", sparse_f32),
        "W_down row by list position": ("sparse_ffn", sparse_wrong_row),
        "W_down read transposed": ("sparse_ffn", sparse_transposed),
        "ReGLU bias on up instead of gate": ("neuron_preactivations", pre_bias_on_up),
    }


@pytest.mark.parametrize("name", list(_mutants().keys()))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception as exc:  # AssertionError or a shape error both count as detection
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects the planted mistake: {name}"
