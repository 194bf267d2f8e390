#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X sparse-FFN path.

Headline workload: the OPT-66B-shaped 64-layer FFN stack (ReLU, d 9216,
ffn 36864, predictor rank 1024, fp16 weights, about 93 GB resident).  Every
layer is profiled on its 4096 calibration tokens and reordered hot-first
(pi_profile, pi_reorder, pi_permute_rows); the neurons that fired on at least
99 % of those tokens, rounded down to whole 32-neuron words, are the layer's
always-listed prefix.  Then the 128-token prompt runs through the stack on
the union path, and the decode steps follow at batch 1.

A step is one decode token through all 64 layers: per layer the predictor
(hidden layer, logits, threshold, ordered compaction) and the neuron-aware
FFN over the listed rows only, inputs already resident in HBM.  Each step's
64 layers are captured once as a HIP graph; K steps are K graph replays
between HIP events on the stream the graphs run on, bracketed by device
synchronisation.  value = decode tokens/s per layer = 64 K / elapsed, with the
achieved HBM GB/s on the bytes each layer step must touch:

  T = 2 r d + (ffn - n_hot)(2 r + 4)    predictor weights + b2 (prefix rows skipped)
    + (m + 1) count 2 d + 4 count       listed rows of W_up [W_gate] W_down + bias
    + 2 d + 4 d + 8 count               x, y, index list write + read

with m = 1 (ReLU) or 2 (gated) and count the layer step's own list length.
The 64 layers cycle through 93 GB, far beyond the 256 MB Infinity Cache, so
every layer is read cache-cold.

Beside the headline: the dense FFN of the same layers through the library
and through torch (hipBLASLt), graph-timed the same way; per-entry-point
kernel times from graphs of back-to-back launches (the roofline of the
dominant kernel); the CPU oracle on a bounded token sample; and the other
configurations' lines (an OPT-30B-shaped layer, the Falcon-40B-shaped batch
sweep, the hot prefix, INT4 rows, the prompt phase against torch).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the single-token kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes over `bench.py --profile-run` (hot-first layers of the
# stack), each scaled by what the same counter reads for an identity
# pi_permute_rows copy of known size.  They hold for the kernel sources with
# this SHA-256 prefix only; for any other source the bench reports traffic as null.
MEASURED_TRAFFIC = {
    # the sources the single-token kernels are built from, hashed in this order
    "sources": ["activation_sparse_predictor_amd/csrc/fused.hip", "activation_sparse_predictor_amd/csrc/common.hpp"],
    "sha256_16": "52529ff632774193",
    "config": "c5",
    "bytes_per_launch": {"pi_ffn_decode_hot_begin": 1.453e+08, "pi_ffn_decode_hot_end": 8.542e+07},
}

# one kernel each at B = 1
KERNEL_OF = {"pi_ffn_predict": "k_predict_fused", "pi_ffn_sparse": "k_sparse_fused",
             "pi_ffn_decode_hot_begin": "k_predict_fused", "pi_ffn_decode_hot_end": "k_sparse_fused"}


def kernel_source_hash():
    """SHA-256 prefix over the single-token kernels' sources (None if one is missing)."""
    import hashlib
    h = hashlib.sha256()
    try:
        for rel in MEASURED_TRAFFIC["sources"]:
            h.update(open(os.path.join(ROOT, rel), "rb").read())
    except OSError:
        return None
    return h.hexdigest()[:16]


def measured_traffic(config_key, entry):
    h = kernel_source_hash()
    if h is None or h != MEASURED_TRAFFIC["sha256_16"] or config_key != MEASURED_TRAFFIC["config"]:
        return None
    return MEASURED_TRAFFIC["bytes_per_launch"].get(entry)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def touched_bytes(kind, d, r, ffn, count, n_hot=0):
    m = 1 if kind == "relu" else 2
    return (2 * r * d + (ffn - n_hot) * (2 * r + 4) + (m + 1) * count * 2 * d + 4 * count
            + 2 * d + 4 * d + 8 * count)


def predict_bytes(d, r, ffn, count, n_hot=0):
    return 2 * r * d + (ffn - n_hot) * (2 * r + 4) + 2 * d + 4 * count


def hot_begin_bytes(kind, d, r, ffn, count, n_hot):
    """The first launch of a hot decode step: the predictor (prefix rows of P2
    skipped) and the prefix's FFN rows."""
    m = 1 if kind == "relu" else 2
    return predict_bytes(d, r, ffn, count, n_hot) + (m + 1) * n_hot * 2 * d + 4 * n_hot


def hot_end_bytes(kind, d, count, n_hot):
    """The second launch: the predicted rows after the prefix, the list and x, y."""
    m = 1 if kind == "relu" else 2
    return (m + 1) * (count - n_hot) * 2 * d + 4 * (count - n_hot) + 4 * count + 4 * d


def sparse_bytes(kind, d, count):
    m = 1 if kind == "relu" else 2
    return (m + 1) * count * 2 * d + 4 * count + 8 * count + 2 * d + 4 * d


def dense_bytes(kind, d, ffn):
    m = 1 if kind == "relu" else 2
    return (m + 1) * ffn * 2 * d + 4 * ffn + 2 * d + 4 * d


def percentiles(vals, qs=(10, 50, 90)):
    v = sorted(vals)
    n = len(v)
    return {f"p{q}": v[min(n - 1, (q * n) // 100)] for q in qs}


class GraphTimer:
    """Captures a callable into a HIP graph on a side stream and times replays
    between HIP events recorded on that same stream."""

    def __init__(self, fn, warm=1):
        import torch
        self.torch = torch
        self.stream = torch.cuda.Stream()
        self.stream.wait_stream(torch.cuda.current_stream())
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            for _ in range(warm):
                fn()
            self.stream.synchronize()
            with torch.cuda.graph(self.graph, stream=self.stream):
                fn()
        torch.cuda.synchronize()

    def time(self, reps):
        """Mean ms per replay over reps replays (one warm replay first)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            self.graph.replay()
            e0.record(self.stream)
            for _ in range(reps):
                self.graph.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def release(self):
        del self.graph


def torch_dense_ffn(kind, L, x):
    """The dense FFN through torch's GEMMs (hipBLASLt), fp16 in, fp32 activations."""
    import torch
    F = torch.nn.functional
    if kind == "reglu":
        a = torch.relu(F.linear(x, L["W_gate"]).float() + L["b_gate"]) * F.linear(x, L["W_up"]).float()
    elif kind == "swiglu":
        a = F.silu(F.linear(x, L["W_gate"]).float() + L["b_gate"]) * F.linear(x, L["W_up"]).float()
    else:
        a = torch.relu(F.linear(x, L["W_up"]).float() + L["b_up"])
    return F.linear(a.half(), L["W_down"].t())


def cpu_baseline(cfg, layer_dev, tokens_dev, budget_s, what):
    """The oracle as it stands, timed on the host cores over a bounded token sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    H = {k: (v.detach().cpu() if hasattr(v, "detach") else v) for k, v in layer_dev.items()}
    X = tokens_dev.cpu()
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_step(H, X[n % X.shape[0]])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= X.shape[0]:
            break
    return {"value": n / el, "unit": "tokens/s per layer", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} decode tokens of {what} (float64 numpy oracle: predict + sparse FFN), {el:.1f} s"}


def hot_prefix_of(counts_sorted, calib_tokens):
    """Neurons that fired on >= 99 % of the calibration tokens, in whole 32-neuron words."""
    import numpy as np
    return 32 * (int(np.count_nonzero(counts_sorted >= 0.99 * calib_tokens)) // 32)


def build_hot_first(cfg, nl, dev, log_fn, label="stack"):
    """nl layers of cfg, each profiled on its calibration tokens, reordered
    hot-first and permuted; returns (layers, n_hot per layer, 80 % hot-set sizes)."""
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import make_calibration, make_layer
    t0 = time.perf_counter()
    layers, hots, hot80 = [], [], []
    for l in range(nl):
        L = make_layer(cfg, layer=l, device=dev)
        Wf, bf = (L["W_up"], L["b_up"]) if cfg.kind == "relu" else (L["W_gate"], L["b_gate"])
        counts = R.profile(make_calibration(cfg, device=dev, layer=l), Wf, bf).cpu().numpy()
        perm, hot = R.reorder(counts, 0.8)
        layers.append(R.permute_layer(L, torch.from_numpy(perm).to(dev)))
        hots.append(hot_prefix_of(counts[perm], cfg.calib_tokens))
        hot80.append(hot)
        del L
        if l % 16 == 15:
            torch.cuda.synchronize()
            log_fn(f"{label}: {l + 1} layers built, profiled and reordered ({time.perf_counter() - t0:.0f} s)")
    torch.cuda.synchronize()
    return layers, hots, hot80, time.perf_counter() - t0


def stack_headline(cfg, args, dev, log_fn):
    """The headline: decode steps of one token through the whole hot-first stack,
    one captured graph per step, plus its baselines and kernel times."""
    import numpy as np
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import make_tokens
    kind, d, r, ffn, NLs = cfg.kind, cfg.d, cfg.r, cfg.ffn, cfg.layers
    m = 1 if kind == "relu" else 2
    layers, hots, hot80, setup_s = build_hot_first(cfg, NLs, dev, log_fn)
    log_fn(f"stack: {NLs} layers ready in {setup_s:.1f} s; n_hot mean {np.mean(hots):.0f}, "
           f"80 % hot set mean {np.mean(hot80):.0f}")

    # ---- prompt: the prompt tokens of every layer at once (union path), one graph
    P = cfg.prompt_tokens
    Xp = [make_tokens(cfg, P, device=dev, layer=l, stream="prompt") for l in range(NLs)]
    idxp = torch.empty(P, ffn, dtype=torch.int32, device=dev)
    cntp = torch.empty(P, dtype=torch.int32, device=dev)
    yp = torch.empty(P, d, dtype=torch.float32, device=dev)

    def prompt_pass():
        for l in range(NLs):
            R.predict(layers[l], Xp[l], idxp, cntp, n_hot=hots[l])
            R.sparse(layers[l], Xp[l], idxp, cntp, yp)

    gp = GraphTimer(prompt_pass)
    prompt_ms = gp.time(2)
    gp.release()
    del Xp, idxp, yp
    log_fn(f"stack prompt: {P} tokens x {NLs} layers {prompt_ms:.2f} ms ({P * 1000.0 / prompt_ms:.0f} tok/s)")

    # ---- decode: one graph per step (one token through every layer)
    S = cfg.decode_steps
    K, W = args.steps, args.warmup
    ng = max(1, min(max(K, W), S))
    Xd = [make_tokens(cfg, S, device=dev, layer=l) for l in range(NLs)]
    xs = [[Xd[l][t:t + 1].contiguous() for t in range(ng)] for l in range(NLs)]
    del Xd
    idx = torch.empty(NLs, ffn, dtype=torch.int32, device=dev)    # each layer keeps its last list
    cnt = torch.empty(NLs, dtype=torch.int32, device=dev)
    y = torch.empty(NLs, d, dtype=torch.float32, device=dev)

    def layer_step(l, x):
        R.decode_hot(layers[l], x, hots[l], y[l:l + 1], idx[l:l + 1], cnt[l:l + 1])

    # list lengths of every (layer, token) the steps use, for the byte accounting
    counts = torch.empty(NLs, ng, dtype=torch.int32, device=dev)
    for t in range(ng):
        for l in range(NLs):
            R.predict(layers[l], xs[l][t], idx[l:l + 1], counts[l, t:t + 1], n_hot=hots[l])
    torch.cuda.synchronize()
    counts_h = counts.cpu().numpy()
    if counts_h.min() < 0:
        raise RuntimeError("the predictor reported an overrun (count -1)")
    T_layer = np.array([[touched_bytes(kind, d, r, ffn, int(counts_h[l, t]), hots[l]) for t in range(ng)]
                        for l in range(NLs)])

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(cs):
        for l in range(NLs):                     # eager pass: every workspace holds its layout
            layer_step(l, xs[l][0])
        cs.synchronize()
        for t in range(ng):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                for l in range(NLs):
                    layer_step(l, xs[l][t])
            graphs.append(g)
    torch.cuda.synchronize()
    log_fn(f"stack decode: {ng} step graphs captured ({NLs} layers each)")
    with torch.cuda.stream(cs):
        for k in range(W):
            graphs[k % ng].replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()                     # one process, one GPU: the barrier is the device sync
    with torch.cuda.stream(cs):
        ev[0].record(cs)
        for k in range(K):
            graphs[k % ng].replay()
            ev[k + 1].record(cs)
    torch.cuda.synchronize()
    step_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(K)]
    total_ms = ev[0].elapsed_time(ev[K])
    T_step = [float(T_layer[:, k % ng].sum()) for k in range(K)]
    layer_us = total_ms * 1000.0 / (K * NLs)
    T_mean = sum(T_step) / (K * NLs)
    value = K * NLs * 1000.0 / total_ms
    log_fn(f"stack decode: {K} steps x {NLs} layers in {total_ms:.2f} ms: {layer_us:.2f} us per layer step, "
           f"{value:.0f} tok/s/layer ({K * 1000.0 / total_ms:.1f} tok/s through the stack), "
           f"T {T_mean / 1e6:.1f} MB -> {T_mean / layer_us / 1e3:.0f} GB/s")
    del graphs

    # ---- per kernel: the step's two launches as separate entry points
    # (pi_ffn_decode_hot_begin, pi_ffn_decode_hot_end), one workspace per layer;
    # a graph of one launch per layer, back to back, for each
    reps = 10
    wss = [R.hot_workspace(layers[l]) for l in range(NLs)]

    def run_begin():
        for l in range(NLs):
            R.decode_hot_begin(layers[l], xs[l][0], hots[l], idx[l:l + 1], cnt[l:l + 1], ws=wss[l])

    def run_end():
        for l in range(NLs):
            R.decode_hot_end(layers[l], xs[l][0], hots[l], idx[l:l + 1], cnt[l:l + 1], y[l:l + 1], ws=wss[l])

    run_begin()
    torch.cuda.synchronize()
    c0 = cnt.cpu().numpy()
    g = GraphTimer(run_begin)
    ms_begin = g.time(reps) / NLs
    g.release()
    g = GraphTimer(run_end)
    ms_end = g.time(reps) / NLs
    g.release()
    bb = float(np.mean([hot_begin_bytes(kind, d, r, ffn, int(c0[l]), hots[l]) for l in range(NLs)]))
    eb = float(np.mean([hot_end_bytes(kind, d, int(c0[l]), hots[l]) for l in range(NLs)]))
    stages = {"pi_ffn_decode_hot_begin": (ms_begin, bb / ms_begin / 1e6, bb),
              "pi_ffn_decode_hot_end": (ms_end, eb / ms_end / 1e6, eb)}
    del wss
    log_fn(f"stack kernels: begin (predictor + hot prefix) {ms_begin * 1000:.2f} us "
           f"({stages['pi_ffn_decode_hot_begin'][1]:.0f} GB/s on {bb / 1e6:.1f} MB), end (FFN rest) "
           f"{ms_end * 1000:.2f} us ({stages['pi_ffn_decode_hot_end'][1]:.0f} GB/s on {eb / 1e6:.1f} MB) per launch")

    # ---- the same steps as two calls (pi_ffn_predict_hot + pi_ffn_sparse: the
    # prefix's rows gathered with the rest), for comparison
    def run_two_calls():
        for l in range(NLs):
            R.predict(layers[l], xs[l][0], idx[l:l + 1], cnt[l:l + 1], n_hot=hots[l])
            R.sparse(layers[l], xs[l][0], idx[l:l + 1], cnt[l:l + 1], y[l:l + 1])

    g = GraphTimer(run_two_calls)
    ms_two = g.time(reps) / NLs
    g.release()
    log_fn(f"stack: the same layer steps as pi_ffn_predict_hot + pi_ffn_sparse: {ms_two * 1000:.2f} us")

    # ---- dense baselines over the same layers, one token each, graph-timed
    dense = None
    if not args.no_dense:
        def run_dense():
            for l in range(NLs):
                R.sparse(layers[l], xs[l][0], None, None, y[l:l + 1], dense=True)

        def run_torch():
            for l in range(NLs):
                torch_dense_ffn(kind, layers[l], xs[l][0])

        g = GraphTimer(run_dense)
        ms_dense = g.time(3) / NLs
        g.release()
        g = GraphTimer(run_torch)
        ms_torch = g.time(3) / NLs
        g.release()
        db = dense_bytes(kind, d, ffn)
        ms_layer = layer_us / 1000.0
        dense = {"pi_dense_us": ms_dense * 1000, "pi_dense_GBs": db / ms_dense / 1e6,
                 "torch_dense_us": ms_torch * 1000, "torch_dense_GBs": db / ms_torch / 1e6,
                 "speedup_vs_pi_dense": ms_dense / ms_layer, "speedup_vs_torch_dense": ms_torch / ms_layer,
                 "ideal_speedup_1_over_active": ffn / float(counts_h.mean()),
                 "target_speedup_half_ideal": 0.5 * ffn / float(counts_h.mean()),
                 "method": f"graph of {NLs} launches (one per layer, one token each), replayed 3 times"}
        log_fn(f"stack dense: library {ms_dense * 1000:.1f} us ({db / ms_dense / 1e6:.0f} GB/s), torch "
               f"{ms_torch * 1000:.1f} us per layer; sparse step {ms_dense / ms_layer:.2f}x / "
               f"{ms_torch / ms_layer:.2f}x faster")

    out = {
        "value": value, "ms_per_step": total_ms / K, "layer_us": layer_us, "T_mean": T_mean,
        "step_us_percentiles": dict(percentiles([s * 1000.0 for s in step_ms]), steps=K,
                                    note="per step (one token through all layers) from HIP events between "
                                         "consecutive graph replays"),
        "layer_step_us_percentiles": percentiles([s * 1000.0 / NLs for s in step_ms]),
        "stages": stages, "dense": dense,
        "info": {"layers": NLs, "setup_s": setup_s, "n_hot_mean": float(np.mean(hots)),
                 "hot80_mean": float(np.mean(hot80)), "mean_active": float(counts_h.mean()),
                 "resident_GB": NLs * ((m + 1) * ffn * d * 2 + r * d * 2 + ffn * r * 2) / 1e9,
                 "step_graphs": ng,
                 "entry_point": "pi_ffn_decode_hot (the prefix's FFN beside the predictor)",
                 "two_calls_us_per_layer_step": ms_two * 1000,
                 "prompt": {"tokens": P, "ms": prompt_ms, "tokens_per_s": P * 1000.0 / prompt_ms,
                            "us_per_layer": prompt_ms * 1000.0 / NLs, "method": "one graph of all layers"},
                 "decode_tokens_per_s": K * 1000.0 / total_ms},
        "cpu_layer": None,
    }
    if not args.no_cpu:
        out["cpu_layer"] = (layers[0], make_tokens(cfg, 64, device=dev, layer=0))
    del layers, xs
    return out


def layer_line(cfg_key, nl, nt, reps, no_dense, log_fn):
    """Single-token steps of one layer shape, cache-cold over nl rotated layers:
    a graph of nl x min(nt, 8) steps replayed, per-entry-point graphs, and the
    dense baselines graph-timed the same way."""
    import numpy as np
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_layer, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    dev = torch.device("cuda:0")
    layers = [make_layer(cfg, layer=l, device=dev) for l in range(nl)]
    toks = [make_tokens(cfg, nt, device=dev, layer=l) for l in range(nl)]
    xs = [[toks[l][t:t + 1].contiguous() for t in range(nt)] for l in range(nl)]
    Kg = nl * max(1, min(nt, 8))
    lt = [(s % nl, (s // nl) % nt) for s in range(Kg)]
    idx_g = torch.empty(Kg, ffn, dtype=torch.int32, device=dev)
    cnt_g = torch.empty(Kg, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)

    def steps():
        for s, (l, t) in enumerate(lt):
            R.predict(layers[l], xs[l][t], idx_g[s:s + 1], cnt_g[s:s + 1])
            R.sparse(layers[l], xs[l][t], idx_g[s:s + 1], cnt_g[s:s + 1], y)

    def run_pred():
        for s, (l, t) in enumerate(lt):
            R.predict(layers[l], xs[l][t], idx_g[s:s + 1], cnt_g[s:s + 1])

    def run_sparse():
        for s, (l, t) in enumerate(lt):
            R.sparse(layers[l], xs[l][t], idx_g[s:s + 1], cnt_g[s:s + 1], y)

    g = GraphTimer(steps)
    ms_step = g.time(reps) / Kg
    g.release()
    c = cnt_g.cpu().numpy()
    T = float(np.mean([touched_bytes(kind, d, r, ffn, int(v)) for v in c]))
    g = GraphTimer(run_pred)
    ms_pred = g.time(reps) / Kg
    g.release()
    g = GraphTimer(run_sparse)
    ms_sp = g.time(reps) / Kg
    g.release()
    pb = predict_bytes(d, r, ffn, float(c.mean()))
    sb = float(np.mean([sparse_bytes(kind, d, int(v)) for v in c]))
    out = {"workload": cfg.workload, "layers_rotated": nl, "mean_active": float(c.mean()),
           "us_per_step": ms_step * 1000, "tokens_per_s_per_layer": 1000.0 / ms_step, "touched_MB": T / 1e6,
           "GBs": T / ms_step / 1e6, "step_frac": T / ms_step / 1e6 / HBM_PEAK_GBS,
           "kernels_us": {"pi_ffn_predict": ms_pred * 1000, "pi_ffn_sparse": ms_sp * 1000},
           "kernels_GBs": {"pi_ffn_predict": pb / ms_pred / 1e6, "pi_ffn_sparse": sb / ms_sp / 1e6},
           "method": f"graph of {Kg} steps over {nl} rotated layers, replayed {reps} times"}
    log_fn(f"{cfg_key} layer: {ms_step * 1000:.2f} us per step, {1000.0 / ms_step:.0f} tok/s/layer, "
           f"T {T / 1e6:.1f} MB -> {T / ms_step / 1e6:.0f} GB/s; predict {ms_pred * 1000:.2f} us, "
           f"sparse {ms_sp * 1000:.2f} us")
    if not no_dense:
        def run_dense():
            for s, (l, t) in enumerate(lt):
                R.sparse(layers[l], xs[l][t], None, None, y, dense=True)

        def run_torch():
            for s, (l, t) in enumerate(lt):
                torch_dense_ffn(kind, layers[l], xs[l][t])

        g = GraphTimer(run_dense)
        ms_dense = g.time(2) / Kg
        g.release()
        g = GraphTimer(run_torch)
        ms_torch = g.time(2) / Kg
        g.release()
        db = dense_bytes(kind, d, ffn)
        out["dense"] = {"pi_dense_us": ms_dense * 1000, "pi_dense_GBs": db / ms_dense / 1e6,
                        "torch_dense_us": ms_torch * 1000, "speedup_vs_pi_dense": ms_dense / ms_step,
                        "speedup_vs_torch_dense": ms_torch / ms_step,
                        "ideal_speedup_1_over_active": ffn / float(c.mean())}
        log_fn(f"{cfg_key} dense: library {ms_dense * 1000:.1f} us, torch {ms_torch * 1000:.1f} us; "
               f"{ms_dense / ms_step:.2f}x / {ms_torch / ms_step:.2f}x")
    del layers, toks, xs
    torch.cuda.empty_cache()
    return out


def profile_run(cfg, nl, dev):
    """The workload the hardware-counter passes run: nl hot-first layers of the
    stack (profiled, reordered), 2 warm-up and 8 counted hot decode steps
    (pi_ffn_decode_hot) per layer, then identity row copies of a known size
    whose FETCH_SIZE / WRITE_SIZE calibrate the counters."""
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import make_tokens
    layers, hots, _, _ = build_hot_first(cfg, nl, dev, log)
    d, ffn = cfg.d, cfg.ffn
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    toks = [make_tokens(cfg, 8, device=dev, layer=l) for l in range(nl)]
    counts = []
    for s in range(nl * 2 + nl * 8):
        l, t = s % nl, (s // nl) % 8
        x = toks[l][t:t + 1].contiguous()
        R.decode_hot(layers[l], x, hots[l], y, idx, cnt)
        if s >= nl * 2:
            counts.append(cnt.clone())
    torch.cuda.synchronize()
    rows, row_bytes = 1 << 16, 4096   # 256 MiB
    src = torch.ones(rows * row_bytes // 2, dtype=torch.float16, device=dev).view(rows, row_bytes // 2)
    perm = torch.arange(rows, dtype=torch.int32, device=dev)
    for _ in range(4):
        R.permute_rows(src, perm)
    torch.cuda.synchronize()
    c = torch.cat(counts).float()
    print(json.dumps({"profile_run": {"workload": cfg.workload, "layers": nl, "decode_steps": len(counts),
                                      "mean_count": float(c.mean()), "n_hot": hots,
                                      "copy_bytes_read": rows * row_bytes, "copy_bytes_written": rows * row_bytes,
                                      "copies": 4}}), flush=True)


def hot_prefix_line(cfg_key, nl, ntok, reps, log_fn):
    """Single-token steps on hot-first layers with the always-listed prefix
    (pi_ffn_predict_hot) against the same layers with the plain predictor.
    Graph-timed, nl rotated layers."""
    import numpy as np
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    dev = torch.device("cuda:0")
    layers, hots, _, _ = build_hot_first(cfg, nl, dev, log_fn, label="hot")
    xs = [[make_tokens(cfg, ntok, device=dev, layer=l)[t:t + 1].contiguous() for t in range(ntok)]
          for l in range(nl)]
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    K = nl * ntok
    out = {"workload": cfg.workload + " hot-first", "n_hot_mean": float(np.mean(hots)),
           "calibration_tokens": cfg.calib_tokens}
    for name, use_hot in (("plain", False), ("hot_prefix", True)):
        def run():
            for s in range(K):
                l, t = s % nl, (s // nl) % ntok
                R.predict(layers[l], xs[l][t], idx, cnt, n_hot=hots[l] if use_hot else 0)
                R.sparse(layers[l], xs[l][t], idx, cnt, y)
        counts = []
        for s in range(K):
            l, t = s % nl, (s // nl) % ntok
            R.predict(layers[l], xs[l][t], idx, cnt, n_hot=hots[l] if use_hot else 0)
            counts.append(int(cnt.item()))
        g = GraphTimer(run)
        ms = g.time(reps) / K
        g.release()
        cmean = float(np.mean(counts))
        skipped = float(np.mean([hots[s % nl] for s in range(K)])) if use_hot else 0.0
        T = touched_bytes(kind, d, r, ffn, cmean, skipped)
        out[name] = {"us_per_step": ms * 1000, "tokens_per_s_per_layer": 1000.0 / ms, "mean_active": cmean,
                     "touched_MB": T / 1e6, "GBs": T / ms / 1e6}
        log_fn(f"{name:10s}: {ms * 1000:7.2f} us  {1000.0 / ms:8.0f} tok/s/layer  active {cmean:7.1f}  "
               f"T {T / 1e6:6.1f} MB  {T / ms / 1e6:6.0f} GB/s  (n_hot {np.mean(hots):.0f})")
    del layers, xs
    torch.cuda.empty_cache()
    return out


def q4_line(cfg_key, nl, ntok, reps, log_fn):
    """Single-token steps with INT4 FFN rows (pi_quantize_rows once per layer,
    then pi_ffn_predict + pi_ffn_sparse_q4 per step with the fp16 predictor,
    and pi_ffn_predict_q4 + pi_ffn_sparse_q4 with an INT4 predictor),
    graph-timed over nl rotated layers, beside the INT4 dense FFN."""
    import numpy as np
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_layer, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    m = 1 if kind == "relu" else 2
    dev = torch.device("cuda:0")
    layers = []
    for l in range(nl):
        L = make_layer(cfg, layer=l, device=dev)
        Q = R.quantize_layer(L)
        for k in ("W_up", "W_gate", "W_down"):
            L.pop(k, None)
        Q.update({k: v for k, v in L.items() if k not in Q})
        layers.append(Q)
    xs = [[make_tokens(cfg, ntok, device=dev, layer=l)[t:t + 1].contiguous() for t in range(ntok)]
          for l in range(nl)]
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    K = nl * ntok
    predictors = {"fp16": R.predict, "int4": R.predict_q4}
    counts = {}
    for pk, pf in predictors.items():
        counts[pk] = []
        for s in range(K):
            l, t = s % nl, (s // nl) % ntok
            pf(layers[l], xs[l][t], idx, cnt)
            counts[pk].append(int(cnt.item()))
    out = {"workload": cfg.workload + " int4 rows (group 64)"}
    for name, pk in (("sparse", "fp16"), ("sparse_int4_predictor", "int4"), ("dense", None)):
        dense = pk is None

        def run():
            for s in range(K):
                l, t = s % nl, (s // nl) % ntok
                if not dense:
                    predictors[pk](layers[l], xs[l][t], idx, cnt)
                R.sparse_q4(layers[l], xs[l][t], idx, cnt, y, dense=dense)
        g = GraphTimer(run)
        ms = g.time(reps) / K
        g.release()
        row = d // 2 + d // 32
        if dense:
            T = (m + 1) * ffn * row + 4 * ffn + 6 * d
        else:
            c = float(np.mean(counts[pk]))
            Pb = 2 * r * d + 2 * ffn * r if pk == "fp16" else r * (d // 2 + d // 32) + ffn * (r // 2 + r // 32)
            T = Pb + 4 * ffn + (m + 1) * c * row + 4 * c + 6 * d + 8 * c
        out[name] = {"us_per_step": ms * 1000, "tokens_per_s_per_layer": 1000.0 / ms, "touched_MB": T / 1e6,
                     "GBs": T / ms / 1e6}
        if not dense:
            out[name]["mean_active"] = float(np.mean(counts[pk]))
        log_fn(f"int4 {name:21s}: {ms * 1000:7.2f} us  {1000.0 / ms:8.0f} tok/s/layer  T {T / 1e6:6.1f} MB  "
               f"{T / ms / 1e6:6.0f} GB/s")
    del layers, xs
    torch.cuda.empty_cache()
    return out


def batch_sweep(cfg_key, batches, reps, nl, log_fn):
    """Decode steps of B tokens on the union path, cache-cold over nl layers,
    graph-timed, beside torch's dense GEMMs for the same B tokens."""
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_layer, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    m = 1 if kind == "relu" else 2
    dev = torch.device("cuda:0")
    layers = [make_layer(cfg, layer=l, device=dev) for l in range(nl)]
    out = []
    for Bt in batches:
        X = [make_tokens(cfg, Bt, device=dev, layer=l, stream="prompt" if Bt >= 64 else "decode")
             for l in range(nl)]
        idx = torch.empty(Bt, ffn, dtype=torch.int32, device=dev)
        cnt = torch.empty(Bt, dtype=torch.int32, device=dev)
        y = torch.empty(Bt, d, dtype=torch.float32, device=dev)
        usize = []   # union sizes for the byte accounting (host side, once per layer)
        for l in range(nl):
            R.predict(layers[l], X[l], idx, cnt)
            torch.cuda.synchronize()
            c = cnt.cpu().tolist()
            ih = idx.cpu()
            sel = torch.zeros(ffn, dtype=torch.bool)
            for t in range(Bt):
                sel[ih[t, :c[t]].long()] = True
            usize.append(int(sel.sum()))

        def run():
            for l in range(nl):
                R.predict(layers[l], X[l], idx, cnt)
                R.sparse(layers[l], X[l], idx, cnt, y)

        def run_torch():
            for l in range(nl):
                torch_dense_ffn(kind, layers[l], X[l])

        g = GraphTimer(run)
        ms = g.time(reps) / nl
        g.release()
        g = GraphTimer(run_torch)
        ms_dense = g.time(max(2, reps // 2)) / nl
        g.release()
        U = sum(usize) / nl
        T = 2 * r * d + 2 * ffn * r + 4 * ffn + (m + 1) * U * 2 * d + 4 * U + Bt * (2 * d + 4 * d)
        row = {"batch": Bt, "us_per_step": ms * 1000, "tokens_per_s_per_layer": Bt * 1000 / ms,
               "union_rows": U, "touched_MB": T / 1e6, "GBs": T / ms / 1e6,
               "torch_dense_us": ms_dense * 1000, "speedup_vs_torch_dense": ms_dense / ms}
        log_fn(f"batch {Bt:3d}: {ms * 1000:8.1f} us  {Bt * 1000 / ms:9.0f} tok/s/layer  |U| {U:8.0f}  "
               f"T {T / 1e6:6.1f} MB  {T / ms / 1e6:6.0f} GB/s  torch dense {ms_dense * 1000:7.1f} us")
        out.append(row)
    del layers
    torch.cuda.empty_cache()
    return {"workload": cfg.workload, "method": f"graph of one step per layer over {nl} rotated layers",
            "rows": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed decode steps (one token through every layer)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="c5", help="headline workload (the layer stack)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--layer", default="c2", help="config of the single-layer rotation line ('' to skip)")
    ap.add_argument("--sweep", default="c4", help="config of the batch sweep ('' to skip)")
    ap.add_argument("--sweep-batches", default="1,4,8,16,32")
    ap.add_argument("--hot", default="c2", help="config of the hot-prefix line ('' to skip)")
    ap.add_argument("--q4", default="c2", help="config of the INT4-rows line ('' to skip)")
    ap.add_argument("--prompt", default="c5",
                    help="config of the prompt-phase line: one prompt batch per layer against torch ('' to skip)")
    ap.add_argument("--layer-only", action="store_true",
                    help="run only the single-layer rotation line (for a per-kernel profile of the B = 1 calls)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the batch sweep (for a per-kernel profile of the union path)")
    ap.add_argument("--profile-run", action="store_true",
                    help="short fixed workload for hardware counters: --profile-layers hot-first layers, one "
                         "rotation of decode steps, then 4 identity pi_permute_rows copies of 256 MiB")
    ap.add_argument("--profile-layers", type=int, default=8)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path shards by neuron across GPUs but "
              f"this build runs on a single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    from activation_sparse_predictor_amd import binding as B
    from synthetic import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.config]
    if args.sweep_only:
        sw = batch_sweep(args.sweep, [int(b) for b in args.sweep_batches.split(",")], 10, 4, log)
        print(json.dumps({"batch_sweep": sw}), flush=True)
        return
    if args.layer_only:
        print(json.dumps({"layer": layer_line(args.layer, 8, 8, 10, args.no_dense, log)}), flush=True)
        return
    if args.profile_run:
        profile_run(cfg, args.profile_layers, dev)
        return

    head = stack_headline(cfg, args, dev, log)
    cpu_layer = head.pop("cpu_layer")
    torch.cuda.empty_cache()
    dom = max(head["stages"], key=lambda k: head["stages"][k][0])
    st = head["stages"]

    layer = layer_line(args.layer, 8, 8, 10, args.no_dense, log) if args.layer else None
    sweep = batch_sweep(args.sweep, [int(b) for b in args.sweep_batches.split(",")], 10, 4, log) \
        if args.sweep else None
    hot = hot_prefix_line(args.hot, 8, 8, 10, log) if args.hot else None
    q4 = q4_line(args.q4, 8, 8, 10, log) if args.q4 else None
    # the prompt of a sequence against torch's dense GEMMs: 3 rotated layers
    prompt = batch_sweep(args.prompt, [CONFIGS[args.prompt].prompt_tokens or 128], 4, 3, log) \
        if args.prompt else None

    cpu = None
    if cpu_layer is not None:
        cpu = cpu_baseline(cfg, cpu_layer[0], cpu_layer[1], args.cpu_seconds,
                           f"layer 0 of the {cfg.workload} (hot-first order)")
        log(f"cpu oracle {cpu['value']:.2f} tok/s/layer on {cpu['cores']} threads")
        del cpu_layer

    out = {
        "metric": "sparse-FFN decode tokens/s per layer + achieved HBM GB/s on touched rows",
        "value": head["value"],
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.workload, "kind": cfg.kind, "d": cfg.d, "ffn": cfg.ffn, "r": cfg.r,
                   "layers": cfg.layers, "batch": 1, "tau": cfg.tau, "hot_first": True,
                   "step": f"one decode token through all {cfg.layers} layers (predict + sparse FFN per layer)",
                   "value_is": f"{cfg.layers} x steps / elapsed (tokens/s per layer)",
                   "mean_active": head["info"]["mean_active"], "n_hot_mean": head["info"]["n_hot_mean"],
                   "touched_MB_per_layer_step": head["T_mean"] / 1e6},
        "us_per_layer_step": head["layer_us"],
        "achieved_GBs_step": head["T_mean"] / head["layer_us"] / 1e3,
        "timing": {"method": "one captured HIP graph per step (all layers); steps replayed back to back "
                             "between HIP events on the graphs' stream, device-synchronised on both sides",
                   "step_us_percentiles": head["step_us_percentiles"],
                   "layer_step_us_percentiles": head["layer_step_us_percentiles"]},
        "roofline": {"bound": "hbm", "kernel": KERNEL_OF[dom], "entry_point": dom, "achieved": st[dom][1],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": st[dom][1] / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.config, dom),
                     "bytes_per_launch": st[dom][2],
                     "step_frac": head["T_mean"] / head["layer_us"] / 1e3 / HBM_PEAK_GBS,
                     "stages_us": {k: v[0] * 1000 for k, v in st.items()},
                     "stages_GBs": {k: v[1] for k, v in st.items()},
                     "stages_method": f"graph of {cfg.layers} back-to-back launches of one entry point "
                                      f"(one per layer, one workspace each), replayed 10 times between HIP "
                                      f"events on the graph's stream"},
        "dense_baseline": head["dense"],
        "cpu_baseline": cpu,
        "stack": head["info"],
        "layer_line": layer,
        "batch_sweep": sweep,
        "hot_prefix": hot,
        "int4_rows": q4,
        "prompt_phase": prompt,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
