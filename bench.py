#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X sparse-FFN path.

A step is one token through one layer: pi_ffn_predict (predictor MLP,
threshold, ordered compaction) then pi_ffn_sparse (gathered up GEMV +
activation, neuron-major W_down accumulate), inputs already resident in HBM.
The metric is decode tokens/s per layer, with achieved HBM GB/s on the bytes
the step must touch:

  T = 2 r d + 2 ffn r + 4 ffn            predictor weights + b2
    + (m + 1) count 2 d + 4 count        active rows of W_up [W_gate] W_down + bias
    + 2 d + 4 d + 8 count                x, y, index list write + read

with m = 1 (ReLU) or 2 (ReGLU) and count the step's own active count.

Cache-cold protocol: steps rotate over several distinct layers (default 8,
about 7 GB for the OPT-30B-shaped layer) so the 256 MB Infinity Cache cannot
hold a layer between its visits.  Timing uses HIP events on the stream the
library launches on.  The dense FFN (every neuron, no predictor) through the
same library, and torch's hipBLASLt GEMVs, are timed the same way.  The CPU
oracle (plain float64 numpy) is timed on a bounded sample of tokens.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the single-token kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes on the OPT-30B-shaped layer, each scaled by what the same
# counter reads for an identity pi_permute_rows copy of known size.  They hold
# for the kernel source with this SHA-256 prefix only; for any other source the
# bench reports traffic as null.
MEASURED_TRAFFIC = {
    # the sources the single-token kernels are built from, hashed in this order
    "sources": ["activation_sparse_predictor_amd/csrc/fused.hip", "activation_sparse_predictor_amd/csrc/common.hpp"],
    "sha256_16": "462d0538a95a109b",
    "config": "c2",
    "bytes_per_launch": {"pi_ffn_predict": 73.02e6, "pi_ffn_sparse": 84.63e6},
}


KERNEL_OF = {"pi_ffn_predict": "k_predict_fused", "pi_ffn_sparse": "k_sparse_fused"}   # one kernel each at B = 1


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
    import hashlib
    h = kernel_source_hash()
    if h is None:
        return None
    if h != MEASURED_TRAFFIC["sha256_16"] or config_key != MEASURED_TRAFFIC["config"]:
        return None
    return MEASURED_TRAFFIC["bytes_per_launch"].get(entry)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def touched_bytes(kind, d, r, ffn, count):
    m = 1 if kind == "relu" else 2
    return (2 * r * d + 2 * ffn * r + 4 * ffn + (m + 1) * count * 2 * d + 4 * count
            + 2 * d + 4 * d + 8 * count)


def dense_bytes(kind, d, ffn):
    m = 1 if kind == "relu" else 2
    return (m + 1) * ffn * 2 * d + 4 * ffn + 2 * d + 4 * d


def cpu_baseline(cfg, layer_dev, tokens_dev, budget_s):
    """The oracle as it stands, timed on the host cores over a bounded token sample."""
    import numpy as np
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
            "sample": f"{n} decode tokens of one {cfg.workload} layer (float64 numpy oracle: "
                      f"predict + sparse FFN), {el:.1f} s"}


def profile_run(layers, tokens, NL, NT, dev):
    """The workload the hardware-counter passes run: a few warm-up steps, one
    rotation of decode steps over every layer, then identity row copies of a
    known size whose FETCH_SIZE / WRITE_SIZE calibrate the counters."""
    import torch
    from activation_sparse_predictor_amd import runtime as R
    d, ffn = layers[0]["d"], layers[0]["ffn"]
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    counts = []
    for s in range(NL * 2 + NL * 8):
        l, t = s % NL, (s // NL) % NT
        x = tokens[l][t:t + 1].contiguous()
        R.predict(layers[l], x, idx, cnt)
        R.sparse(layers[l], x, idx, cnt, y)
        if s >= NL * 2:
            counts.append(cnt.clone())
    torch.cuda.synchronize()
    rows, row_bytes = 1 << 16, 4096   # 256 MiB
    src = torch.ones(rows * row_bytes // 2, dtype=torch.float16, device=dev).view(rows, row_bytes // 2)
    perm = torch.arange(rows, dtype=torch.int32, device=dev)
    for _ in range(4):
        R.permute_rows(src, perm)
    torch.cuda.synchronize()
    c = torch.cat(counts).float()
    print(json.dumps({"profile_run": {"decode_steps": len(counts), "mean_count": float(c.mean()),
                                      "copy_bytes_read": rows * row_bytes, "copy_bytes_written": rows * row_bytes,
                                      "copies": 4}}), flush=True)


def hot_prefix_line(cfg_key, nl, ntok, reps, log_fn):
    """Single-token steps on hot-first layers: each layer profiled on its 4096
    calibration tokens and reordered, the neurons that fired on >= 99 % of them
    (whole 32-neuron words) listed without the predictor (pi_ffn_predict_hot),
    against the same layers with the plain predictor.  Graph-timed, nl rotated
    layers."""
    import numpy as np
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_calibration, make_layer, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    dev = torch.device("cuda:0")
    layers, hots = [], []
    for l in range(nl):
        L = make_layer(cfg, layer=l, device=dev)
        Wf, bf = (L["W_up"], L["b_up"]) if kind == "relu" else (L["W_gate"], L["b_gate"])
        counts = R.profile(make_calibration(cfg, device=dev, layer=l), Wf, bf).cpu().numpy()
        perm, _ = R.reorder(counts, 0.8)
        P = R.permute_layer(L, torch.from_numpy(perm).to(dev))
        hots.append(32 * (int(np.count_nonzero(counts[perm] >= 0.99 * cfg.calib_tokens)) // 32))
        layers.append(P)
        del L
    xs = [[make_tokens(cfg, ntok, device=dev, layer=l)[t:t + 1].contiguous() for t in range(ntok)]
          for l in range(nl)]
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    K = nl * ntok
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            run()
            cs.synchronize()
            with torch.cuda.graph(g, stream=cs):
                run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * K)
        del g
        m = 1 if kind == "relu" else 2
        cmean = float(np.mean(counts))
        skipped = float(np.mean([hots[s % nl] for s in range(K)])) if use_hot else 0.0
        T = (2 * r * d + (ffn - skipped) * (2 * r + 4) + (m + 1) * cmean * 2 * d + 4 * cmean
             + 2 * d + 4 * d + 8 * cmean)
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
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            run()
            cs.synchronize()
            with torch.cuda.graph(g, stream=cs):
                run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * K)
        del g
        row = d // 2 + d // 32
        if dense:
            T = (m + 1) * ffn * row + 4 * ffn + 6 * d
        else:
            c = float(np.mean(counts[pk]))
            P = 2 * r * d + 2 * ffn * r if pk == "fp16" else r * (d // 2 + d // 32) + ffn * (r // 2 + r // 32)
            T = P + 4 * ffn + (m + 1) * c * row + 4 * c + 6 * d + 8 * c
        out[name] = {"us_per_step": ms * 1000, "tokens_per_s_per_layer": 1000.0 / ms, "touched_MB": T / 1e6,
                     "GBs": T / ms / 1e6}
        if not dense:
            out[name]["mean_active"] = float(np.mean(counts[pk]))
        log_fn(f"int4 {name:21s}: {ms * 1000:7.2f} us  {1000.0 / ms:8.0f} tok/s/layer  T {T / 1e6:6.1f} MB  "
               f"{T / ms / 1e6:6.0f} GB/s")
    del layers, xs
    torch.cuda.empty_cache()
    return out


def stack_run(cfg_key, log_fn):
    """The whole stack of the workload (64 OPT-66B-shaped layers, ~93 GB
    resident): every layer profiled on its calibration tokens and reordered
    hot-first, then the prompt (one batch of prompt tokens per layer, the
    union path) and the decode steps at batch 1 (predict + sparse per layer,
    graph-replayed one step at a time).  Inputs are independent per layer:
    x ~ N(0, I) for every (layer, token)."""
    import numpy as np
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_calibration, make_layer, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn, NLs = cfg.kind, cfg.d, cfg.r, cfg.ffn, cfg.layers
    P, S = cfg.prompt_tokens, cfg.decode_steps
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    layers, hot_counts = [], []
    for l in range(NLs):
        L = make_layer(cfg, layer=l, device=dev)
        Wf, bf = (L["W_up"], L["b_up"]) if kind == "relu" else (L["W_gate"], L["b_gate"])
        counts = R.profile(make_calibration(cfg, device=dev, layer=l), Wf, bf).cpu().numpy()
        perm, hot = R.reorder(counts, 0.8)
        layers.append(R.permute_layer(L, torch.from_numpy(perm).to(dev)))
        hot_counts.append(hot)
        del L
        if l % 16 == 15:
            torch.cuda.synchronize()
            log_fn(f"stack: {l + 1} layers built, profiled and reordered ({time.perf_counter() - t0:.0f} s)")
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # prompt: P tokens per layer at once
    Xp = [make_tokens(cfg, P, device=dev, layer=l, stream="prompt") for l in range(NLs)]
    idxp = torch.empty(P, ffn, dtype=torch.int32, device=dev)
    cntp = torch.empty(P, dtype=torch.int32, device=dev)
    yp = torch.empty(P, d, dtype=torch.float32, device=dev)
    for l in range(2):
        R.predict(layers[l], Xp[l], idxp, cntp)
        R.sparse(layers[l], Xp[l], idxp, cntp, yp)
    torch.cuda.synchronize()
    e0.record(stream)
    for l in range(NLs):
        R.predict(layers[l], Xp[l], idxp, cntp)
        R.sparse(layers[l], Xp[l], idxp, cntp, yp)
    e1.record(stream)
    torch.cuda.synchronize()
    prompt_ms = e0.elapsed_time(e1)
    del Xp
    # decode: S steps, each through every layer, batch 1
    Xd = [make_tokens(cfg, S, device=dev, layer=l) for l in range(NLs)]
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    xs = [[Xd[l][t:t + 1].contiguous() for t in range(S)] for l in range(NLs)]
    for l in range(NLs):
        R.predict(layers[l], xs[l][0], idx, cnt)
        R.sparse(layers[l], xs[l][0], idx, cnt, y)
    torch.cuda.synchronize()
    counts = []
    e0.record(stream)
    for t in range(S):
        for l in range(NLs):
            R.predict(layers[l], xs[l][t], idx, cnt)
            R.sparse(layers[l], xs[l][t], idx, cnt, y)
    e1.record(stream)
    torch.cuda.synchronize()
    decode_ms = e0.elapsed_time(e1)
    for l in range(0, NLs, 8):
        R.predict(layers[l], xs[l][0], idx, cnt)
        counts.append(int(cnt.item()))
    m = 1 if kind == "relu" else 2
    out = {"workload": cfg.workload, "layers": NLs,
           "resident_GB": NLs * ((m + 1) * ffn * d * 2 + r * d * 2 + ffn * r * 2) / 1e9,
           "setup_s": setup_s, "hot_count_mean": float(np.mean(hot_counts)),
           "prompt": {"tokens": P, "ms": prompt_ms, "tokens_per_s": P * 1000.0 / prompt_ms,
                      "us_per_layer": prompt_ms * 1000.0 / NLs},
           "decode": {"steps": S, "ms": decode_ms, "tokens_per_s": S * 1000.0 / decode_ms,
                      "us_per_layer_step": decode_ms * 1000.0 / (S * NLs),
                      "sampled_active_mean": float(np.mean(counts)),
                      "method": "eager calls, HIP events around all steps"}}
    log_fn(f"stack: prompt {P} tokens x {NLs} layers {prompt_ms:.1f} ms ({P * 1000.0 / prompt_ms:.0f} tok/s); "
           f"decode {S} steps x {NLs} layers {decode_ms:.1f} ms ({S * 1000.0 / decode_ms:.1f} tok/s, "
           f"{decode_ms * 1000.0 / (S * NLs):.1f} us per layer step)")
    del layers, xs, Xd
    torch.cuda.empty_cache()
    return out


def batch_sweep(cfg_key, batches, steps, nl, log_fn):
    """Decode steps of B tokens on the union path, cache-cold over nl layers."""
    import torch
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_layer, make_tokens
    cfg = CONFIGS[cfg_key]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    m = 1 if kind == "relu" else 2
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    layers = [make_layer(cfg, layer=l, device=dev) for l in range(nl)]
    out = []
    F = torch.nn.functional
    for Bt in batches:
        X = [make_tokens(cfg, Bt, device=dev, layer=l) for l in range(nl)]
        idx = torch.empty(Bt, ffn, dtype=torch.int32, device=dev)
        cnt = torch.empty(Bt, dtype=torch.int32, device=dev)
        y = torch.empty(Bt, d, dtype=torch.float32, device=dev)
        # union sizes for the byte accounting (host side, once per layer)
        usize = []
        for l in range(nl):
            R.predict(layers[l], X[l], idx, cnt)
            torch.cuda.synchronize()
            c = cnt.cpu().tolist()
            ih = idx.cpu()
            sel = torch.zeros(ffn, dtype=torch.bool)
            for t in range(Bt):
                sel[ih[t, :c[t]].long()] = True
            usize.append(int(sel.sum()))
        for s in range(10):
            R.predict(layers[s % nl], X[s % nl], idx, cnt)
            R.sparse(layers[s % nl], X[s % nl], idx, cnt, y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            R.predict(layers[s % nl], X[s % nl], idx, cnt)
            R.sparse(layers[s % nl], X[s % nl], idx, cnt, y)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        U = sum(usize[s % nl] for s in range(steps)) / steps
        T = 2 * r * d + 2 * ffn * r + 4 * ffn + (m + 1) * U * 2 * d + 4 * U + Bt * (2 * d + 4 * d)
        # dense reference: torch GEMMs over every neuron for the same B tokens
        def torch_dense(L, x):
            if kind == "reglu":
                a = torch.relu(F.linear(x, L["W_gate"]).float() + L["b_gate"]) * F.linear(x, L["W_up"]).float()
            elif kind == "swiglu":
                a = F.silu(F.linear(x, L["W_gate"]).float() + L["b_gate"]) * F.linear(x, L["W_up"]).float()
            else:
                a = torch.relu(F.linear(x, L["W_up"]).float() + L["b_up"])
            return F.linear(a.half(), L["W_down"].t())
        for s in range(5):
            torch_dense(layers[s % nl], X[s % nl])
        torch.cuda.synchronize()
        e0.record(stream)
        kd = max(10, steps // 4)
        for s in range(kd):
            torch_dense(layers[s % nl], X[s % nl])
        e1.record(stream)
        torch.cuda.synchronize()
        ms_dense = e0.elapsed_time(e1) / kd
        row = {"batch": Bt, "us_per_step": ms * 1000, "tokens_per_s_per_layer": Bt * 1000 / ms,
               "union_rows": U, "touched_MB": T / 1e6, "GBs": T / ms / 1e6,
               "torch_dense_us": ms_dense * 1000, "speedup_vs_torch_dense": ms_dense / ms}
        log_fn(f"batch {Bt:3d}: {ms * 1000:8.1f} us  {Bt * 1000 / ms:9.0f} tok/s/layer  |U| {U:8.0f}  "
               f"T {T / 1e6:6.1f} MB  {T / ms / 1e6:6.0f} GB/s  torch dense {ms_dense * 1000:7.1f} us")
        out.append(row)
    del layers
    torch.cuda.empty_cache()
    return {"workload": cfg.workload, "rows": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--layers", type=int, default=8, help="distinct layer copies in the rotation")
    ap.add_argument("--tokens", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--sweep", default="c4", help="config of the batch sweep ('' to skip)")
    ap.add_argument("--sweep-batches", default="1,4,8,16,32")
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--hot", default="c2",
                    help="config of the hot-prefix line: hot-first layers, predictor trimmed ('' to skip)")
    ap.add_argument("--q4", default="c2", help="config of the INT4-rows line ('' to skip)")
    ap.add_argument("--stack", default="", help="also run a whole layer stack (c5: 64 layers, ~93 GB), "
                                                "prompt then decode; off by default")
    ap.add_argument("--prompt", default="c5",
                    help="config of the prompt-phase line: one 128-token batch per layer ('' to skip)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the batch sweep (for a per-kernel profile of the union path)")
    ap.add_argument("--profile-run", action="store_true",
                    help="short fixed workload for hardware counters: one rotation of decode steps, "
                         "then 4 identity pi_permute_rows copies of 256 MiB (the calibration copy)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path shards by neuron across GPUs but "
              f"this build runs on a single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from activation_sparse_predictor_amd import binding as B
    from activation_sparse_predictor_amd import runtime as R
    from synthetic import CONFIGS, make_layer, make_tokens

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep_only:
        sw = batch_sweep(args.sweep, [int(b) for b in args.sweep_batches.split(",")], args.sweep_steps, 4, log)
        print(json.dumps({"batch_sweep": sw}), flush=True)
        return
    cfg = CONFIGS[args.config]
    kind, d, r, ffn = cfg.kind, cfg.d, cfg.r, cfg.ffn
    NL, NT = args.layers, args.tokens
    t_gen = time.perf_counter()
    layers = [make_layer(cfg, layer=l, device=dev) for l in range(NL)]
    tokens = [make_tokens(cfg, NT, device=dev, layer=l) for l in range(NL)]
    torch.cuda.synchronize()
    log(f"generated {NL} x {cfg.workload} in {time.perf_counter() - t_gen:.1f} s")

    stream = torch.cuda.current_stream()
    if args.profile_run:
        profile_run(layers, tokens, NL, NT, dev)
        return
    idx = torch.empty(1, ffn, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    xs = [[tokens[l][t:t + 1].contiguous() for t in range(NT)] for l in range(NL)]

    def step(s):
        l, t = s % NL, (s // NL) % NT
        L = layers[l]
        R.predict(L, xs[l][t], idx, cnt)
        R.sparse(L, xs[l][t], idx, cnt, y)

    # active counts of every (layer, token) in the rotation, for the byte accounting
    counts = torch.empty(NL, NT, dtype=torch.int32, device=dev)
    for l in range(NL):
        for t in range(NT):
            R.predict(layers[l], xs[l][t], idx, counts[l, t:t + 1])
    torch.cuda.synchronize()
    counts_h = counts.cpu()
    if int(counts_h.min()) < 0:
        raise RuntimeError("compaction reported an error count")

    def steps_bytes(s0, K):
        tot = 0
        for s in range(s0, s0 + K):
            tot += touched_bytes(kind, d, r, ffn, int(counts_h[s % NL, (s // NL) % NT]))
        return tot

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0 = args.warmup

    # Eager: one host call per entry point per step.
    e0.record(stream)
    for s in range(s0, s0 + args.steps):
        step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps

    # Graph: one rotation of steps (every layer, several tokens each) captured
    # once and replayed, so the timed region holds only the GPU work of the
    # steps (the library's kernels take their launch epoch from the workspace,
    # so replays are valid).  This is the headline number.
    Kg = NL * max(1, min(NT, 8))
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        for s in range(Kg):
            step(s)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for s in range(Kg):
                step(s)
    torch.cuda.synchronize()
    reps = max(1, (args.steps + Kg - 1) // Kg)
    for _ in range(max(1, args.warmup // Kg)):
        graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    n_graph = reps * Kg
    ms_step = e0.elapsed_time(e1) / n_graph
    T_avg = steps_bytes(0, Kg) / Kg
    value = 1000.0 / ms_step
    log(f"step {ms_step * 1000:.2f} us (graph; eager {ms_eager * 1000:.2f} us), {value:.0f} tok/s/layer, "
        f"T {T_avg / 1e6:.1f} MB -> {T_avg / ms_step / 1e6:.0f} GB/s")
    del graph

    # The same steps through pi_ffn_decode (one call per step), graph-timed.
    def dstep(s):
        l, t = s % NL, (s // NL) % NT
        R.decode(layers[l], xs[l][t], y, idx, cnt)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for s in range(Kg):
            dstep(s)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for s in range(Kg):
                dstep(s)
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup // Kg)):
        graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_decode = e0.elapsed_time(e1) / n_graph
    del graph
    log(f"decode step (pi_ffn_decode) {ms_decode * 1000:.2f} us, {1000.0 / ms_decode:.0f} tok/s/layer")

    # Per entry point: a graph of Kg back-to-back launches of that entry point
    # alone (rotating layers and tokens as above), replayed between HIP events
    # on the launching stream, so that the average covers the kernel itself
    # and not the host's launch gap.  The sparse launches read the lists the
    # predict launches wrote, one list per step.
    idx_g = torch.empty(Kg, ffn, dtype=torch.int32, device=dev)
    cnt_g = torch.empty(Kg, dtype=torch.int32, device=dev)
    lt = [(s % NL, (s // NL) % NT) for s in range(Kg)]

    def run_pred():
        for s, (l, t) in enumerate(lt):
            R.predict(layers[l], xs[l][t], idx_g[s:s + 1], cnt_g[s:s + 1])

    def run_sparse():
        for s, (l, t) in enumerate(lt):
            R.sparse(layers[l], xs[l][t], idx_g[s:s + 1], cnt_g[s:s + 1], y)

    def graph_time(fn):
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            fn()
            cs.synchronize()
            with torch.cuda.graph(g, stream=cs):
                fn()
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / (reps * Kg)

    run_pred()
    torch.cuda.synchronize()
    ms_pred = graph_time(run_pred)
    ms_sp = graph_time(run_sparse)
    pred_bytes = 2 * r * d + 2 * ffn * r + 4 * ffn + 2 * d
    m = 1 if kind == "relu" else 2
    sp_bytes = [(m + 1) * int(counts_h[l, t]) * (2 * d + 4) + 4 * d for (l, t) in lt]
    gbs_pred = pred_bytes / ms_pred / 1e6
    gbs_sp = statistics.mean(sp_bytes) / ms_sp / 1e6

    # the same, eagerly: HIP events between the two calls of each step (the
    # per-call figure includes the host's launch gap)
    K2 = min(args.steps, 400)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * K2)]
    for k in range(K2):
        s = s0 + k
        l, t = s % NL, (s // NL) % NT
        ev[3 * k].record(stream)
        R.predict(layers[l], xs[l][t], idx, cnt)
        ev[3 * k + 1].record(stream)
        R.sparse(layers[l], xs[l][t], idx, cnt, y)
        ev[3 * k + 2].record(stream)
    torch.cuda.synchronize()
    eager_steps = sorted(1000 * ev[3 * k].elapsed_time(ev[3 * k + 2]) for k in range(K2))
    pct = {f"p{q}": eager_steps[min(K2 - 1, (q * K2) // 100)] for q in (10, 50, 90)}
    eager_us = {"pi_ffn_predict": 1000 * statistics.mean(ev[3 * k].elapsed_time(ev[3 * k + 1]) for k in range(K2)),
                "pi_ffn_sparse": 1000 * statistics.mean(ev[3 * k + 1].elapsed_time(ev[3 * k + 2])
                                                        for k in range(K2))}
    log(f"predict {ms_pred * 1000:.2f} us ({gbs_pred:.0f} GB/s), sparse {ms_sp * 1000:.2f} us "
        f"({gbs_sp:.0f} GB/s) per launch in graphs; eager per call {eager_us['pi_ffn_predict']:.2f} / "
        f"{eager_us['pi_ffn_sparse']:.2f} us")

    stages = {"pi_ffn_predict": (ms_pred, gbs_pred, pred_bytes),
              "pi_ffn_sparse": (ms_sp, gbs_sp, statistics.mean(sp_bytes))}
    dom = max(stages, key=lambda k: stages[k][0])

    dense = None
    if not args.no_dense:
        Kd = min(args.steps, 200)
        for s in range(20):
            l = s % NL
            R.sparse(layers[l], xs[l][0], None, None, y, dense=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(Kd):
            l, t = s % NL, (s // NL) % NT
            R.sparse(layers[l], xs[l][t], None, None, y, dense=True)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_dense = e0.elapsed_time(e1) / Kd
        # torch hipBLASLt GEMVs of the same dense FFN (fp16 in, fp32 out via fp16 GEMM)
        F = torch.nn.functional
        def torch_dense(L, x):
            if kind == "reglu":
                a = torch.relu(F.linear(x, L["W_gate"], None).float() + L["b_gate"]) * F.linear(x, L["W_up"]).float()
            elif kind == "swiglu":
                a = F.silu(F.linear(x, L["W_gate"], None).float() + L["b_gate"]) * F.linear(x, L["W_up"]).float()
            else:
                a = torch.relu(F.linear(x, L["W_up"]).float() + L["b_up"])
            return F.linear(a.half(), L["W_down"].t())
        for s in range(10):
            torch_dense(layers[s % NL], xs[s % NL][0])
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(Kd):
            l, t = s % NL, (s // NL) % NT
            torch_dense(layers[l], xs[l][t])
        e1.record(stream)
        torch.cuda.synchronize()
        ms_torch = e0.elapsed_time(e1) / Kd
        db = dense_bytes(kind, d, ffn)
        dense = {"pi_dense_us": ms_dense * 1000, "pi_dense_GBs": db / ms_dense / 1e6,
                 "torch_dense_us": ms_torch * 1000, "speedup_vs_pi_dense": ms_dense / ms_step,
                 "speedup_vs_torch_dense": ms_torch / ms_step,
                 "ideal_speedup_1_over_active": ffn / float(counts_h.float().mean())}
        log(f"dense {ms_dense * 1000:.1f} us ({db / ms_dense / 1e6:.0f} GB/s), torch {ms_torch * 1000:.1f} us, "
            f"speedup {ms_dense / ms_step:.2f}x")

    sweep = None
    if args.sweep:
        del layers, tokens, xs
        torch.cuda.empty_cache()
        sweep = batch_sweep(args.sweep, [int(b) for b in args.sweep_batches.split(",")],
                            args.sweep_steps, 4, log)

    hot = None
    if args.hot:
        if not args.sweep:
            del layers, tokens, xs
        torch.cuda.empty_cache()
        hot = hot_prefix_line(args.hot, 8, 8, 16, log)

    stack = None
    if args.stack:
        if not args.sweep and not args.hot:
            del layers, tokens, xs
        torch.cuda.empty_cache()
        stack = stack_run(args.stack, log)

    q4 = None
    if args.q4:
        if not args.sweep and not args.hot and not args.stack:
            del layers, tokens, xs
        torch.cuda.empty_cache()
        q4 = q4_line(args.q4, 8, 8, 16, log)

    prompt = None
    if args.prompt:
        # the prompt of a sequence: 128 tokens through the union path at once,
        # 3 rotated layers (about 4.4 GB at the OPT-66B shape)
        torch.cuda.empty_cache()
        prompt = batch_sweep(args.prompt, [128], 40, 3, log)

    cpu = None
    if not args.no_cpu:
        cpu_layer = make_layer(cfg, layer=0, device=dev)
        cpu_tokens = make_tokens(cfg, NT, device=dev, layer=0)
        cpu = cpu_baseline(cfg, cpu_layer, cpu_tokens, args.cpu_seconds)
        log(f"cpu oracle {cpu['value']:.2f} tok/s/layer on {cpu['cores']} threads")

    out = {
        "metric": "sparse-FFN decode tokens/s per layer + achieved HBM GB/s on touched rows",
        "value": value,
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": n_graph,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 weights, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": cfg.workload, "kind": kind, "d": d, "ffn": ffn, "r": r,
                   "batch": 1, "tau": cfg.tau, "layers_rotated": NL, "tokens_per_layer": NT,
                   "mean_active": float(counts_h.float().mean()),
                   "touched_MB_per_step": T_avg / 1e6},
        "achieved_GBs_step": T_avg / ms_step / 1e6,
        "decode_call": {"us_per_step": ms_decode * 1000, "tokens_per_s_per_layer": 1000.0 / ms_decode,
                        "GBs": T_avg / ms_decode / 1e6},
        "timing": {"method": f"hipGraph of {Kg} steps replayed {reps} times, HIP events around the replays",
                   "ms_per_step_eager": ms_eager,
                   "step_us_eager_percentiles": dict(pct, steps=K2,
                                                     note="per step from HIP events around each eager "
                                                          "predict + sparse pair (launch gaps included)")},
        "roofline": {"bound": "hbm", "kernel": KERNEL_OF[dom], "entry_point": dom, "achieved": stages[dom][1],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": stages[dom][1] / HBM_PEAK_GBS, "traffic": measured_traffic(args.config, dom),
                     "step_frac": T_avg / ms_step / 1e6 / HBM_PEAK_GBS,
                     "stages_us": {k: v[0] * 1000 for k, v in stages.items()},
                     "stages_method": f"graph of {Kg} back-to-back launches of one entry point, "
                                      f"replayed {reps} times between HIP events",
                     "stages_us_eager_per_call": eager_us},
        "dense_baseline": dense,
        "cpu_baseline": cpu,
        "batch_sweep": sweep,
        "hot_prefix": hot,
        "int4_rows": q4,
        "stack": stack,
        "prompt_phase": prompt,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
