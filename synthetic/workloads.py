"""Synthetic power-law-sparse FFN layers, predictors and tokens.

The pages measure PowerInfer on trained OPT / LLaMA2 / Falcon checkpoints,
profiled on C4 and Wikipedia and driven by ChatGPT-prompts, Alpaca and
Chatbot-Arena inputs (PowerInfer reading report, Part A section 2.2).  None of
those are available, so these seeded stand-ins reproduce the statistics the
pages state instead:

* a skewed (power-law) firing distribution in which a minority of neurons
  carries 80% of all activations (Part A section 3.1, finding 1: 17% for
  OPT-30B, 26% for LLaMA2(ReGLU)-70B);
* ReLU-family sparsity, i.e. most neurons are zero for a given token
  (Part A section 4.3).

Construction (all of it input preparation, none of it the method):

* every weight row is drawn N(0, 1) and scaled to unit L2 norm in fp32, then
  rounded to fp16;
* firing probabilities follow f_k = clip(c * k**-s, 1e-4, 0.999) over rank
  k = 1..ffn, with c chosen for the configured mean activity and s either
  given or solved so the top-q fraction of neurons carries 80% of sum(f);
* ranks are scattered over neurons by a seeded permutation, so an offline
  profile + reorder has real work to do;
* the bias on the ReLU input is b_i = Phi^-1(f_i): with a unit-norm row and a
  token x ~ N(0, I), w_i.x ~ N(0, 1), hence P(w_i.x + b_i > 0) = f_i exactly
  (up to fp16 rounding of the row);
* the predictor is d -> r -> ffn with a ReLU hidden layer, unit-norm rows and
  an output bias chosen so that P(z_i > 0) ~= f_i when the hidden units are
  treated as i.i.d. ReLU(N(0, 1)) (mean 1/sqrt(2 pi), variance
  1/2 - 1/(2 pi)); with tau = 0.5 the decision threshold on z is 0.  The
  predicted set is statistically independent of the true one given f, which
  fixes the active count (the quantity that sets the cost) but not accuracy.

Seeds follow one scheme: tensor seed = 1000*k + tensor_id + 100000*layer,
with k the config number (1..5) and tensor ids W_up 1, W_gate 2, W_down 3,
P1 4, P2 5, rank permutation 6, calibration tokens 7, decode tokens 8.
Weights are drawn with torch generators on the requested device: CPU and GPU
streams differ, so a run hands the same tensors to both sides it compares.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch
from scipy.special import ndtri

TENSOR_IDS = {
    "W_up": 1,
    "W_gate": 2,
    "W_down": 3,
    "P1": 4,
    "P2": 5,
    "rank_perm": 6,
    "calib": 7,
    "decode": 8,
    "prompt": 9,
}

# hidden-unit moments of ReLU(N(0,1)): mean 1/sqrt(2*pi), variance 1/2 - 1/(2*pi)
RELU_NORMAL_MEAN = 1.0 / math.sqrt(2.0 * math.pi)
RELU_NORMAL_VAR = 0.5 - 1.0 / (2.0 * math.pi)


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    key: str            # "c1".."c5" or "custom"
    number: int         # k in the seed scheme
    workload: str       # human-readable name with the model shape it mimics
    kind: str           # "relu", "reglu" or "swiglu"
    d: int              # hidden size
    ffn: int            # FFN neurons
    r: int              # predictor rank
    mean: float         # mean firing probability
    exponent: Optional[float]   # power-law exponent s, or None to solve it
    hot_quantile: Optional[float]  # fraction of neurons that carries hot_share
    hot_share: float = 0.80
    tau: float = 0.5
    batches: tuple = (1,)
    tokens: int = 64
    layers: int = 1
    calib_tokens: int = 4096
    prompt_tokens: int = 0
    decode_steps: int = 0


CONFIGS: Dict[str, WorkloadConfig] = {
    "c1": WorkloadConfig("c1", 1, "tiny-relu-ffn d256 ffn1024 r64", "relu",
                         256, 1024, 64, 0.10, 1.1, None, tokens=16),
    "c2": WorkloadConfig("c2", 2, "opt30b-shaped-relu-ffn d7168 ffn28672 r1024", "relu",
                         7168, 28672, 1024, 0.10, None, 0.17, tokens=64),
    "c3": WorkloadConfig("c3", 3, "llama2-70b-shaped-reglu-ffn d8192 ffn28672 r1024", "reglu",
                         8192, 28672, 1024, 0.20, None, 0.26, tokens=64),
    "c4": WorkloadConfig("c4", 4, "falcon40b-shaped-relu-ffn d8192 ffn32768 r1024", "relu",
                         8192, 32768, 1024, 0.08, 1.1, None,
                         batches=(1, 4, 8, 16, 32), tokens=64),
    "c5": WorkloadConfig("c5", 5, "opt66b-shaped-relu-ffn-stack d9216 ffn36864 r1024 x64", "relu",
                         9216, 36864, 1024, 0.10, None, 0.17, tokens=128, layers=64,
                         prompt_tokens=128, decode_steps=128),
    # SiLU-gated variant of the LLaMA2-70B shape: about half the neurons listed per
    # token, 75% of them carrying 80% of the activations ([R] Part A 3.1, 4.4)
    "c3s": WorkloadConfig("c3s", 6, "llama2-70b-shaped-swiglu-ffn d8192 ffn28672 r1024", "swiglu",
                          8192, 28672, 1024, 0.50, None, 0.75, tokens=64),
}


def custom_config(kind: str, d: int, ffn: int, r: int, mean: float = 0.10,
                  exponent: float = 1.1, number: int = 90, tau: float = 0.5) -> WorkloadConfig:
    """A small layer of arbitrary shape for tests (seeded through `number`)."""
    return WorkloadConfig("custom", number, f"custom-{kind} d{d} ffn{ffn} r{r}", kind,
                          d, ffn, r, mean, exponent, None, tau=tau)


def firing_law(n: int, mean: float, s: float, lo: float = 1e-4, hi: float = 0.999) -> np.ndarray:
    """f_k = clip(c * k**-s, lo, hi) for ranks k = 1..n, with c bisected so mean(f) = mean."""
    k = np.arange(1, n + 1, dtype=np.float64)
    base = k ** (-s)
    a, b = 1e-12, 1e12
    for _ in range(200):
        c = math.sqrt(a * b)
        if np.clip(c * base, lo, hi).mean() > mean:
            b = c
        else:
            a = c
    return np.clip(math.sqrt(a * b) * base, lo, hi)


def _top_share(f: np.ndarray, q: float) -> float:
    m = int(round(q * len(f)))
    return float(f[:m].sum() / f.sum())


def solve_exponent(n: int, mean: float, q: float, share: float = 0.80) -> float:
    """Exponent s for which the top q*n ranks carry `share` of sum(f)."""
    lo, hi = 0.05, 6.0
    for _ in range(100):
        s = 0.5 * (lo + hi)
        if _top_share(firing_law(n, mean, s), q) < share:
            lo = s
        else:
            hi = s
    return 0.5 * (lo + hi)


def rank_probabilities(cfg: WorkloadConfig) -> np.ndarray:
    """Firing probability by rank (descending), float64."""
    s = cfg.exponent if cfg.exponent is not None else solve_exponent(
        cfg.ffn, cfg.mean, cfg.hot_quantile, cfg.hot_share)
    return firing_law(cfg.ffn, cfg.mean, s)


def _seed(cfg: WorkloadConfig, tensor: str, layer: int) -> int:
    return 1000 * cfg.number + TENSOR_IDS[tensor] + 100000 * layer


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(rows: int, cols: int, seed: int, device) -> torch.Tensor:
    w = torch.randn(rows, cols, generator=_generator(device, seed), device=device,
                    dtype=torch.float32)
    w /= torch.linalg.vector_norm(w, dim=1, keepdim=True)
    return w.to(torch.float16)


def make_layer(cfg: WorkloadConfig, layer: int = 0, device="cpu",
               predictor: bool = True) -> Dict[str, object]:
    """One FFN layer (+ predictor) as a dict of tensors on `device`.

    Keys: W_up, W_gate (ReGLU only, else None), W_down (all ffn x d, fp16,
    neuron-major rows), b_up / b_gate (fp32 bias on the ReLU input, the other
    one None), P1 (r x d), b1 (None), P2 (ffn x r), b2 (fp32), f (per-neuron
    firing probability, float64 numpy), tau, kind.
    """
    device = torch.device(device)
    f_rank = rank_probabilities(cfg)
    perm = torch.randperm(cfg.ffn, generator=_generator("cpu", _seed(cfg, "rank_perm", layer)))
    # neuron perm[k] gets rank k
    f = np.empty(cfg.ffn, dtype=np.float64)
    f[perm.numpy()] = f_rank
    bias = torch.from_numpy(ndtri(f).astype(np.float32)).to(device)

    out: Dict[str, object] = {"kind": cfg.kind, "tau": cfg.tau, "f": f,
                              "d": cfg.d, "ffn": cfg.ffn, "r": cfg.r}
    out["W_up"] = _unit_rows(cfg.ffn, cfg.d, _seed(cfg, "W_up", layer), device)
    out["W_down"] = _unit_rows(cfg.ffn, cfg.d, _seed(cfg, "W_down", layer), device)
    if cfg.kind in ("reglu", "swiglu"):
        out["W_gate"] = _unit_rows(cfg.ffn, cfg.d, _seed(cfg, "W_gate", layer), device)
        out["b_gate"], out["b_up"] = bias, None
    elif cfg.kind == "relu":
        out["W_gate"], out["b_gate"], out["b_up"] = None, None, bias
    else:
        raise ValueError(f"unknown FFN kind {cfg.kind!r}")

    if predictor:
        P1 = _unit_rows(cfg.r, cfg.d, _seed(cfg, "P1", layer), device)
        P2 = _unit_rows(cfg.ffn, cfg.r, _seed(cfg, "P2", layer), device)
        row_sum = P2.to(torch.float64).sum(dim=1).cpu().numpy()
        b2 = -RELU_NORMAL_MEAN * row_sum + math.sqrt(RELU_NORMAL_VAR) * ndtri(f)
        out.update(P1=P1, b1=None, P2=P2,
                   b2=torch.from_numpy(b2.astype(np.float32)).to(device))
    return out


def make_tokens(cfg: WorkloadConfig, n: int, device="cpu", layer: int = 0,
                stream: str = "decode") -> torch.Tensor:
    """n tokens x ~ N(0, I_d) rounded to fp16, shape (n, d)."""
    g = _generator(torch.device(device), _seed(cfg, stream, layer))
    return torch.randn(n, cfg.d, generator=g, device=device,
                       dtype=torch.float32).to(torch.float16)


def make_calibration(cfg: WorkloadConfig, n: Optional[int] = None, device="cpu",
                     layer: int = 0) -> torch.Tensor:
    """Calibration tokens for the offline profile (separate seed from decode)."""
    return make_tokens(cfg, n or cfg.calib_tokens, device=device, layer=layer, stream="calib")
