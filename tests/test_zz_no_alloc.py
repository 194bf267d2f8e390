"""pi_ffn_decode_noalloc (the decode step on the library's static scratch)
against pi_ffn_decode on a caller's workspace: same kernels, so the list, the
count and y must be bitwise equal, call after call, also when the sizes
shrink between calls; sizes whose workspace exceeds the static scratch are
rejected before anything is launched."""

import numpy as np
import pytest
import torch

import oracle as O
from activation_sparse_predictor_amd import binding as B
from activation_sparse_predictor_amd import runtime as R
from synthetic import CONFIGS, custom_config, make_layer, make_tokens
from tests.parity import check_idx, check_y

DEV = "cuda"


def _noalloc(L, x, idx, cnt, y, flags=0):
    Bt, d = x.shape
    return B.pi_ffn_decode_noalloc(B.KINDS[L["kind"]], x, Bt, d, L["ffn"], L["P1"], L.get("b1"), B.PI_ACT_RELU,
                                   L["P2"], L.get("b2"), L["r"], float(L["tau"]), L["W_up"], L.get("b_up"),
                                   L.get("W_gate"), L.get("b_gate"), L["W_down"], idx, cnt, y, flags)


def _host(layer):
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}


@pytest.mark.gpu
def test_noalloc_decode_equals_decode():
    """Two calls in a row, the second on a smaller layer (and a third back on the
    larger one): each bitwise equal to pi_ffn_decode, and within the parity bar
    of the oracle."""
    big = custom_config("reglu", 2048, 4160, 256, mean=0.2, number=110)
    small = custom_config("relu", 520, 1000, 72, mean=0.15, number=111)
    layers = {k: R.to_device(make_layer(c), DEV) for k, c in (("big", big), ("small", small))}
    for key, t in (("big", 0), ("small", 0), ("big", 1)):
        L = layers[key]
        d, ffn = L["d"], L["ffn"]
        x = make_tokens(big if key == "big" else small, 2).to(DEV)[t:t + 1].contiguous()
        y_ref, idx_ref, cnt_ref = R.decode(L, x)
        idx = torch.full((1, ffn), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        y = torch.full((1, d), float("nan"), dtype=torch.float32, device=DEV)
        B.check(_noalloc(L, x, idx, cnt, y), "pi_ffn_decode_noalloc")
        torch.cuda.synchronize()
        c = int(cnt.cpu()[0])
        assert c == int(cnt_ref.cpu()[0]), f"{key}: count {c} vs {int(cnt_ref.cpu()[0])}"
        assert torch.equal(idx[0, :c], idx_ref[0, :c]), f"{key}: index list differs"
        assert torch.equal(y, y_ref), f"{key}: y differs from pi_ffn_decode"
        H = _host(L)
        gi = idx[0, :c].cpu().numpy()
        z = O.predictor_logits(x[0].cpu(), H["P1"], None, "relu", H["P2"], H["b2"])
        check_idx(gi, z, O.logit_threshold(L["tau"]), where=f"noalloc {key}")
        ref = O.sparse_ffn(H["kind"], x[0].cpu(), H["W_up"], H.get("b_up"), H.get("W_gate"), H.get("b_gate"),
                           H["W_down"], gi)
        check_y(y[0].cpu().numpy(), ref, where=f"noalloc {key}")


@pytest.mark.gpu
def test_noalloc_decode_full_size_layer():
    """The OPT-66B-shaped layer (d 9216, ffn 36864, r 1024: about 2 MB of the
    4 MB scratch), two tokens, bitwise equal to pi_ffn_decode."""
    cfg = CONFIGS["c5"]
    L = make_layer(cfg, layer=5, device=DEV)
    X = make_tokens(cfg, 2, device=DEV, layer=5)
    for t in range(2):
        x = X[t:t + 1].contiguous()
        y_ref, idx_ref, cnt_ref = R.decode(L, x)
        idx = torch.empty(1, cfg.ffn, dtype=torch.int32, device=DEV)
        cnt = torch.empty(1, dtype=torch.int32, device=DEV)
        y = torch.empty(1, cfg.d, dtype=torch.float32, device=DEV)
        B.check(_noalloc(L, x, idx, cnt, y), "pi_ffn_decode_noalloc")
        torch.cuda.synchronize()
        c = int(cnt.cpu()[0])
        assert c == int(cnt_ref.cpu()[0]) and c > 0
        assert torch.equal(idx[0, :c], idx_ref[0, :c])
        assert torch.equal(y, y_ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """Checked before any HIP call: a batch whose union workspace is larger than
    the static scratch, and a single token of a very wide layer."""
    import os
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libpi.so not built")
    A = 1 << 20   # an aligned, never dereferenced address
    assert B.pi_workspace_size(B.PI_OP_DECODE, 2, 9216, 1024, 36864) > B.PI_NOALLOC_SCRATCH_BYTES
    st = B.pi_ffn_decode_noalloc(B.PI_FFN_RELU, A, 2, 9216, 36864, A, None, B.PI_ACT_RELU, A, A, 1024, 0.5,
                                 A, A, None, None, A, A, A, A, 0, 0)
    assert st == B.PI_ERR_WORKSPACE and "static scratch" in B.last_error()
    st = B.pi_ffn_decode_noalloc(B.PI_FFN_RELU, A, 1, 16384, 400000, A, None, B.PI_ACT_RELU, A, A, 1024, 0.5,
                                 A, A, None, None, A, A, A, A, 0, 0)
    assert st == B.PI_ERR_WORKSPACE
    # argument errors come first, as in pi_ffn_decode
    st = B.pi_ffn_decode_noalloc(B.PI_FFN_RELU, None, 1, 64, 64, A, None, B.PI_ACT_RELU, A, A, 8, 0.5,
                                 A, A, None, None, A, A, A, A, 0, 0)
    assert st == B.PI_ERR_INVALID_ARG
