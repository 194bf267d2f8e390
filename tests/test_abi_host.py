"""C ABI checks that need no GPU: exports, host-only reorder, argument validation.

Every validation case below fails before the library makes any HIP call, so
these run on a machine without a GPU.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from activation_sparse_predictor_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libpi.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pi_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = _declared()
    for want in ("pi_ffn_predict", "pi_ffn_sparse", "pi_ffn_decode", "pi_profile", "pi_reorder",
                 "pi_permute_rows", "pi_workspace_size", "pi_status_string", "pi_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    assert B.status_string(0) == "PI_OK"
    assert B.status_string(3) == "PI_ERR_WORKSPACE"
    assert B.status_string(99) == "PI_ERR_UNKNOWN"


def _reorder(counts, share):
    return __import__("activation_sparse_predictor_amd.runtime", fromlist=["reorder"]).reorder(counts, share)


def test_reorder_matches_oracle_on_golden_cases():
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "reorder_cases.json")))["cases"]
    for c in cases:
        perm, hot = _reorder(c["counts"], c["hot_share"])
        assert perm.tolist() == c["perm"] and hot == c["hot_count"], c


@pytest.mark.parametrize("n", [1, 5, 64, 1000, 28672])
def test_reorder_matches_oracle_random(n):
    rng = np.random.default_rng(n)
    for share in (0.5, 0.8, 0.95, 1.0):
        counts = (rng.zipf(1.3, size=n) * rng.integers(0, 2, size=n)).clip(max=4096).astype(np.uint32)
        perm, hot = _reorder(counts, share)
        operm, ohot = oracle.reorder_plan(counts, share)
        assert np.array_equal(perm, operm) and hot == ohot


def test_reorder_rejects_bad_arguments():
    c = np.ones(4, np.uint32)
    perm = np.empty(4, np.int32)
    hot = np.zeros(1, np.int32)
    assert B.pi_reorder(c, 4, 0.0, perm, hot) == B.PI_ERR_INVALID_ARG
    assert B.pi_reorder(c, 4, 1.5, perm, hot) == B.PI_ERR_INVALID_ARG
    assert B.pi_reorder(c, 0, 0.8, perm, hot) == B.PI_ERR_INVALID_ARG
    assert B.pi_reorder(None, 4, 0.8, perm, hot) == B.PI_ERR_INVALID_ARG
    assert "hot_share" in B.last_error() or "NULL" in B.last_error() or "ffn" in B.last_error()


def test_workspace_size_queries():
    p = B.pi_workspace_size(B.PI_OP_PREDICT, 1, 7168, 1024, 28672)
    s = B.pi_workspace_size(B.PI_OP_SPARSE, 1, 7168, 1024, 28672)
    assert p >= 1024 * 4 and s >= 28672 * 4
    assert B.pi_workspace_size(B.PI_OP_SPARSE, 4, 7168, 1024, 28672) > s
    for Bt in (1, 4):   # the decode step's workspace: both calls' data areas behind one 8 KB header
        dec = B.pi_workspace_size(B.PI_OP_DECODE, Bt, 7168, 1024, 28672)
        assert dec >= B.pi_workspace_size(B.PI_OP_PREDICT, Bt, 7168, 1024, 28672) + \
            B.pi_workspace_size(B.PI_OP_SPARSE, Bt, 7168, 1024, 28672) - 8192
    out = ctypes.c_size_t(0)
    assert B.load().pi_workspace_size(9, 1, 8, 8, 8, ctypes.byref(out)) == B.PI_ERR_INVALID_ARG
    assert B.load().pi_workspace_size(0, 0, 8, 8, 8, ctypes.byref(out)) == B.PI_ERR_INVALID_ARG


# Fake, aligned, never-dereferenced addresses: validation rejects each call first.
A = 1 << 20          # 16-byte aligned
W = (1 << 20) + 4096


def _predict(**kw):
    args = dict(x=A, B=1, d=64, P1=A, b1=None, act=B.PI_ACT_RELU, P2=A, b2=None, r=16, ffn=128,
                tau=0.5, idx=A, count=A, ws=A, ws_bytes=0, stream=0)
    args.update(kw)
    return B.pi_ffn_predict(*args.values())


def _sparse(**kw):
    args = dict(kind=B.PI_FFN_RELU, x=A, B=1, d=64, ffn=128, W_up=A, b_up=None, W_gate=None,
                b_gate=None, W_down=A, idx=A, count=A, y=A, flags=0, ws=A, ws_bytes=0, stream=0)
    args.update(kw)
    return B.pi_ffn_sparse(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.PI_ERR_INVALID_ARG),
    (dict(P1=None), B.PI_ERR_INVALID_ARG),
    (dict(P2=None), B.PI_ERR_INVALID_ARG),
    (dict(idx=None), B.PI_ERR_INVALID_ARG),
    (dict(count=None), B.PI_ERR_INVALID_ARG),
    (dict(B=0), B.PI_ERR_INVALID_ARG),
    (dict(B=257), B.PI_ERR_INVALID_ARG),
    (dict(d=0), B.PI_ERR_INVALID_ARG),
    (dict(r=0), B.PI_ERR_INVALID_ARG),
    (dict(ffn=-1), B.PI_ERR_INVALID_ARG),
    (dict(tau=0.0), B.PI_ERR_INVALID_ARG),
    (dict(tau=1.0), B.PI_ERR_INVALID_ARG),
    (dict(tau=float("nan")), B.PI_ERR_INVALID_ARG),
    (dict(act=7), B.PI_ERR_INVALID_ARG),
    (dict(d=60), B.PI_ERR_UNSUPPORTED),
    (dict(r=12), B.PI_ERR_UNSUPPORTED),
    (dict(x=A + 8), B.PI_ERR_UNSUPPORTED),
    (dict(P2=A + 2), B.PI_ERR_UNSUPPORTED),
    (dict(b2=A + 2), B.PI_ERR_UNSUPPORTED),
    (dict(d=32768), B.PI_ERR_UNSUPPORTED),
    (dict(ws=None), B.PI_ERR_WORKSPACE),
    (dict(ws_bytes=16), B.PI_ERR_WORKSPACE),
])
def test_predict_rejects_before_launch(kw, code):
    assert _predict(**kw) == code
    assert B.last_error() != ""


def _predict_hot(**kw):
    args = dict(x=A, B=1, d=64, P1=A, b1=None, act=B.PI_ACT_RELU, P2=A, b2=None, r=16, ffn=128, n_hot=32,
                tau=0.5, idx=A, count=A, ws=A, ws_bytes=0, stream=0)
    args.update(kw)
    return B.pi_ffn_predict_hot(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(n_hot=-32), B.PI_ERR_INVALID_ARG),
    (dict(n_hot=160), B.PI_ERR_INVALID_ARG),          # beyond ffn
    (dict(n_hot=16), B.PI_ERR_UNSUPPORTED),           # not whole 32-neuron mask words
    (dict(n_hot=97, ffn=100), B.PI_ERR_UNSUPPORTED),  # ffn may be ragged, n_hot may not
    (dict(x=None), B.PI_ERR_INVALID_ARG),
    (dict(tau=1.0), B.PI_ERR_INVALID_ARG),
    (dict(ws_bytes=16), B.PI_ERR_WORKSPACE),
])
def test_predict_hot_rejects_before_launch(kw, code):
    assert _predict_hot(**kw) == code
    assert B.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(kind=5), B.PI_ERR_INVALID_ARG),
    (dict(x=None), B.PI_ERR_INVALID_ARG),
    (dict(W_up=None), B.PI_ERR_INVALID_ARG),
    (dict(W_down=None), B.PI_ERR_INVALID_ARG),
    (dict(y=None), B.PI_ERR_INVALID_ARG),
    (dict(idx=None), B.PI_ERR_INVALID_ARG),
    (dict(count=None), B.PI_ERR_INVALID_ARG),
    (dict(W_gate=A), B.PI_ERR_INVALID_ARG),                 # gate given for ReLU
    (dict(kind=B.PI_FFN_REGLU), B.PI_ERR_INVALID_ARG),      # gate missing for ReGLU
    (dict(kind=B.PI_FFN_SWIGLU), B.PI_ERR_INVALID_ARG),     # gate missing for SwiGLU
    (dict(kind=3), B.PI_ERR_INVALID_ARG),                   # no such kind
    (dict(b_gate=W), B.PI_ERR_INVALID_ARG),                 # gate bias for ReLU
    (dict(flags=0x80), B.PI_ERR_INVALID_ARG),
    (dict(B=300), B.PI_ERR_INVALID_ARG),
    (dict(d=12), B.PI_ERR_UNSUPPORTED),
    (dict(W_down=A + 4), B.PI_ERR_UNSUPPORTED),
    (dict(y=A + 4), B.PI_ERR_UNSUPPORTED),
    (dict(idx=A + 2), B.PI_ERR_UNSUPPORTED),
    (dict(ws=None), B.PI_ERR_WORKSPACE),
    (dict(ws_bytes=64), B.PI_ERR_WORKSPACE),
])
def test_sparse_rejects_before_launch(kw, code):
    assert _sparse(**kw) == code
    assert B.last_error() != ""


def _decode(**kw):
    args = dict(kind=B.PI_FFN_RELU, x=A, B=1, d=64, ffn=128, P1=A, b1=None, act=B.PI_ACT_RELU, P2=A, b2=None,
                r=16, tau=0.5, W_up=A, b_up=None, W_gate=None, b_gate=None, W_down=A, idx=A, count=A, y=A,
                flags=0, ws=A, ws_bytes=0, stream=0)
    args.update(kw)
    return B.pi_ffn_decode(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.PI_ERR_INVALID_ARG),
    (dict(P1=None), B.PI_ERR_INVALID_ARG),
    (dict(W_up=None), B.PI_ERR_INVALID_ARG),
    (dict(y=None), B.PI_ERR_INVALID_ARG),
    (dict(idx=None), B.PI_ERR_INVALID_ARG),
    (dict(tau=1.5), B.PI_ERR_INVALID_ARG),
    (dict(kind=B.PI_FFN_REGLU), B.PI_ERR_INVALID_ARG),      # gate missing for ReGLU
    (dict(kind=B.PI_FFN_SWIGLU), B.PI_ERR_INVALID_ARG),     # gate missing for SwiGLU
    (dict(kind=3), B.PI_ERR_INVALID_ARG),                   # no such kind
    (dict(flags=B.PI_DENSE), B.PI_ERR_INVALID_ARG),         # a dense step has no predictor
    (dict(flags=0x80), B.PI_ERR_INVALID_ARG),
    (dict(r=12), B.PI_ERR_UNSUPPORTED),
    (dict(y=A + 4), B.PI_ERR_UNSUPPORTED),
    (dict(ws=None), B.PI_ERR_WORKSPACE),
    (dict(ws_bytes=64), B.PI_ERR_WORKSPACE),
])
def test_decode_rejects_before_launch(kw, code):
    assert _decode(**kw) == code
    assert B.last_error() != ""


def test_dense_flag_allows_null_index_list():
    # with PI_DENSE the index list is not required: the call gets as far as the workspace check
    assert _sparse(flags=B.PI_DENSE, idx=None, count=None, ws=None) == B.PI_ERR_WORKSPACE


def test_flag_values_match_the_header():
    text = open(HEADER).read()
    for name in ("PI_DENSE", "PI_PER_TOKEN", "PI_DETERMINISTIC", "PI_CHECK_IDX"):
        m = re.search(r"#define\s+%s\s+(0x[0-9a-fA-F]+)u" % name, text)
        assert m, name
        assert int(m.group(1), 16) == getattr(B, name), name


def test_check_and_deterministic_flags_are_accepted():
    # both flags pass the flag check: the call gets as far as the workspace check
    assert _sparse(flags=B.PI_CHECK_IDX | B.PI_DETERMINISTIC, ws=None) == B.PI_ERR_WORKSPACE


def test_profile_and_permute_reject_before_launch():
    assert B.pi_profile(None, 4, 64, 128, A, None, A, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_profile(A, 0, 64, 128, A, None, A, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_profile(A, 4, 60, 128, A, None, A, stream=0) == B.PI_ERR_UNSUPPORTED
    assert B.pi_profile(A, 4, 64, 128, A + 2, None, A, stream=0) == B.PI_ERR_UNSUPPORTED
    assert B.pi_permute_rows(A, None, 4, 16, A, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_permute_rows(A, W, 4, 6, A, stream=0) == B.PI_ERR_UNSUPPORTED
    assert B.pi_permute_rows(A, A + 16, 4, 16, A, stream=0) == B.PI_ERR_INVALID_ARG   # overlap
    assert B.pi_permute_rows(A, W, 0, 16, A, stream=0) == B.PI_ERR_INVALID_ARG


def _predict_q4(**kw):
    args = dict(x=A, B=1, d=64, q_P1=A, s_P1=W, b1=None, act=B.PI_ACT_RELU, q_P2=A, s_P2=W, b2=None, r=64,
                ffn=128, n_hot=0, tau=0.5, idx=A, count=A, ws=A, ws_bytes=0, stream=0)
    args.update(kw)
    return B.pi_ffn_predict_q4(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.PI_ERR_INVALID_ARG),
    (dict(q_P1=None), B.PI_ERR_INVALID_ARG),
    (dict(q_P2=None), B.PI_ERR_INVALID_ARG),
    (dict(s_P1=None), B.PI_ERR_INVALID_ARG),
    (dict(s_P2=None), B.PI_ERR_INVALID_ARG),
    (dict(idx=None), B.PI_ERR_INVALID_ARG),
    (dict(B=0), B.PI_ERR_INVALID_ARG),
    (dict(act=3), B.PI_ERR_INVALID_ARG),
    (dict(tau=0.0), B.PI_ERR_INVALID_ARG),
    (dict(n_hot=-32), B.PI_ERR_INVALID_ARG),
    (dict(n_hot=160), B.PI_ERR_INVALID_ARG),
    (dict(n_hot=16), B.PI_ERR_UNSUPPORTED),
    (dict(d=96), B.PI_ERR_UNSUPPORTED),          # a multiple of 8, not of the INT4 group
    (dict(r=32), B.PI_ERR_UNSUPPORTED),          # likewise for P2's rows
    (dict(s_P2=W + 1), B.PI_ERR_UNSUPPORTED),
    (dict(ws=None), B.PI_ERR_WORKSPACE),
    (dict(ws_bytes=16), B.PI_ERR_WORKSPACE),
])
def test_predict_q4_rejects_before_launch(kw, code):
    assert _predict_q4(**kw) == code
    assert B.last_error() != ""


def _sparse_q4(**kw):
    args = dict(kind=B.PI_FFN_RELU, x=A, B=1, d=64, ffn=128, q_up=A, s_up=W, b_up=None, q_gate=None,
                s_gate=None, b_gate=None, q_down=A, s_down=W, idx=A, count=A, y=A, flags=0, ws=A, ws_bytes=0,
                stream=0)
    args.update(kw)
    return B.pi_ffn_sparse_q4(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.PI_ERR_INVALID_ARG),
    (dict(q_up=None), B.PI_ERR_INVALID_ARG),
    (dict(q_down=None), B.PI_ERR_INVALID_ARG),
    (dict(s_up=None), B.PI_ERR_INVALID_ARG),
    (dict(s_down=None), B.PI_ERR_INVALID_ARG),
    (dict(kind=B.PI_FFN_REGLU, q_gate=A), B.PI_ERR_INVALID_ARG),   # gate codes without scales
    (dict(kind=B.PI_FFN_SWIGLU), B.PI_ERR_INVALID_ARG),            # gate missing
    (dict(q_gate=A), B.PI_ERR_INVALID_ARG),                        # gate given for ReLU
    (dict(flags=B.PI_PER_TOKEN), B.PI_ERR_INVALID_ARG),            # not an INT4 flag
    (dict(flags=B.PI_CHECK_IDX), B.PI_ERR_INVALID_ARG),
    (dict(d=96), B.PI_ERR_UNSUPPORTED),
    (dict(s_down=W + 1), B.PI_ERR_UNSUPPORTED),
    (dict(y=A + 4), B.PI_ERR_UNSUPPORTED),
    (dict(ws=None), B.PI_ERR_WORKSPACE),
    (dict(ws_bytes=64), B.PI_ERR_WORKSPACE),
])
def test_sparse_q4_rejects_before_launch(kw, code):
    assert _sparse_q4(**kw) == code
    assert B.last_error() != ""


def test_quantize_rows_rejects_before_launch():
    assert B.pi_quantize_rows(None, 4, 64, A, W, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_quantize_rows(A, 0, 64, A, W, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_quantize_rows(A, 4, 0, A, W, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_quantize_rows(A, 4, 96, A, W, stream=0) == B.PI_ERR_UNSUPPORTED
    assert B.pi_quantize_rows(A, 4, 64, None, W, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_quantize_rows(A, 4, 64, A, None, stream=0) == B.PI_ERR_INVALID_ARG
    assert B.pi_quantize_rows(A, 4, 64, A + 8, W, stream=0) == B.PI_ERR_UNSUPPORTED
    assert B.pi_quantize_rows(A, 4, 64, A, W + 1, stream=0) == B.PI_ERR_UNSUPPORTED
    assert B.pi_quantize_rows(A, 4, 32768, A, W, stream=0) == B.PI_ERR_UNSUPPORTED


def test_decode_hot_rejects_before_launch():
    args = dict(kind=B.PI_FFN_RELU, x=A, B=1, d=64, ffn=128, P1=A, b1=None, act=B.PI_ACT_RELU, P2=A, b2=None, r=16,
                n_hot=0, tau=0.5, W_up=A, b_up=None, W_gate=None, b_gate=None, W_down=A, idx=A, count=A, y=A,
                flags=0, ws=A, ws_bytes=0, stream=0)
    for kw, code in ((dict(n_hot=160), B.PI_ERR_INVALID_ARG), (dict(n_hot=-32), B.PI_ERR_INVALID_ARG),
                     (dict(n_hot=48), B.PI_ERR_UNSUPPORTED), (dict(flags=B.PI_DENSE), B.PI_ERR_INVALID_ARG),
                     (dict(), B.PI_ERR_WORKSPACE)):
        a = dict(args)
        a.update(kw)
        assert B.pi_ffn_decode_hot(*a.values()) == code, kw
