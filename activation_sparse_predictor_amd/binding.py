"""ctypes binding of libpi (include/pi.h): same names, argument marshalling only.

Every function takes device tensors (torch), raw integer addresses or None
(NULL) for pointer arguments and returns the pi_status integer.  The stream
defaults to torch's current stream on the current device.  Nothing here
computes any part of the path: each call goes straight to the HIP library,
and a missing library raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpi.so")

PI_OK = 0
PI_ERR_INVALID_ARG = 1
PI_ERR_UNSUPPORTED = 2
PI_ERR_WORKSPACE = 3
PI_ERR_HIP = 4

PI_FFN_RELU = 0
PI_FFN_REGLU = 1
PI_FFN_SWIGLU = 2
PI_ACT_RELU = 0
PI_ACT_NONE = 1
PI_OP_PREDICT = 0
PI_OP_SPARSE = 1
PI_OP_PROFILE = 2
PI_OP_DECODE = 3
PI_OP_DECODE_HOT = 4
PI_DENSE = 0x1
PI_PER_TOKEN = 0x2
PI_DETERMINISTIC = 0x4
PI_CHECK_IDX = 0x8
PI_NOALLOC_SCRATCH_BYTES = 4 << 20   # the static scratch of pi_ffn_decode_noalloc, per GPU

KINDS = {"relu": PI_FFN_RELU, "reglu": PI_FFN_REGLU, "swiglu": PI_FFN_SWIGLU}
ACTS = {"relu": PI_ACT_RELU, "none": PI_ACT_NONE}

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "pi_ffn_predict": (_I, [_P, _I, _I, _P, _P, _I, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "pi_ffn_predict_hot": (_I, [_P, _I, _I, _P, _P, _I, _P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "pi_ffn_sparse": (_I, [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "pi_ffn_decode": (_I, [_I, _P, _I, _I, _I, _P, _P, _I, _P, _P, _I, ctypes.c_float, _P, _P, _P, _P, _P,
                           _P, _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "pi_ffn_decode_hot": (_I, [_I, _P, _I, _I, _I, _P, _P, _I, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P, _P, _P,
                               _P, _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "pi_ffn_decode_hot_begin": (_I, [_I, _P, _I, _I, _P, _P, _I, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P, _P, _P,
                                     _P, _P, _P, _SZ, _P]),
    "pi_ffn_decode_hot_end": (_I, [_I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint32, _P, _SZ,
                                   _P]),
    "pi_ffn_decode_noalloc": (_I, [_I, _P, _I, _I, _I, _P, _P, _I, _P, _P, _I, ctypes.c_float, _P, _P, _P, _P, _P,
                                   _P, _P, _P, ctypes.c_uint32, _P]),
    "pi_ffn_predict_q4": (_I, [_P, _I, _I, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P,
                               _SZ, _P]),
    "pi_quantize_rows": (_I, [_P, _I, _I, _P, _P, _P]),
    "pi_ffn_sparse_q4": (_I, [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint32,
                              _P, _SZ, _P]),
    "pi_profile": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "pi_reorder": (_I, [_P, _I, ctypes.c_double, _P, _P]),
    "pi_permute_rows": (_I, [_P, _P, _I, _I, _P, _P]),
    "pi_workspace_size": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "pi_status_string": (ctypes.c_char_p, [_I]),
    "pi_last_error": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


class PiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {last_error()}")


def load() -> ctypes.CDLL:
    """Load libpi.so from the package directory (built by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m activation_sparse_predictor_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_string(status: int) -> str:
    return load().pi_status_string(status).decode()


def last_error() -> str:
    return load().pi_last_error().decode()


def check(status: int, where: str = "libpi") -> None:
    if status != PI_OK:
        raise PiError(status, where)


def pi_workspace_size(op: int, B: int, d: int, r: int, ffn: int) -> int:
    out = _SZ(0)
    check(load().pi_workspace_size(op, B, d, r, ffn, ctypes.byref(out)), "pi_workspace_size")
    return out.value


def pi_ffn_predict(x, B, d, P1, b1, act, P2, b2, r, ffn, tau, idx, count, ws, ws_bytes,
                   stream=None) -> int:
    return load().pi_ffn_predict(_ptr(x), B, d, _ptr(P1), _ptr(b1), act, _ptr(P2), _ptr(b2), r,
                                 ffn, tau, _ptr(idx), _ptr(count), _ptr(ws), ws_bytes,
                                 _stream(stream))


def pi_ffn_predict_hot(x, B, d, P1, b1, act, P2, b2, r, ffn, n_hot, tau, idx, count, ws, ws_bytes,
                       stream=None) -> int:
    return load().pi_ffn_predict_hot(_ptr(x), B, d, _ptr(P1), _ptr(b1), act, _ptr(P2), _ptr(b2), r,
                                     ffn, n_hot, tau, _ptr(idx), _ptr(count), _ptr(ws), ws_bytes,
                                     _stream(stream))


def pi_ffn_predict_q4(x, B, d, q_P1, s_P1, b1, act, q_P2, s_P2, b2, r, ffn, n_hot, tau, idx, count, ws,
                      ws_bytes, stream=None) -> int:
    return load().pi_ffn_predict_q4(_ptr(x), B, d, _ptr(q_P1), _ptr(s_P1), _ptr(b1), act, _ptr(q_P2), _ptr(s_P2),
                                    _ptr(b2), r, ffn, n_hot, tau, _ptr(idx), _ptr(count), _ptr(ws), ws_bytes,
                                    _stream(stream))


def pi_quantize_rows(W, rows, d, q, scales, stream=None) -> int:
    return load().pi_quantize_rows(_ptr(W), rows, d, _ptr(q), _ptr(scales), _stream(stream))


def pi_ffn_sparse_q4(kind, x, B, d, ffn, q_up, s_up, b_up, q_gate, s_gate, b_gate, q_down, s_down, idx, count,
                     y, flags, ws, ws_bytes, stream=None) -> int:
    return load().pi_ffn_sparse_q4(kind, _ptr(x), B, d, ffn, _ptr(q_up), _ptr(s_up), _ptr(b_up), _ptr(q_gate),
                                   _ptr(s_gate), _ptr(b_gate), _ptr(q_down), _ptr(s_down), _ptr(idx), _ptr(count),
                                   _ptr(y), flags, _ptr(ws), ws_bytes, _stream(stream))


def pi_ffn_sparse(kind, x, B, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags,
                  ws, ws_bytes, stream=None) -> int:
    return load().pi_ffn_sparse(kind, _ptr(x), B, d, ffn, _ptr(W_up), _ptr(b_up), _ptr(W_gate),
                                _ptr(b_gate), _ptr(W_down), _ptr(idx), _ptr(count), _ptr(y), flags,
                                _ptr(ws), ws_bytes, _stream(stream))


def pi_ffn_decode(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down,
                  idx, count, y, flags, ws, ws_bytes, stream=None) -> int:
    return load().pi_ffn_decode(kind, _ptr(x), B, d, ffn, _ptr(P1), _ptr(b1), act, _ptr(P2), _ptr(b2), r, tau,
                                _ptr(W_up), _ptr(b_up), _ptr(W_gate), _ptr(b_gate), _ptr(W_down), _ptr(idx),
                                _ptr(count), _ptr(y), flags, _ptr(ws), ws_bytes, _stream(stream))


def pi_ffn_decode_hot(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, n_hot, tau, W_up, b_up, W_gate, b_gate, W_down,
                      idx, count, y, flags, ws, ws_bytes, stream=None) -> int:
    return load().pi_ffn_decode_hot(kind, _ptr(x), B, d, ffn, _ptr(P1), _ptr(b1), act, _ptr(P2), _ptr(b2), r, n_hot,
                                    tau, _ptr(W_up), _ptr(b_up), _ptr(W_gate), _ptr(b_gate), _ptr(W_down), _ptr(idx),
                                    _ptr(count), _ptr(y), flags, _ptr(ws), ws_bytes, _stream(stream))


def pi_ffn_decode_hot_begin(kind, x, d, ffn, P1, b1, act, P2, b2, r, n_hot, tau, W_up, b_up, W_gate, b_gate,
                            W_down, idx, count, ws, ws_bytes, stream=None) -> int:
    return load().pi_ffn_decode_hot_begin(kind, _ptr(x), d, ffn, _ptr(P1), _ptr(b1), act, _ptr(P2), _ptr(b2), r, n_hot,
                                          tau, _ptr(W_up), _ptr(b_up), _ptr(W_gate), _ptr(b_gate), _ptr(W_down),
                                          _ptr(idx), _ptr(count), _ptr(ws), ws_bytes, _stream(stream))


def pi_ffn_decode_hot_end(kind, x, d, ffn, r, n_hot, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags, ws,
                          ws_bytes, stream=None) -> int:
    return load().pi_ffn_decode_hot_end(kind, _ptr(x), d, ffn, r, n_hot, _ptr(W_up), _ptr(b_up), _ptr(W_gate),
                                        _ptr(b_gate), _ptr(W_down), _ptr(idx), _ptr(count), _ptr(y), flags, _ptr(ws),
                                        ws_bytes, _stream(stream))


def pi_ffn_decode_noalloc(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down,
                          idx, count, y, flags, stream=None) -> int:
    return load().pi_ffn_decode_noalloc(kind, _ptr(x), B, d, ffn, _ptr(P1), _ptr(b1), act, _ptr(P2), _ptr(b2), r,
                                        tau, _ptr(W_up), _ptr(b_up), _ptr(W_gate), _ptr(b_gate), _ptr(W_down),
                                        _ptr(idx), _ptr(count), _ptr(y), flags, _stream(stream))


def pi_profile(X, n, d, ffn, W_fire, b_fire, counts, ws=None, ws_bytes=0, stream=None) -> int:
    return load().pi_profile(_ptr(X), n, d, ffn, _ptr(W_fire), _ptr(b_fire), _ptr(counts),
                             _ptr(ws), ws_bytes, _stream(stream))


def pi_reorder(counts, ffn, hot_share, perm, hot_count) -> int:
    """Host-only: counts, perm and hot_count are host buffers (numpy arrays or addresses)."""
    def hp(a):
        if a is None or isinstance(a, int):
            return a
        return a.ctypes.data
    return load().pi_reorder(hp(counts), ffn, float(hot_share), hp(perm), hp(hot_count))


def pi_permute_rows(src, dst, rows, row_bytes, perm, stream=None) -> int:
    return load().pi_permute_rows(_ptr(src), _ptr(dst), rows, row_bytes, _ptr(perm), _stream(stream))
