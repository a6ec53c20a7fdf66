"""ctypes wrapper of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg.  The product package never imports it.
Arguments are numpy arrays (or CPU torch tensors); this file only marshals.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

F32, BF16, FP8 = 0, 1, 2
DEFAULT, RENORMALIZE, DEEPSEEKV3, LLAMA4, RENORMALIZE_NAIVE, MINIMAX2, SIGMOID_RENORM = 0, 1, 2, 3, 4, 5, 6
DTYPE_CODE = {"f32": F32, "bf16": BF16, "fp8": FP8}

_lib = None


class _Weights(C.Structure):
    _fields_ = [("H", C.c_int), ("I", C.c_int), ("wdt", C.c_int),
                ("w13", C.c_void_p), ("w2", C.c_void_p),
                ("w13_scale", C.c_void_p), ("w2_scale", C.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build(verbose=False)
        L = C.CDLL(_build.LIB)
        P = C.c_void_p
        i = C.c_int
        L.oracle_decode_bf16.argtypes = [C.c_uint16]
        L.oracle_decode_bf16.restype = C.c_double
        L.oracle_decode_e4m3.argtypes = [C.c_uint8]
        L.oracle_decode_e4m3.restype = C.c_double
        L.oracle_encode_e4m3.argtypes = [C.c_float]
        L.oracle_encode_e4m3.restype = C.c_uint8
        L.oracle_quantize_fp8.argtypes = [P, i, i, i, P, P]
        L.oracle_sigmoid_f32.argtypes = [C.c_float, C.POINTER(C.c_int)]
        L.oracle_sigmoid_f32.restype = C.c_float
        L.oracle_route.argtypes = [P, i, i, i, i, i, i, P, C.c_double, i, P, P, P]
        L.oracle_permute.argtypes = [P, i, i, i, i, P, P, P]
        L.oracle_expert_rows.argtypes = [C.POINTER(_Weights), P, i, P, i, i, i, i, P, P, P, i, P, P]
        L.oracle_layer_tokens.argtypes = [C.POINTER(_Weights), P, i, P, i, i, i, i, P, P, P, i, P]
        L.oracle_finalize.argtypes = [P, i, P, P, i, i, i, i, P]
        L.oracle_set_num_threads.argtypes = [i]
        _lib = L
    return _lib


def _np(a, dtype=None):
    """Contiguous host numpy view of a numpy array or CPU torch tensor."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.uint16) if hasattr(torch, "uint16") else a.view(torch.int16)
            elif a.dtype == torch.float8_e4m3fn:
                a = a.view(torch.uint8)
            a = a.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def decode_bf16(bits: int) -> float:
    return lib().oracle_decode_bf16(int(bits))


def decode_e4m3(bits: int) -> float:
    return lib().oracle_decode_e4m3(int(bits))


def encode_e4m3(f: float) -> int:
    """fp32 value -> OCP e4m3fn code (nearest, ties to even, saturating)."""
    return int(lib().oracle_encode_e4m3(float(f)))


def quantize_fp8(x, dt="bf16"):
    """1x128 block quantisation of x [rows, cols] -> (codes uint8 [rows, cols],
    scales float32 [rows, cols/128])."""
    xa = _np(x)
    rows, cols = xa.shape
    q = np.zeros((rows, cols), np.uint8)
    s = np.zeros((rows, cols // 128), np.float32)
    rc = lib().oracle_quantize_fp8(_ptr(xa), DTYPE_CODE[dt] if isinstance(dt, str) else dt,
                                   rows, cols, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_quantize_fp8: cols must be a multiple of 128, dtype f32/bf16")
    return q, s


def sigmoid_f32(l: float):
    """(fp32 sigmoid value, whether it was a hard rounding case)."""
    hard = C.c_int(0)
    v = lib().oracle_sigmoid_f32(float(l), C.byref(hard))
    return v, hard.value


def route(logits, k, method, n_group=1, topk_group=1, bias=None, scaling=1.0, renorm=False):
    """-> (ids int32 [T,k], scales float64 [T,k], hard_case_count)."""
    lg = _np(logits, np.float32)
    T, E = lg.shape
    b = _np(bias, np.float32)
    ids = np.zeros((T, k), np.int32)
    sc = np.zeros((T, k), np.float64)
    hard = C.c_int64(0)
    rc = lib().oracle_route(_ptr(lg), T, E, method, k, n_group, topk_group, _ptr(b),
                            float(scaling), int(bool(renorm)), _ptr(ids), _ptr(sc),
                            C.cast(C.pointer(hard), C.c_void_p))
    if rc != 0:
        raise ValueError("oracle_route rejected the arguments")
    return ids, sc, hard.value


def permute(ids, E, n_shared=0):
    """-> (offsets int32 [G+1], permuted_pair int32 [P], unpermute int32 [P])."""
    a = _np(ids, np.int32)
    T, k = a.shape
    off = np.zeros(E + n_shared + 1, np.int32)
    pp = np.zeros(T * k, np.int32)
    up = np.zeros(T * k, np.int32)
    rc = lib().oracle_permute(_ptr(a), T, k, E, n_shared, _ptr(off), _ptr(pp), _ptr(up))
    if rc != 0:
        raise ValueError("oracle_permute: expert id out of range")
    return off, pp, up


class Weights:
    """Host copies of the expert weights kept alive for the C struct."""

    def __init__(self, w13, w2, wdt, w13_scale=None, w2_scale=None):
        self.w13 = _np(w13)
        self.w2 = _np(w2)
        self.s13 = _np(w13_scale, np.float32)
        self.s2 = _np(w2_scale, np.float32)
        G, twoI, H = self.w13.shape
        self.H, self.I = H, twoI // 2
        self.wdt = DTYPE_CODE[wdt] if isinstance(wdt, str) else int(wdt)
        self.struct = _Weights(self.H, self.I, self.wdt, _ptr(self.w13), _ptr(self.w2),
                               _ptr(self.s13), _ptr(self.s2))


def expert_rows(W: Weights, x, act, T, k, E, n_shared, offsets, permuted_pair, rows,
                want_h=False, x_scale=None):
    """FFN output rows (fp64 [len(rows), H]) and optionally h (fp64 [len(rows), I]).
    act "fp8": x holds e4m3 codes with 1x128 scales x_scale [T, H/128]."""
    xa = _np(x)
    xs = _np(x_scale, np.float32)
    off = _np(offsets, np.int32)
    pp = _np(permuted_pair, np.int32)
    rw = _np(rows, np.int32)
    out = np.zeros((len(rw), W.H), np.float64)
    h = np.zeros((len(rw), W.I), np.float64) if want_h else None
    rc = lib().oracle_expert_rows(C.byref(W.struct), _ptr(xa), DTYPE_CODE[act] if isinstance(act, str) else act,
                                  _ptr(xs), T, k, E, n_shared, _ptr(off), _ptr(pp), _ptr(rw), len(rw),
                                  _ptr(h), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_expert_rows: row outside every group")
    return (out, h) if want_h else out


def layer_tokens(W: Weights, x, act, T, k, E, n_shared, ids, scales, tokens, x_scale=None):
    """The layer output (fp64 [len(tokens), H]) by its definition.
    act "fp8": x holds e4m3 codes with 1x128 scales x_scale [T, H/128]."""
    xa = _np(x)
    xs = _np(x_scale, np.float32)
    ia = _np(ids, np.int32)
    sa = _np(scales, np.float64)
    tk = _np(tokens, np.int32)
    y = np.zeros((len(tk), W.H), np.float64)
    rc = lib().oracle_layer_tokens(C.byref(W.struct), _ptr(xa),
                                   DTYPE_CODE[act] if isinstance(act, str) else act,
                                   _ptr(xs), T, k, E, n_shared, _ptr(ia), _ptr(sa), _ptr(tk), len(tk),
                                   _ptr(y))
    if rc != 0:
        raise ValueError("oracle_layer_tokens: token out of range")
    return y


def finalize(fc2, dt, unpermute, scales, T, k, H, n_shared=0):
    """fp64 [T, H] weighted sum of the FFN rows."""
    f = _np(fc2)
    up = _np(unpermute, np.int32)
    sa = _np(scales, np.float64)
    y = np.zeros((T, H), np.float64)
    lib().oracle_finalize(_ptr(f), DTYPE_CODE[dt] if isinstance(dt, str) else dt, _ptr(up),
                          _ptr(sa), T, k, H, n_shared, _ptr(y))
    return y
