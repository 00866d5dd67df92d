"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes marshalling over ``oracle.c`` (plain C, fp64). Only the
tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package; the HIP library never does, and this package imports
nothing from it. Inputs are canonical GGUF block bytes (see ``synth``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

TYPE_Q4_0 = 2
TYPE_Q8_0 = 8
TYPE_Q4_K = 12
TYPE_Q5_K = 13
TYPE_Q6_K = 14


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.or_fp16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_fp16_to_f64.restype = ctypes.c_double
        L.or_f32_to_fp16_rne.argtypes = [ctypes.c_float]
        L.or_f32_to_fp16_rne.restype = ctypes.c_uint16
        L.or_block_bytes.argtypes = [ctypes.c_int]
        L.or_block_bytes.restype = ctypes.c_size_t
        L.or_block_elems.argtypes = [ctypes.c_int]
        L.or_block_elems.restype = I64
        L.or_dequantize.argtypes = [ctypes.c_int, P, I64, I64, P]
        L.or_matvec.argtypes = [ctypes.c_int, P, I64, I64, P, P, P]
        L.or_matvec_rows.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P, P, P]
        L.or_quantize_q8_0.argtypes = [P, I64, I64, P, P]
        L.or_blockdots.argtypes = [ctypes.c_int, P, I64, I64, P, P, I64, P, P, P]
        L.or_gelu_tanh.argtypes = [ctypes.c_double]
        L.or_gelu_tanh.restype = ctypes.c_double
        L.or_ffn_gate_up.argtypes = [ctypes.c_int, P, P, I64, I64, P, P, P, P, P, P]
        L.or_rmsnorm.argtypes = [P, I64, P, ctypes.c_double, P]
        L.or_softcap.argtypes = [ctypes.c_double, ctypes.c_double]
        L.or_softcap.restype = ctypes.c_double
        L.or_argmax_f32.argtypes = [P, I64]
        L.or_argmax_f32.restype = I64
        for f in ("or_dequantize", "or_matvec", "or_matvec_rows", "or_quantize_q8_0",
                  "or_blockdots", "or_ffn_gate_up", "or_rmsnorm"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _blocks_u8(blocks):
    b = np.ascontiguousarray(blocks)
    return b.view(np.uint8).reshape(-1)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def fp16_to_f64(bits: int) -> float:
    return lib().or_fp16_to_f64(int(bits))


def fp16_to_f64_array(bits) -> np.ndarray:
    f = lib().or_fp16_to_f64
    bits = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([f(int(b)) for b in bits], dtype=np.float64)


def f32_to_fp16(x: float) -> int:
    return int(lib().or_f32_to_fp16_rne(float(np.float32(x))))


def block_elems(qtype) -> int:
    return int(lib().or_block_elems(qtype))


def dequantize(qtype, blocks, n, k) -> np.ndarray:
    w = np.empty((n, k), dtype=np.float64)
    _check(lib().or_dequantize(qtype, _p(_blocks_u8(blocks)), n, k, _p(w)), "dequantize")
    return w


def matvec(qtype, blocks, n, k, x):
    """Returns (y, a): y = W x in fp64, a = sum |w x| per row."""
    xd = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    assert xd.size == k
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    _check(lib().or_matvec(qtype, _p(_blocks_u8(blocks)), n, k, _p(xd), _p(y), _p(a)), "matvec")
    return y, a


def matvec_rows(qtype, blocks, n, k, rows, x):
    xd = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    y = np.empty(rows.size, dtype=np.float64)
    a = np.empty(rows.size, dtype=np.float64)
    _check(lib().or_matvec_rows(qtype, _p(_blocks_u8(blocks)), n, k, _p(rows), rows.size,
                                _p(xd), _p(y), _p(a)), "matvec_rows")
    return y, a


def quantize_q8_0(x):
    """x [m][k] fp32 -> (xq int8 [m][k], xd uint16 [m][k/32])."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim == 1:
        x = x.reshape(1, -1)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.int8)
    xd = np.empty((m, k // 32), dtype=np.uint16)
    _check(lib().or_quantize_q8_0(_p(x), m, k, _p(xq), _p(xd)), "quantize_q8_0")
    return xq, xd


def blockdots(qtype, blocks, n, k, xq, xd, want_s=True):
    """Integer path. Returns (S int32 [m][n][k/32] or None, y [m][n], a [m][n])."""
    xq = np.ascontiguousarray(np.asarray(xq, dtype=np.int8))
    xd = np.ascontiguousarray(np.asarray(xd, dtype=np.uint16))
    if xq.ndim == 1:
        xq = xq.reshape(1, -1)
        xd = xd.reshape(1, -1)
    m = xq.shape[0]
    S = np.empty((m, n, k // 32), dtype=np.int32) if want_s else None
    y = np.empty((m, n), dtype=np.float64)
    a = np.empty((m, n), dtype=np.float64)
    _check(lib().or_blockdots(qtype, _p(_blocks_u8(blocks)), n, k, _p(xq), _p(xd), m,
                              _p(S), _p(y), _p(a)), "blockdots")
    return S, y, a


def gelu_tanh(t: float) -> float:
    return lib().or_gelu_tanh(float(t))


def gelu_tanh_array(t) -> np.ndarray:
    f = lib().or_gelu_tanh
    t = np.asarray(t, dtype=np.float64).reshape(-1)
    return np.array([f(float(v)) for v in t], dtype=np.float64)


def ffn_gate_up(qtype, gblocks, ublocks, n_ff, k, x):
    """Returns dict g, u, h, ag, au (all fp64 [n_ff])."""
    xd = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    out = {name: np.empty(n_ff, dtype=np.float64) for name in ("g", "u", "h", "ag", "au")}
    _check(lib().or_ffn_gate_up(qtype, _p(_blocks_u8(gblocks)), _p(_blocks_u8(ublocks)),
                                n_ff, k, _p(xd), _p(out["g"]), _p(out["u"]), _p(out["h"]),
                                _p(out["ag"]), _p(out["au"])), "ffn_gate_up")
    return out


def rmsnorm(x, w=None, eps=1e-6):
    """x * (mean(x^2) + eps)^-1/2 * w in fp64 (w None: no scale)."""
    xd = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    wd = None if w is None else np.ascontiguousarray(np.asarray(w, dtype=np.float64).reshape(-1))
    out = np.empty_like(xd)
    _check(lib().or_rmsnorm(_p(xd), xd.size, _p(wd), float(eps), _p(out)), "rmsnorm")
    return out


def softcap(y, cap):
    f = lib().or_softcap
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    return np.array([f(float(v), float(cap)) for v in y], dtype=np.float64)


def argmax_f32(v):
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(-1))
    return int(lib().or_argmax_f32(_p(v), v.size))


# Tolerances stated by the method's accuracy contract.
def fp32_path_bound(a):
    """|y_gpu - y_ref| <= 1e-4 * sum|w x| + 1e-6 for the fp32-activation path."""
    return 1e-4 * np.asarray(a) + 1e-6


GELU_LIPSCHITZ = 1.13  # >= max |G'(t)| of the tanh GELU (about 1.1290 near t = 1.42)


def ffn_h_bound(g, u, ag, au, h_ref):
    """First-order bound for h = G(g) u given the fp32-path bounds on g and u."""
    tg = fp32_path_bound(ag)
    tu = fp32_path_bound(au)
    G = np.array([gelu_tanh(v) for v in np.asarray(g).reshape(-1)])
    return (GELU_LIPSCHITZ * np.abs(u) * tg + (np.abs(G) + GELU_LIPSCHITZ * tg) * tu
            + 1e-6 * np.abs(h_ref) + 1e-6)
