"""CPU oracle of the K-quant x Q8_K matmul -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It wraps the plain scalar C in kq_oracle.c (built
with gcc into liboracle.so next to this file) and shares nothing with the
HIP library.  See kq_oracle.c for what each function follows on the
K-quant kernel arc page.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FORMATS = {"q4_k": 4, "q5_k": 5, "q6_k": 6}
QK = 256


def build() -> str:
    """Compile kq_oracle.c with gcc (strict IEEE: no fast-math, no FMA
    contraction) into liboracle.so."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_double.restype = ctypes.c_double
        lib.orc_dequantize.argtypes = [ctypes.c_int, p, i64, i64, p]
        lib.orc_quantize_q8k.argtypes = [p, i64, i64, p, p, p]
        lib.orc_partials.argtypes = [ctypes.c_int, p, i64, i64, p, p, i64, p, p]
        lib.orc_matmul.argtypes = [ctypes.c_int, p, i64, i64, p, p, p, i64, p]
        lib.orc_rowmag.argtypes = [ctypes.c_int, p, i64, i64, p, p, i64, p]
        lib.orc_decode.argtypes = [ctypes.c_int, p, p]
        for f in ("orc_dequantize", "orc_quantize_q8k", "orc_partials", "orc_matmul",
                  "orc_rowmag", "orc_decode"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc == -2:
        raise OverflowError(f"{what}: an int32 partial overflowed")
    if rc != 0:
        raise ValueError(f"{what}: bad arguments (rc={rc})")


def f16_to_double(bits: int) -> float:
    return _load().orc_f16_to_double(bits)


class Block(ctypes.Structure):
    _fields_ = [("d", ctypes.c_double), ("dmin", ctypes.c_double),
                ("sc", ctypes.c_int * 16), ("m", ctypes.c_int * 16),
                ("q", ctypes.c_int * 256)]


def decode(fmt: str, rec: np.ndarray) -> dict:
    """Decoded integer fields of one superblock record."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    b = Block()
    _check(_load().orc_decode(FORMATS[fmt], _ptr(rec), ctypes.byref(b)), "decode")
    nsub = 16 if fmt == "q6_k" else 8
    return {"d": b.d, "dmin": b.dmin, "sc": np.array(b.sc[:nsub]),
            "m": np.array(b.m[:nsub]), "q": np.array(b.q[:])}


def dequantize(fmt: str, recs: np.ndarray) -> np.ndarray:
    """recs (n, k/256, bytes) uint8 -> w (n, k) float64."""
    recs = np.ascontiguousarray(recs, dtype=np.uint8)
    n, nsb = recs.shape[:2]
    w = np.empty((n, nsb * QK), np.float64)
    _check(_load().orc_dequantize(FORMATS[fmt], _ptr(recs), n, nsb * QK, _ptr(w)), "dequantize")
    return w


def quantize_q8k(x: np.ndarray):
    """x (t, k) float32 -> (xq int8 (t,k), xs float32 (t,k/256), xbs int16 (t,k/16))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    t, k = x.shape
    xq = np.empty((t, k), np.int8)
    xs = np.empty((t, k // QK), np.float32)
    xbs = np.empty((t, k // 16), np.int16)
    _check(_load().orc_quantize_q8k(_ptr(x), t, k, _ptr(xq), _ptr(xs), _ptr(xbs)), "quantize_q8k")
    return xq, xs, xbs


def partials(fmt: str, recs: np.ndarray, xq: np.ndarray, xbs: np.ndarray):
    """Per-superblock int32 partials P, M of shape (t, n, k/256)."""
    recs = np.ascontiguousarray(recs, dtype=np.uint8)
    n, nsb = recs.shape[:2]
    t = xq.shape[0]
    P = np.empty((t, n, nsb), np.int32)
    M = np.empty((t, n, nsb), np.int32)
    _check(_load().orc_partials(FORMATS[fmt], _ptr(recs), n, nsb * QK,
                                _ptr(np.ascontiguousarray(xq)), _ptr(np.ascontiguousarray(xbs)),
                                t, _ptr(P), _ptr(M)), "partials")
    return P, M


def matmul(fmt: str, recs: np.ndarray, xq: np.ndarray, xs: np.ndarray, xbs: np.ndarray):
    """y (t, n) float64 from the per-superblock integer folds."""
    recs = np.ascontiguousarray(recs, dtype=np.uint8)
    n, nsb = recs.shape[:2]
    t = xq.shape[0]
    y = np.empty((t, n), np.float64)
    _check(_load().orc_matmul(FORMATS[fmt], _ptr(recs), n, nsb * QK,
                              _ptr(np.ascontiguousarray(xq)), _ptr(np.ascontiguousarray(xs)),
                              _ptr(np.ascontiguousarray(xbs)), t, _ptr(y)), "matmul")
    return y


def rowmag(fmt: str, recs: np.ndarray, xq: np.ndarray, xs: np.ndarray):
    """R (t, n) = sum_i |w_i * d8 * a_i|, the row-magnitude tolerance scale."""
    recs = np.ascontiguousarray(recs, dtype=np.uint8)
    n, nsb = recs.shape[:2]
    t = xq.shape[0]
    R = np.empty((t, n), np.float64)
    _check(_load().orc_rowmag(FORMATS[fmt], _ptr(recs), n, nsb * QK,
                              _ptr(np.ascontiguousarray(xq)), _ptr(np.ascontiguousarray(xs)),
                              t, _ptr(R)), "rowmag")
    return R
