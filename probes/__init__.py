"""Measurement probes for the benchmark (kq_probe.h): a plain streaming read
and a plain int8 matrix-core loop, built into libkq_probe.so beside this
file by quant_matmul_amd/build.py.  They are not part of the matmul library;
bench.py uses them to put an "achievable on this machine" figure beside the
datasheet peaks."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (torch's HIP runtime first, as for libkq.so)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq_probe.so")
SYMBOLS = ("kq_probe_read", "kq_probe_read_u", "kq_probe_mfma_i8")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python quant_matmul_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)
_p, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.kq_probe_read.argtypes = [_p, ctypes.c_size_t, _p, _int, _p]
lib.kq_probe_read.restype = _int
lib.kq_probe_read_u.argtypes = [_p, ctypes.c_size_t, _p, _int, _int, _p]
lib.kq_probe_read_u.restype = _int
lib.kq_probe_mfma_i8.argtypes = [_i64, _int, _p, _p]
lib.kq_probe_mfma_i8.restype = _int


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _ptr(t):
    return t if isinstance(t, int) else t.data_ptr()


def _ok(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def kq_probe_read(buf, nbytes: int, sink, grid: int, stream=None):
    """Streaming-read probe: reads nbytes at buf once."""
    _ok(lib.kq_probe_read(_ptr(buf), nbytes, _ptr(sink), grid, _stream(stream)), "kq_probe_read")


def kq_probe_read_u(buf, nbytes: int, sink, grid: int, unroll: int, stream=None):
    """Streaming-read probe with `unroll` loads in flight per thread."""
    _ok(lib.kq_probe_read_u(_ptr(buf), nbytes, _ptr(sink), grid, unroll, _stream(stream)), "kq_probe_read_u")


def kq_probe_mfma_i8(iters: int, grid: int, sink, stream=None):
    """Matrix-core probe: grid*4*iters*4 int8 32x32x32 MFMAs."""
    _ok(lib.kq_probe_mfma_i8(iters, grid, _ptr(sink), _stream(stream)), "kq_probe_mfma_i8")
