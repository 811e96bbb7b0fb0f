"""Python binding of the kq C ABI (include/kq.h) for AMD MI355X.

Argument marshalling only: every function below passes device pointers of
torch tensors and the current HIP stream to the same-named C entry point in
libkq.so, and raises KqError on a non-zero status.  Nothing here computes
any part of the matmul.  The library must have been built in-tree
(``python quant_matmul_amd/build.py``); importing this package without it
raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime; it must be the one in the process before
# libkq.so is loaded, so that libkq.so binds to it (same SONAME) instead of
# pulling in a second HIP/HSA runtime next to torch's.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq.so")

KQ_Q4_K, KQ_Q5_K, KQ_Q6_K = 4, 5, 6
FORMATS = {"q4_k": KQ_Q4_K, "q5_k": KQ_Q5_K, "q6_k": KQ_Q6_K}
KQ_OK, KQ_EINVAL, KQ_EFORMAT, KQ_EALIGN, KQ_ELAUNCH = 0, -1, -2, -3, -4

# every entry point of include/kq.h
SYMBOLS = ("kq_record_bytes", "kq_packed_bytes", "kq_pack", "kq_unpack", "kq_quantize_q8k",
           "kq_q8k_tiles_bytes", "kq_quantize_q8k_tiles", "kq_quantize_q8k_tiles_gather", "kq_gemv",
           "kq_gemv_f32", "kq_gemm_workspace_bytes", "kq_gemm", "kq_gemm_tiles_workspace_bytes",
           "kq_gemm_tile_tokens", "kq_gemm_tiles", "kq_gemm_grouped", "kq_gemv_partials", "kq_gemm_partials",
           "kq_gemm_tiles_partials", "kq_gemm_noalloc", "kq_strerror")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python quant_matmul_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)
_p, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.kq_record_bytes.argtypes = [_int]
lib.kq_record_bytes.restype = ctypes.c_size_t
lib.kq_packed_bytes.argtypes = [_int, _i64, _i64]
lib.kq_packed_bytes.restype = ctypes.c_size_t
lib.kq_pack.argtypes = [_int, _p, _i64, _i64, _p, _p]
lib.kq_unpack.argtypes = [_int, _p, _i64, _i64, _p, _p]
lib.kq_quantize_q8k.argtypes = [_p, _i64, _i64, _p, _p, _p, _p]
lib.kq_q8k_tiles_bytes.argtypes = [_i64, _i64]
lib.kq_q8k_tiles_bytes.restype = ctypes.c_size_t
lib.kq_quantize_q8k_tiles.argtypes = [_p, _i64, _i64, _p, _p, _p, _p]
lib.kq_quantize_q8k_tiles_gather.argtypes = [_p, _i64, _i64, _p, _i64, _p, _p, _p, _p]
lib.kq_gemm_grouped.argtypes = [_int, _p, _i64, _i64, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p]
lib.kq_gemv.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p]
lib.kq_gemm_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
lib.kq_gemm_workspace_bytes.restype = ctypes.c_size_t
lib.kq_gemm.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, ctypes.c_size_t, _p]
lib.kq_gemm_noalloc.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p]
lib.kq_gemm_tiles_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
lib.kq_gemm_tiles_workspace_bytes.restype = ctypes.c_size_t
lib.kq_gemm_tile_tokens.argtypes = [_int, _i64, _i64, _i64]
lib.kq_gemm_tile_tokens.restype = _int
lib.kq_gemm_tiles.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, ctypes.c_size_t, _p]
lib.kq_gemv_f32.argtypes = [_int, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
lib.kq_gemv_partials.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _p, _p]
lib.kq_gemm_partials.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _p, _p, ctypes.c_size_t, _p]
lib.kq_gemm_tiles_partials.argtypes = [_int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _p, _p]
lib.kq_strerror.argtypes = [_int]
lib.kq_strerror.restype = ctypes.c_char_p
for _f in ("kq_pack", "kq_unpack", "kq_quantize_q8k", "kq_quantize_q8k_tiles", "kq_quantize_q8k_tiles_gather",
           "kq_gemv", "kq_gemv_f32", "kq_gemm", "kq_gemm_tiles", "kq_gemm_grouped",
           "kq_gemv_partials", "kq_gemm_partials", "kq_gemm_tiles_partials", "kq_gemm_noalloc"):
    getattr(lib, _f).restype = _int


class KqError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {lib.kq_strerror(code).decode()} ({code})")


def _fmt(fmt) -> int:
    return FORMATS.get(fmt, fmt) if isinstance(fmt, str) else int(fmt)


def _ptr(t) -> int | None:
    """Device pointer of a torch tensor (or None / a raw int)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(rc: int, what: str):
    if rc != KQ_OK:
        raise KqError(rc, what)


def kq_record_bytes(fmt) -> int:
    return lib.kq_record_bytes(_fmt(fmt))


def kq_packed_bytes(fmt, n: int, k: int) -> int:
    return lib.kq_packed_bytes(_fmt(fmt), n, k)


def kq_pack(fmt, w_ggml, n: int, k: int, w_planes, stream=None):
    _ok(lib.kq_pack(_fmt(fmt), _ptr(w_ggml), n, k, _ptr(w_planes), _stream(stream)), "kq_pack")


def kq_unpack(fmt, w_planes, n: int, k: int, w_ggml, stream=None):
    _ok(lib.kq_unpack(_fmt(fmt), _ptr(w_planes), n, k, _ptr(w_ggml), _stream(stream)), "kq_unpack")


def kq_quantize_q8k(x, t: int, k: int, xq, xs, xbs, stream=None):
    _ok(lib.kq_quantize_q8k(_ptr(x), t, k, _ptr(xq), _ptr(xs), _ptr(xbs), _stream(stream)),
        "kq_quantize_q8k")


def kq_q8k_tiles_bytes(t: int, k: int) -> int:
    return lib.kq_q8k_tiles_bytes(t, k)


def kq_quantize_q8k_tiles(x, t: int, k: int, xq_tiles, xs, xbs, stream=None):
    _ok(lib.kq_quantize_q8k_tiles(_ptr(x), t, k, _ptr(xq_tiles), _ptr(xs), _ptr(xbs), _stream(stream)),
        "kq_quantize_q8k_tiles")


def kq_quantize_q8k_tiles_gather(x, t: int, k: int, rows, m: int, xq_tiles, xs, xbs, stream=None):
    _ok(lib.kq_quantize_q8k_tiles_gather(_ptr(x), t, k, _ptr(rows), m, _ptr(xq_tiles), _ptr(xs), _ptr(xbs),
                                         _stream(stream)), "kq_quantize_q8k_tiles_gather")


def kq_gemv(fmt, w_planes, n: int, k: int, xq, xs, xbs, t: int, y, stream=None):
    _ok(lib.kq_gemv(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq), _ptr(xs), _ptr(xbs), t, _ptr(y),
                    _stream(stream)), "kq_gemv")


def kq_gemv_f32(fmt, w_planes, n: int, k: int, x, t: int, y, xq=None, xs=None, xbs=None, stream=None):
    _ok(lib.kq_gemv_f32(_fmt(fmt), _ptr(w_planes), n, k, _ptr(x), t, _ptr(y), _ptr(xq), _ptr(xs),
                        _ptr(xbs), _stream(stream)), "kq_gemv_f32")


def _nbytes(buf, nbytes):
    if nbytes is not None:
        return nbytes
    return 0 if buf is None or isinstance(buf, int) else buf.numel() * buf.element_size()


def kq_gemm_workspace_bytes(fmt, n: int, k: int, m: int) -> int:
    return lib.kq_gemm_workspace_bytes(_fmt(fmt), n, k, m)


def kq_gemm(fmt, w_planes, n: int, k: int, xq, xs, xbs, m: int, y, workspace, workspace_bytes=None, stream=None):
    """GEMM on the row image of kq_quantize_q8k (workspace required)."""
    _ok(lib.kq_gemm(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq), _ptr(xs), _ptr(xbs), m, _ptr(y),
                    _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)), "kq_gemm")


KQ_SCRATCH_BYTES = 64 << 20


def kq_gemm_noalloc(fmt, w_planes, n: int, k: int, xq, xs, xbs, m: int, y, stream=None):
    """kq_gemm with the library's own device scratch array as its workspace."""
    _ok(lib.kq_gemm_noalloc(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq), _ptr(xs), _ptr(xbs), m, _ptr(y),
                            _stream(stream)), "kq_gemm_noalloc")


def kq_gemm_tiles_workspace_bytes(fmt, n: int, k: int, m: int) -> int:
    return lib.kq_gemm_tiles_workspace_bytes(_fmt(fmt), n, k, m)


def kq_gemm_tile_tokens(fmt, n: int, k: int, m: int) -> int:
    return lib.kq_gemm_tile_tokens(_fmt(fmt), n, k, m)


def kq_gemm_tiles(fmt, w_planes, n: int, k: int, xq_tiles, xs, xbs, m: int, y, workspace=None,
                  workspace_bytes=None, stream=None):
    """GEMM on the tile image of kq_quantize_q8k_tiles (workspace optional)."""
    _ok(lib.kq_gemm_tiles(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq_tiles), _ptr(xs), _ptr(xbs), m, _ptr(y),
                          _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)), "kq_gemm_tiles")


def kq_gemm_grouped(fmt, w_planes, w_stride: int, experts: int, tile_expert, n: int, k: int, xq_tiles, xs, xbs,
                    m: int, y, stream=None):
    _ok(lib.kq_gemm_grouped(_fmt(fmt), _ptr(w_planes), w_stride, experts, _ptr(tile_expert), n, k, _ptr(xq_tiles),
                            _ptr(xs), _ptr(xbs), m, _ptr(y), _stream(stream)), "kq_gemm_grouped")


def kq_gemv_partials(fmt, w_planes, n: int, k: int, xq, xs, xbs, t: int, y, P, M, stream=None):
    _ok(lib.kq_gemv_partials(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq), _ptr(xs), _ptr(xbs), t,
                             _ptr(y), _ptr(P), _ptr(M), _stream(stream)), "kq_gemv_partials")


def kq_gemm_partials(fmt, w_planes, n: int, k: int, xq, xs, xbs, m: int, y, P, M, workspace, workspace_bytes=None,
                     stream=None):
    _ok(lib.kq_gemm_partials(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq), _ptr(xs), _ptr(xbs), m, _ptr(y), _ptr(P),
                             _ptr(M), _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)),
        "kq_gemm_partials")


def kq_gemm_tiles_partials(fmt, w_planes, n: int, k: int, xq_tiles, xs, xbs, m: int, y, P, M, stream=None):
    _ok(lib.kq_gemm_tiles_partials(_fmt(fmt), _ptr(w_planes), n, k, _ptr(xq_tiles), _ptr(xs), _ptr(xbs), m,
                                   _ptr(y), _ptr(P), _ptr(M), _stream(stream)), "kq_gemm_tiles_partials")


def kq_strerror(code: int) -> str:
    return lib.kq_strerror(code).decode()
