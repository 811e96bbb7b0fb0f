"""CPU tier: libkq.so loads, exports every entry point include/kq.h declares
(and the benchmark's probe library every entry point of probes/kq_probe.h),
and rejects bad arguments with the documented status code before any HIP
call (so these run on a host without a GPU; no call here reaches a kernel
launch)."""
import os
import re

import pytest

import probes
import quant_matmul_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", "kq.h")]
PROBE_HEADER = os.path.join(ROOT, "probes", "kq_probe.h")

GOOD16 = 0x10000   # fake but 16-byte aligned "device pointers": never dereferenced,
GOOD16B = 0x20000  # every call below fails validation first
ODD = 0x10001


def header_symbols(headers):
    text = "".join(open(h).read() for h in headers)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_symbols(HEADERS)
    assert set(names) == set(kq.SYMBOLS)
    for name in names:
        assert hasattr(kq.lib, name), name
    # the probes live in their own library, not in libkq.so
    pnames = header_symbols([PROBE_HEADER])
    assert set(pnames) == set(probes.SYMBOLS)
    for name in pnames:
        assert hasattr(probes.lib, name), name
        assert not hasattr(kq.lib, name), name


def test_record_and_packed_bytes():
    assert [kq.kq_record_bytes(f) for f in (4, 5, 6)] == [144, 176, 210]
    assert kq.kq_record_bytes(7) == 0
    for fmt, rb in ((4, 144), (5, 176), (6, 210)):
        for n, k in ((1, 256), (17, 2560), (9728, 2560), (2560, 9728)):
            b = kq.kq_packed_bytes(fmt, n, k)
            base = n * (k // 256) * rb
            assert base <= b <= base + 4 * 255
            assert b % 256 == 0
    assert kq.kq_packed_bytes(4, 0, 256) == 0
    assert kq.kq_packed_bytes(4, 4, 300) == 0
    assert kq.kq_packed_bytes(4, 4, 0) == 0
    assert kq.kq_packed_bytes(9, 4, 256) == 0


def _gemv(fmt=4, w=GOOD16, n=16, k=256, xq=GOOD16, xs=GOOD16, xbs=GOOD16, t=1, y=GOOD16):
    return kq.lib.kq_gemv(fmt, w, n, k, xq, xs, xbs, t, y, None)


def test_gemv_argument_checks():
    assert _gemv(fmt=3) == kq.KQ_EFORMAT
    assert _gemv(fmt=7) == kq.KQ_EFORMAT
    assert _gemv(k=300) == kq.KQ_EINVAL
    assert _gemv(k=0) == kq.KQ_EINVAL
    assert _gemv(n=0) == kq.KQ_EINVAL
    assert _gemv(n=-5) == kq.KQ_EINVAL
    assert _gemv(t=0) == kq.KQ_EINVAL
    assert _gemv(t=9) == kq.KQ_EINVAL
    for name in ("w", "xq", "xs", "xbs", "y"):
        assert _gemv(**{name: None}) == kq.KQ_EINVAL, name
    for name in ("w", "xq", "xbs"):
        assert _gemv(**{name: GOOD16 + 4}) == kq.KQ_EALIGN, name
    for name in ("xs", "y"):
        assert _gemv(**{name: ODD}) == kq.KQ_EALIGN, name


def _gemm_tiles(fmt=4, w=GOOD16, n=16, k=256, xq=GOOD16, xs=GOOD16, xbs=GOOD16, m=4, y=GOOD16, ws=None, wsb=0):
    return kq.lib.kq_gemm_tiles(fmt, w, n, k, xq, xs, xbs, m, y, ws, wsb, None)


def _gemm(fmt=4, w=GOOD16, n=16, k=256, xq=GOOD16, xs=GOOD16, xbs=GOOD16, m=4, y=GOOD16, ws=GOOD16B, wsb=None):
    if wsb is None:
        wsb = kq.kq_gemm_workspace_bytes(fmt, n, k, m)
    return kq.lib.kq_gemm(fmt, w, n, k, xq, xs, xbs, m, y, ws, wsb, None)


def test_gemm_tiles_argument_checks():
    assert _gemm_tiles(fmt=8) == kq.KQ_EFORMAT
    assert _gemm_tiles(k=512 + 16) == kq.KQ_EINVAL
    assert _gemm_tiles(m=0) == kq.KQ_EINVAL
    assert _gemm_tiles(xq=None) == kq.KQ_EINVAL
    assert _gemm_tiles(w=GOOD16 + 8) == kq.KQ_EALIGN
    # the workspace is optional, and 256-byte aligned when given
    assert _gemm_tiles(ws=GOOD16 + 16, wsb=1 << 20, y=ODD) == kq.KQ_EALIGN
    assert _gemm_tiles(ws=GOOD16 + 16, wsb=1 << 20) == kq.KQ_EALIGN


def test_gemm_row_image_argument_checks():
    # kq_gemm reads kq_quantize_q8k's row image and needs its workspace
    assert _gemm(fmt=8) == kq.KQ_EFORMAT
    assert _gemm(k=512 + 16) == kq.KQ_EINVAL
    assert _gemm(m=0) == kq.KQ_EINVAL
    assert _gemm(xbs=None) == kq.KQ_EINVAL
    assert _gemm(ws=None) == kq.KQ_EINVAL
    need = kq.kq_gemm_workspace_bytes(4, 16, 256, 4)
    assert _gemm(wsb=need - 1) == kq.KQ_EINVAL
    assert _gemm(ws=GOOD16B + 16) == kq.KQ_EALIGN
    assert _gemm(xbs=GOOD16 + 8) == kq.KQ_EALIGN  # the row image's int16 bsums: 16-byte aligned
    p = kq.lib.kq_gemm_partials
    assert p(4, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 4, GOOD16, GOOD16, GOOD16, None, need, None) == kq.KQ_EINVAL
    assert p(4, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 4, GOOD16, None, GOOD16, GOOD16B, need, None) == kq.KQ_EINVAL


def test_gemm_workspace_bytes():
    # on 256 CUs (2 x 256 workgroup slots; a host without a GPU assumes 256):
    # W_down at pp512 (160 tiles of 256 x 32) splits all its tiles in 3,
    # W_up (608 tiles, more than one round) runs unsplit; the tile GEMM's
    # workspace is one 8-byte counter per split tile (rounded up to 256
    # bytes), then the partial tiles
    tile = 256 * 32 * 4
    assert kq.kq_gemm_tiles_workspace_bytes("q6_k", 2560, 9728, 512) == 1280 + 160 * 3 * tile
    assert kq.kq_gemm_tiles_workspace_bytes("q4_k", 9728, 2560, 512) == 0
    assert kq.kq_gemm_tiles_workspace_bytes("q4_k", 8192, 2560, 512) == 0  # exactly one round
    # the 32-token tile (m <= 192): S = 3 partial slices of the m x n output
    assert kq.kq_gemm_tiles_workspace_bytes("q4_k", 300, 2560, 100) > 0
    assert kq.kq_gemm_tiles_workspace_bytes("q4_k", 300, 300, 130) == 0
    assert kq.kq_gemm_tiles_workspace_bytes(9, 300, 2560, 130) == 0
    # kq_gemm's workspace: the tile image (codes, then f16 bsums, each
    # 256-byte aligned) in front of the tile GEMM's own
    for fmt, n, k, m in (("q6_k", 2560, 9728, 512), ("q4_k", 9728, 2560, 512), ("q5_k", 300, 2560, 100),
                         ("q4_k", 17, 256, 1)):
        codes = kq.kq_q8k_tiles_bytes(m, k)
        img = (codes + 255) // 256 * 256 + (codes // 8 + 255) // 256 * 256
        assert kq.kq_gemm_workspace_bytes(fmt, n, k, m) == img + kq.kq_gemm_tiles_workspace_bytes(fmt, n, k, m)
    assert kq.kq_gemm_workspace_bytes(9, 300, 2560, 130) == 0


def test_gemm_noalloc_size_limit():
    # kq_gemm_noalloc takes no workspace: shapes whose kq_gemm workspace is
    # larger than the library's array are refused before any device call
    f = kq.lib.kq_gemm_noalloc
    assert kq.kq_gemm_workspace_bytes(4, 5120, 17408, 8192) > kq.KQ_SCRATCH_BYTES
    assert f(4, GOOD16, 5120, 17408, GOOD16, GOOD16, GOOD16, 8192, GOOD16, None) == kq.KQ_EINVAL
    assert f(9, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 4, GOOD16, None) == kq.KQ_EFORMAT
    assert f(4, GOOD16, 16, 256, None, GOOD16, GOOD16, 4, GOOD16, None) == kq.KQ_EINVAL
    assert f(4, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16 + 2, 4, GOOD16, None) == kq.KQ_EALIGN


def test_gemm_tile_choice():
    # m <= 192: the 32-token tile; from 193 tokens the 256-token tile
    for m, tok in ((1, 32), (64, 32), (192, 32), (193, 256), (200, 256), (512, 256)):
        assert kq.kq_gemm_tile_tokens("q4_k", 9728, 2560, m) == tok
    assert kq.kq_gemm_tile_tokens("q4_k", 9728, 300, 64) == 0
    assert kq.kq_gemm_tile_tokens(3, 9728, 2560, 64) == 0


def test_gemm_k_bound():
    kmax = (1 << 23) - 256
    assert _gemm_tiles(k=kmax + 256) == kq.KQ_EINVAL
    assert _gemm(k=kmax + 256, wsb=1 << 40) == kq.KQ_EINVAL
    # the bound is the GEMM's: the GEMV takes the same k (fails later, on alignment)
    assert kq.lib.kq_gemv(4, GOOD16, 16, kmax + 256, GOOD16, GOOD16, GOOD16, 1, ODD, None) == kq.KQ_EALIGN
    assert _gemm_tiles(k=kmax, y=ODD) == kq.KQ_EALIGN


def test_tile_image_bytes_and_checks():
    assert kq.kq_q8k_tiles_bytes(1, 256) == 32 * 256
    assert kq.kq_q8k_tiles_bytes(32, 512) == 32 * 512
    assert kq.kq_q8k_tiles_bytes(33, 2560) == 64 * 2560
    assert kq.kq_q8k_tiles_bytes(512, 9728) == 512 * 9728
    assert kq.kq_q8k_tiles_bytes(0, 256) == 0 and kq.kq_q8k_tiles_bytes(4, 100) == 0
    q = kq.lib.kq_quantize_q8k_tiles
    assert q(GOOD16, 0, 256, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert q(GOOD16, 1, 300, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert q(GOOD16, 1, 256, None, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert q(GOOD16, 1, 256, GOOD16 + 8, GOOD16, GOOD16, None) == kq.KQ_EALIGN
    # the grid bound: (t + 15) * k/256 chunks at most 2^32
    assert q(GOOD16, (1 << 31) - 1, 1 << 16, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL


def test_gather_and_grouped_argument_checks():
    g = kq.lib.kq_quantize_q8k_tiles_gather
    assert g(GOOD16, 4, 256, None, 32, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert g(GOOD16, 4, 256, GOOD16, 0, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert g(GOOD16, 4, 300, GOOD16, 32, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert g(GOOD16, 4, 256, GOOD16 + 2, 32, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EALIGN
    f = kq.lib.kq_gemm_grouped
    stride = kq.kq_packed_bytes(4, 96, 512)

    def call(fmt=4, stride=stride, experts=4, te=GOOD16, n=96, k=512, m=64):
        return f(fmt, GOOD16, stride, experts, te, n, k, GOOD16, GOOD16, GOOD16, m, GOOD16, None)
    assert call(fmt=2) == kq.KQ_EFORMAT
    assert call(te=None) == kq.KQ_EINVAL
    assert call(experts=0) == kq.KQ_EINVAL
    assert call(stride=stride - 256) == kq.KQ_EINVAL  # smaller than one expert's planes
    assert call(stride=stride + 8) == kq.KQ_EALIGN
    assert call(te=GOOD16 + 2) == kq.KQ_EALIGN
    assert call(m=0) == kq.KQ_EINVAL


def test_partials_argument_checks():
    for f in (kq.lib.kq_gemv_partials, kq.lib.kq_gemm_tiles_partials):
        # P missing
        assert f(4, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 1, GOOD16, None, GOOD16, None) == kq.KQ_EINVAL
        # M missing is an error for Q4_K / Q5_K ...
        assert f(5, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 1, GOOD16, GOOD16, None, None) == kq.KQ_EINVAL
        # ... and misaligned partials are rejected
        assert f(6, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 1, GOOD16, ODD, None, None) == kq.KQ_EALIGN


def test_fused_gemv_argument_checks():
    f = kq.lib.kq_gemv_f32
    ok = dict(fmt=4, w=GOOD16, n=16, k=256, x=GOOD16, t=1, y=GOOD16, xq=None, xs=None, xbs=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["fmt"], a["w"], a["n"], a["k"], a["x"], a["t"], a["y"], a["xq"], a["xs"], a["xbs"], None)
    assert call(fmt=0) == kq.KQ_EFORMAT
    assert call(k=384) == kq.KQ_EINVAL
    assert call(t=0) == kq.KQ_EINVAL and call(t=9) == kq.KQ_EINVAL
    assert call(x=None) == kq.KQ_EINVAL and call(y=None) == kq.KQ_EINVAL
    # the image buffers come all three or none, and batches past 2 need them
    assert call(xq=GOOD16) == kq.KQ_EINVAL
    assert call(t=3) == kq.KQ_EINVAL
    assert call(x=GOOD16 + 4) == kq.KQ_EALIGN
    assert call(xq=GOOD16 + 4, xs=GOOD16, xbs=GOOD16) == kq.KQ_EALIGN
    # the one-kernel form stages the image and its scales in LDS: past
    # 147456 bytes (k = 129024 at t = 1, 64512 at t = 2) the call needs the
    # image buffers for its two launches
    assert call(k=129280) == kq.KQ_EINVAL
    assert call(t=2, k=64768) == kq.KQ_EINVAL


def test_quantize_and_pack_argument_checks():
    q = kq.lib.kq_quantize_q8k
    assert q(GOOD16, 0, 256, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert q(GOOD16, 1, 100, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert q(None, 1, 256, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EINVAL
    assert q(GOOD16 + 4, 1, 256, GOOD16, GOOD16, GOOD16, None) == kq.KQ_EALIGN
    for f in (kq.lib.kq_pack, kq.lib.kq_unpack):
        assert f(1, GOOD16, 4, 256, GOOD16B, None) == kq.KQ_EFORMAT
        assert f(4, GOOD16, 4, 255, GOOD16B, None) == kq.KQ_EINVAL
        assert f(4, None, 4, 256, GOOD16B, None) == kq.KQ_EINVAL
        assert f(6, GOOD16 + 2, 4, 256, GOOD16B, None) == kq.KQ_EALIGN


def test_strerror_and_python_error():
    assert kq.kq_strerror(0) == "ok"
    assert "format" in kq.kq_strerror(kq.KQ_EFORMAT)
    assert "unknown" in kq.kq_strerror(12345)
    with pytest.raises(kq.KqError) as e:
        kq.kq_gemv(9, GOOD16, 16, 256, GOOD16, GOOD16, GOOD16, 1, GOOD16, stream=0)
    assert e.value.code == kq.KQ_EFORMAT


def test_probe_arg_checks():
    lib = probes.lib
    assert lib.kq_probe_read(None, 1024, GOOD16, 256, None) == kq.KQ_EINVAL
    assert lib.kq_probe_read(GOOD16, 1000, GOOD16, 256, None) == kq.KQ_EINVAL  # not a multiple of 16
    assert lib.kq_probe_read(GOOD16, 1024, GOOD16, 0, None) == kq.KQ_EINVAL
    assert lib.kq_probe_read(ODD, 1024, GOOD16, 256, None) == kq.KQ_EALIGN
    assert lib.kq_probe_mfma_i8(0, 256, GOOD16, None) == kq.KQ_EINVAL
    assert lib.kq_probe_mfma_i8(1 << 25, 256, GOOD16, None) == kq.KQ_EINVAL
    assert lib.kq_probe_mfma_i8(10, 70000, GOOD16, None) == kq.KQ_EINVAL
    assert lib.kq_probe_mfma_i8(10, 256, ODD, None) == kq.KQ_EALIGN
