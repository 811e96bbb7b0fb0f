"""GPU tier: the HIP path (through the C ABI) against the CPU oracle.

Bar (K-quant kernel arc page, "Testing" and the per-format-tune commit
message's tolerance rule): the Q8_K activation image and the per-superblock
int32 partials are bit-exact; float outputs agree within 1e-5 * R per
output, R = sum_i |w_i * xhat_i| -- a row-magnitude tolerance, because the
signed Q6_K sub-scales cancel inside a row and an element-relative bound
would trip on fold-order noise.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from q8k_cases import quotient_chunks
from q8k_tiles import bsum_tiles, from_bsum_tiles, from_tiles, to_tiles
from quant_matmul_amd import torch_ops as ops
import quant_matmul_amd as kq

pytestmark = pytest.mark.gpu
FMTS = ["q4_k", "q5_k", "q6_k"]
TOL = 1e-5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def fused_same_bits(t, k):
    """Whether kq_gemv_f32's y equals quantise-then-kq_gemv's bit for bit: the
    one-kernel form (t <= 2) takes 16-row steps on rows of at most 16
    superblocks and then sums each row's superblock folds in another order."""
    return t > 2 or k // 256 > 16


class Case:
    """Seeded weights and activations, the oracle's view and the device's."""

    def __init__(self, fmt, n, k, t, seed=1, x=None):
        self.fmt, self.n, self.k, self.t = fmt, n, k, t
        self.recs = synth.weights(fmt, n, k, seed)
        self.x = synth.activations(t, k, seed + 1000) if x is None else x
        self.q8_host = oracle.quantize_q8k(self.x)
        self.planes = ops.pack(fmt, ops.upload_records(self.recs), n, k)
        self.q8 = tuple(dev(a) for a in self.q8_host)
        # the GEMM's image: the same codes re-laid as the tile image
        self.q8t = (dev(to_tiles(self.q8_host[0])), self.q8[1], dev(bsum_tiles(self.q8_host[2])))

    def oracle_rows(self, rows=None):
        key = None if rows is None else tuple(rows)
        cache = self.__dict__.setdefault("_oracle", {})
        if key not in cache:
            cache[key] = self._oracle_rows(rows)
        return cache[key]

    def _oracle_rows(self, rows):
        recs = self.recs if rows is None else self.recs[rows]
        xq, xs, xbs = self.q8_host
        P, M = oracle.partials(self.fmt, recs, xq, xbs)
        y = oracle.matmul(self.fmt, recs, xq, xs, xbs)
        R = oracle.rowmag(self.fmt, recs, xq, xs)
        return y, P, M, R


def check(case, y, P, M, rows=None):
    y_o, P_o, M_o, R = case.oracle_rows(rows)
    y, P, M = host(y), host(P), host(M)
    if rows is not None:
        y, P, M = y[:, rows], P[:, rows], M[:, rows]
    assert np.array_equal(P, P_o), f"P mismatch at {np.argwhere(P != P_o)[:5]}"
    if case.fmt != "q6_k":
        assert np.array_equal(M, M_o), f"M mismatch at {np.argwhere(M != M_o)[:5]}"
    err = np.abs(y.astype(np.float64) - y_o)
    assert np.all(np.isfinite(y))
    bad = err > TOL * R
    assert not bad.any(), f"{bad.sum()} outputs beyond tolerance, worst ratio {np.max(err / R):.3g}"


def check_y(case, y, rows=None):
    y_o, _, _, R = case.oracle_rows(rows)
    y = host(y) if rows is None else host(y)[:, rows]
    assert np.all(np.isfinite(y))
    err = np.abs(y.astype(np.float64) - y_o)
    assert np.all(err <= TOL * R), f"worst ratio {np.max(err / R):.3g}"


# ------------------------------------------------------------ Q8_K ------
@pytest.mark.parametrize("t,k", [(1, 256), (3, 2560), (8, 9728), (512, 2560), (129, 768)])
def test_quantize_bit_exact(t, k):
    x = synth.activations(t, k, 40 + t)
    # edge chunks: all zero, a single value, exact .5 ties, tiny magnitudes
    x[0, :256] = 0.0
    if k >= 768:
        x[0, 256:512] = 0.0
        x[0, 300] = -0.3
        x[0, 512:768] = np.round(x[0, 512:768] * 20) / 2
        x[0, 512] = 127.0
    if t > 1:
        x[1, :256] *= np.float32(1e-30)
    xq, xs, xbs = ops.quantize_q8k(dev(x))
    rq, rs, rbs = oracle.quantize_q8k(x)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(xbs), rbs)


@pytest.mark.parametrize("t,k", [(1, 256), (32, 512), (21, 2560), (512, 9728), (130, 768)])
def test_quantize_tiles_bit_exact(t, k):
    x = synth.activations(t, k, 60 + t)
    x[0, :256] = 0.0
    xq, xs, xbs = ops.quantize_q8k_tiles(dev(x))
    rq, rs, rbs = oracle.quantize_q8k(x)
    codes = from_tiles(host(xq), t, k)
    assert np.array_equal(codes[:t], rq)
    assert not codes[t:].any()  # padding tokens are zero codes
    assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))
    bs = from_bsum_tiles(host(xbs), t, k)
    assert np.array_equal(bs[:t], rbs.astype(np.float64))
    assert not bs[t:].any()


def _every_quantiser_matches_oracle(x, seed):
    """Every device quantiser (row, tile, gather, and the one fused into the
    GEMV) gives the oracle's Q8_K bits for x[t][k]."""
    t, k = x.shape
    rq, rs, rbs = oracle.quantize_q8k(x)
    xd = dev(x)
    xq, xs, xbs = ops.quantize_q8k(xd)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(xbs), rbs)
    tq, ts, tbs = ops.quantize_q8k_tiles(xd)
    assert np.array_equal(from_tiles(host(tq), t, k)[:t], rq)
    assert np.array_equal(host(ts).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(from_bsum_tiles(host(tbs), t, k)[:t], rbs.astype(np.float64))
    # gathered rows in reverse order, with one padding index
    rows = np.concatenate([np.arange(t)[::-1], [-1]]).astype(np.int32)
    gq, gs, gbs = ops.quantize_q8k_tiles_gather(xd, dev(rows))
    assert np.array_equal(from_tiles(host(gq), t + 1, k)[:t], rq[::-1])
    assert np.array_equal(host(gs)[:t].view(np.uint32), rs[::-1].view(np.uint32))
    if t <= 8:
        n = 64
        recs = synth.weights("q4_k", n, k, seed)
        planes = ops.pack("q4_k", ops.upload_records(recs), n, k)
        _, (fq, fs, fbs) = ops.gemv_f32("q4_k", planes, n, k, xd, keep_image=True)
        assert np.array_equal(host(fq), rq)
        assert np.array_equal(host(fs).view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(host(fbs), rbs)
        if t <= 2:  # the one-kernel form quantises inside every workgroup
            y1 = ops.gemv_f32("q4_k", planes, n, k, xd)
            y2 = ops.gemv("q4_k", planes, n, k, (xq, xs, xbs))
            if fused_same_bits(t, k):
                assert torch.equal(y1, y2)
            else:
                d = np.abs(host(y1).astype(np.float64) - host(y2).astype(np.float64))
                assert np.all(d <= TOL * np.abs(host(y2)).max() + 1e-30)


@pytest.mark.parametrize("t,k", [(1, 2560), (2, 1024), (5, 1536), (40, 768), (300, 2560)])
def test_quantize_quotient_chunks_every_form(t, k):
    # chunks built so that rint(x/d8) and rint(x * (1/d8)) differ in many
    # places: every device quantiser must take the binary32 quotient, as
    # the oracle does
    nsb = k // 256
    x = synth.activations(t, k, 80 + t)
    edge = quotient_chunks(min(t * nsb, 12), seed=81 + t)
    x.reshape(-1, 256)[: len(edge)] = edge
    _every_quantiser_matches_oracle(x, 82)


@pytest.mark.parametrize("t,k", [(1, 2560), (2, 1024), (6, 768), (300, 1024)])
def test_quantize_tiny_and_huge_scales_every_form(t, k):
    # chunks scaled by powers of two from 2^-90 to 2^99 (d8 from about
    # 2^-95 to 2^94): below d8 = 2^-64 the device divides per value, above
    # it it multiplies by 1/d8 and corrects twice; both must give the
    # oracle's bits, the quotient-edge chunks included
    x = synth.activations(t, k, 85 + t).reshape(-1, 256)
    edge = quotient_chunks(min(len(x), 12), seed=86 + t)
    x[: len(edge)] = edge
    e = np.random.default_rng(87 + t).integers(-90, 100, size=len(x))
    e[: min(len(x), 4)] = [-90, -62, -58, 99][: min(len(x), 4)]
    x = (x.astype(np.float64) * np.ldexp(1.0, e)[:, None]).astype(np.float32).reshape(t, k)
    _every_quantiser_matches_oracle(x, 88)


# ------------------------------------------------------------ pack ------
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 256), (17, 2560), (300, 768)])
def test_pack_round_trip_and_planes(fmt, n, k):
    recs = synth.weights(fmt, n, k, 7)
    planes = ops.pack(fmt, ops.upload_records(recs), n, k)
    back = host(ops.unpack(fmt, planes, n, k))
    assert np.array_equal(back, recs.reshape(-1))
    # the planes are the record fields regrouped, each plane 256-B aligned
    fields = {"q4_k": [(0, 16), (16, 144)], "q5_k": [(0, 16), (16, 48), (48, 176)],
              "q6_k": [(0, 128), (128, 192), (192, 208), (208, 210)]}[fmt]
    p = host(planes)
    off = 0
    flat = recs.reshape(n * (k // 256), -1)
    for a, b in fields:
        size = flat.shape[0] * (b - a)
        assert np.array_equal(p[off:off + size], flat[:, a:b].reshape(-1))
        off += (size + 255) // 256 * 256
    assert off == len(p)


# ------------------------------------------------------------ GEMV ------
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(256, 2560), (37, 256), (1, 512), (17, 9728)])
def test_gemv_parity(fmt, t, n, k):
    c = Case(fmt, n, k, t, seed=10 * t + n)
    y, P, M = ops.matmul_partials("gemv", fmt, c.planes, n, k, c.q8)
    check(c, y, P, M)
    # the production entry point runs the same body without the stores
    y2 = ops.gemv(fmt, c.planes, n, k, c.q8)
    assert torch.equal(y, y2)


# ------------------------------------------------- fused quantise+GEMV --
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("t", [1, 2, 3, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(256, 2560), (37, 256), (2560, 9728), (9728, 2560)])
def test_gemv_f32_fused_matches_two_step(fmt, t, n, k):
    c = Case(fmt, n, k, t, seed=30 + t)
    xd = dev(c.x)
    y, (xq, xs, xbs) = ops.gemv_f32(fmt, c.planes, n, k, xd, keep_image=True)
    # the fused quantiser writes the same Q8_K image bits as the oracle
    rq, rs, rbs = c.q8_host
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(xbs), rbs)
    # and the same y as quantise-then-GEMV: bit for bit, except that the
    # one-kernel form on rows of at most 16 superblocks sums a row's
    # superblock folds in another order (within rounding of each other)
    y2 = ops.gemv(fmt, c.planes, n, k, c.q8)
    rows = sample_rows(n) if n > 512 else None
    y_o, _, _, R = c.oracle_rows(rows)
    if fused_same_bits(t, k):
        assert torch.equal(y, y2)
    else:
        d = np.abs(host(y).astype(np.float64) - host(y2).astype(np.float64))
        assert np.all(d <= TOL * np.abs(host(y2)).max() + 1e-30)
    if t <= 2:  # the image is optional for the one-kernel path
        y3 = ops.gemv_f32(fmt, c.planes, n, k, xd)
        assert torch.equal(y, y3)
    yh = host(y) if rows is None else host(y)[:, rows]
    assert np.all(np.abs(yh.astype(np.float64) - y_o) <= TOL * R)


# ------------------------------------------------------------ GEMM ------
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", [(128, 256, 2560), (129, 100, 768), (1, 64, 256), (300, 65, 512),
                                   (256, 300, 1024),
                                   # the 32-token tile (m <= 127): ragged tokens and rows
                                   (9, 256, 2560), (32, 128, 512), (33, 300, 768), (100, 129, 1024),
                                   (127, 40, 256),
                                   # 128-192 tokens: paired 32-token tiles (176: six tiles;
                                   # 160: five, the last pair's second tile empty); 200: the
                                   # 256-token tile, one ragged block
                                   (176, 130, 1024), (160, 64, 512), (200, 96, 768),
                                   # 64 tokens, k = 4096: four k-parts per workgroup and
                                   # slices across workgroups (Q6_K: as many as fill the CUs)
                                   (64, 300, 4096), (64, 1100, 4096),
                                   # three tiles: the last pair's second tile empty
                                   (80, 200, 2560)])
def test_gemm_parity(fmt, m, n, k):
    c = Case(fmt, n, k, m, seed=m + n)
    y, P, M = ops.matmul_partials("gemm_tiles", fmt, c.planes, n, k, c.q8t)
    check(c, y, P, M)
    # the production entry point, unsplit: the same body without the stores
    y2 = ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=None)
    assert torch.equal(y, y2)
    # with a workspace a grid this small is split along k: same tolerance
    y3 = ops.gemm_tiles(fmt, c.planes, n, k, c.q8t)
    check_y(c, y3)
    # the row image of kq_quantize_q8k: re-laid in the workspace, then the
    # same kernels with the same split, so the same bits
    assert torch.equal(ops.gemm(fmt, c.planes, n, k, c.q8), y3)
    yr, Pr, Mr = ops.matmul_partials("gemm", fmt, c.planes, n, k, c.q8)
    assert torch.equal(yr, y) and torch.equal(Pr, P)
    if fmt != "q6_k":
        assert torch.equal(Mr, M)
    assert kq.kq_gemm_tile_tokens(fmt, n, k, m) == (32 if m <= 192 else 256)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_and_gemm_partials_agree(fmt):
    # the page's tile-vs-gemv bit-exactness gate (kq v3 commit message)
    n, k, t = 200, 2560, 8
    c = Case(fmt, n, k, t, seed=5)
    _, P1, M1 = ops.matmul_partials("gemv", fmt, c.planes, n, k, c.q8)
    _, P2, M2 = ops.matmul_partials("gemm_tiles", fmt, c.planes, n, k, c.q8t)
    assert torch.equal(P1, P2)
    if fmt != "q6_k":
        assert torch.equal(M1, M2)


# --------------------------------------------- full-size, sampled rows --
def sample_rows(n):
    return sorted(set([0, 1, n // 2, n - 2, n - 1] + list(range(7, n, 613))))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(9728, 2560), (2560, 9728)])
@pytest.mark.parametrize("t", [1, 4, 6, 7, 8])
def test_gemv_full_size_sampled(fmt, n, k, t):
    # batch 1 on the dot-product kernel with its image staged in LDS;
    # batches 4-8 on the matrix-core kernel at both shapes (one launch, the
    # partials entry point in the same sum order)
    c = Case(fmt, n, k, t, seed=3)
    y, P, M = ops.matmul_partials("gemv", fmt, c.planes, n, k, c.q8)
    check(c, y, P, M, rows=sample_rows(n))
    y2 = ops.gemv(fmt, c.planes, n, k, c.q8)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(9728, 2560), (2560, 9728)])
def test_gemm_pp512_full_size_sampled(fmt, n, k):
    m = 512
    x = synth.activations(m, k, 77)
    xd = dev(x)
    q8 = ops.quantize_q8k_tiles(xd)  # quantised on device, as in the prefill path
    c = Case(fmt, n, k, m, seed=4, x=x)
    for a, b in zip(q8, c.q8t):
        assert torch.equal(a, b)
    assert kq.kq_gemm_tile_tokens(fmt, n, k, m) == 256
    y = ops.gemm_tiles(fmt, c.planes, n, k, q8)  # with a workspace: W_down splits k
    rows = sample_rows(n)[:24]
    check_y(c, y, rows)
    y1 = ops.gemm_tiles(fmt, c.planes, n, k, q8, workspace=None)
    check_y(c, y1, rows)
    # the pages' sequence: kq_quantize_q8k, then kq_gemm on its row image
    yr = ops.gemm(fmt, c.planes, n, k, ops.quantize_q8k(xd))
    assert torch.equal(yr, y)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,m", [(640, 2560, 300), (96, 2560, 512), (640, 2560, 64), (300, 2560, 40)])
def test_gemm_split_parts_meet_through_any_workspace(fmt, n, k, m):
    # 256-token tile: (640, 2560, 300): 40 tiles; (96, 2560, 512): 6 tiles,
    # whose parts run on different XCDs (the XCD-blocked order has runs of
    # one part there); every tile split along k in 3 parts, the last part of
    # each tile to finish adds the others.  32-token tile: (640, 2560, 64)
    # and (300, 2560, 40, ragged rows and tokens) split along k in 5
    # whole-output slices that a second kernel adds.  The 256-token tile's
    # counters are tagged per call, so for either tile a workspace holding
    # garbage or another call's counters and parts gives the same bits as a
    # zeroed one.
    c = Case(fmt, n, k, m, seed=14)
    nbytes = kq.kq_gemm_tiles_workspace_bytes(fmt, n, k, m)
    nbytes2 = kq.kq_gemm_tiles_workspace_bytes(fmt, 200, 2560, 256)
    assert nbytes > 0 and nbytes2 > 0
    ws = torch.zeros(max(nbytes, nbytes2) + 65536, dtype=torch.uint8, device="cuda")
    y0 = ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=ws)
    check_y(c, y0, sample_rows(n) if n > 2048 else None)
    ws.random_(0, 256)
    assert torch.equal(ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=ws), y0)
    for _ in range(2):
        assert torch.equal(ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=ws), y0)
    # another split call in the same workspace, then this one again
    c2 = Case(fmt, 200, 2560, 256, seed=15)
    check_y(c2, ops.gemm_tiles(fmt, c2.planes, 200, 2560, c2.q8t, workspace=ws))
    assert torch.equal(ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=ws), y0)
    # unsplit: the same outputs within the fold's float tolerance
    check_y(c, ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=None), sample_rows(n) if n > 2048 else None)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(9728, 2560), (2560, 9728)])
@pytest.mark.parametrize("m", [16, 64, 96, 128, 150])  # 64, 128, 150: token tiles paired
def test_gemm_mid_full_size_sampled(fmt, n, k, m):
    c = Case(fmt, n, k, m, seed=6)
    y, P, M = ops.matmul_partials("gemm_tiles", fmt, c.planes, n, k, c.q8t)
    check(c, y, P, M, rows=sample_rows(n))
    check_y(c, ops.gemm_tiles(fmt, c.planes, n, k, c.q8t), rows=sample_rows(n))  # K split with a workspace


# ------------------------------------------ poison, guards, determinism --
@pytest.mark.parametrize("kind", ["gemv", "gemm", "gemm_rows", "gemm_mid", "gemm_mid_pair", "gemm_mid_parts",
                                  "gemm_mid_parts_slices"])
@pytest.mark.parametrize("fmt", FMTS)
def test_outputs_fully_written_and_guards_intact(kind, fmt):
    # gemm: the 256-token tile (200 tokens, one ragged block); gemm_rows: the
    # same through kq_gemm's row image; gemm_mid_pair: an even number of
    # 32-token tiles, paired on 64-row panels; gemm_mid_parts: the same with a
    # workspace, so k is split inside the workgroup; _slices: k = 2048, split
    # inside the workgroup and into whole-output slices too
    n, t = 70, {"gemv": 3, "gemm": 200, "gemm_rows": 200, "gemm_mid": 70, "gemm_mid_pair": 60, "gemm_mid_parts": 60,
                "gemm_mid_parts_slices": 60}[kind]
    k = 2048 if kind == "gemm_mid_parts_slices" else 768
    c = Case(fmt, n, k, t, seed=9)
    assert kq.kq_gemm_tile_tokens(fmt, n, k, t) == (256 if kind in ("gemm", "gemm_rows") else 32)
    g = 4096
    buf = torch.full((g + t * n + g,), float("nan"), dtype=torch.float32, device="cuda")
    canary = torch.tensor([1234.5], device="cuda")
    buf[:g] = canary
    buf[-g:] = canary
    y = buf[g:g + t * n]
    if kind == "gemv":
        kq.kq_gemv(fmt, c.planes, n, k, *c.q8, t, y)
    elif kind == "gemm_rows":
        kq.kq_gemm(fmt, c.planes, n, k, *c.q8, t, y, ops.gemm_workspace(fmt, n, k, t))
    elif kind.startswith("gemm_mid_parts"):
        kq.kq_gemm_tiles(fmt, c.planes, n, k, *c.q8t, t, y, ops.gemm_tiles_workspace(fmt, n, k, t))
    else:
        kq.kq_gemm_tiles(fmt, c.planes, n, k, *c.q8t, t, y)
    torch.cuda.synchronize()
    assert torch.all(buf[:g] == 1234.5) and torch.all(buf[-g:] == 1234.5)
    assert not torch.isnan(y).any()
    if kind.startswith("gemm_mid_parts"):
        check_y(c, y.view(t, n))


@pytest.mark.parametrize("kind", ["gemv", "gemm", "gemm_mid"])
def test_repeat_runs_are_bitwise_identical(kind):
    # gemm_mid: 64 tokens of W_down, k split inside the workgroup and into
    # whole-output slices
    n, k = 2560, 9728
    t = {"gemv": 4, "gemm": 256, "gemm_mid": 64}[kind]
    c = Case("q6_k" if kind != "gemm_mid" else "q4_k", n, k, t, seed=12)
    if kind == "gemv":
        ys = [ops.gemv("q6_k", c.planes, n, k, c.q8) for _ in range(3)]
    else:
        # one workspace reused: the split sums come out the same every call
        fmt = "q6_k" if kind == "gemm" else "q4_k"
        ws = ops.gemm_tiles_workspace(fmt, n, k, t)
        assert ws is not None
        ys = [ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=ws) for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


# ------------------------------------------------------- long rows ------
@pytest.mark.parametrize("fmt", FMTS)
def test_long_k_all_kernels(fmt):
    # k = 65536 (256 superblocks per row): the large offsets of every path --
    # GEMV (batch 1 and 5), the 32-token tile (40 and 130 tokens, k split)
    # and the 256-token tile (200 and 300 tokens: 2 and 4 tiles, k split in
    # 8, and unsplit), whose 32-bit code offsets GEMM_KMAX bounds
    n, k = 40, 65536
    for t, kind in ((1, "gemv"), (5, "gemv"), (40, "gemm"), (130, "gemm"), (200, "gemm"), (300, "gemm")):
        c = Case(fmt, n, k, t, seed=90 + t)
        if kind == "gemv":
            check_y(c, ops.gemv(fmt, c.planes, n, k, c.q8))
            continue
        assert kq.kq_gemm_tile_tokens(fmt, n, k, t) == (32 if t <= 192 else 256)
        y = ops.gemm_tiles(fmt, c.planes, n, k, c.q8t)
        check_y(c, y)
        if t > 192:
            ws = kq.kq_gemm_tiles_workspace_bytes(fmt, n, k, t)
            assert ws > 0  # the split form ran above
            check_y(c, ops.gemm_tiles(fmt, c.planes, n, k, c.q8t, workspace=None))
            assert torch.equal(ops.gemm(fmt, c.planes, n, k, c.q8), y)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_rows_past_the_lds_stage(fmt):
    # a batch of 1-2 stages its Q8_K image and scales in LDS up to 147456
    # bytes (k = 129024 at t = 1, 64512 at t = 2); longer rows read their
    # codes from L2, and kq_gemv_f32 then runs quantiser + GEMV, which needs
    # the image buffers.  Batches 3-8 (the matrix-core kernel) stage one
    # superblock per wave, so no row length moves them off their path.
    n = 24
    c = Case(fmt, n, 129280, 7, seed=94)
    y, P, M = ops.matmul_partials("gemv", fmt, c.planes, n, 129280, c.q8)
    check(c, y, P, M)
    assert torch.equal(ops.gemv(fmt, c.planes, n, 129280, c.q8), y)
    for t, k, fits in ((1, 129024, True), (1, 129280, False), (2, 64768, False)):
        c = Case(fmt, n, k, t, seed=95 + t)
        y, P, M = ops.matmul_partials("gemv", fmt, c.planes, n, k, c.q8)
        check(c, y, P, M)
        assert torch.equal(ops.gemv(fmt, c.planes, n, k, c.q8), y)
        xd = dev(c.x)
        yf, (xq, xs, xbs) = ops.gemv_f32(fmt, c.planes, n, k, xd, keep_image=True)
        assert torch.equal(yf, y)
        rq, rs, rbs = c.q8_host
        assert np.array_equal(host(xq), rq) and np.array_equal(host(xbs), rbs)
        assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))
        if fits:
            assert torch.equal(ops.gemv_f32(fmt, c.planes, n, k, xd), y)
        else:
            with pytest.raises(kq.KqError):
                ops.gemv_f32(fmt, c.planes, n, k, xd)
