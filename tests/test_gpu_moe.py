"""GPU tier: the grouped GEMM of a mixture-of-experts layer (one launch over
all experts) and the gather-quantiser that fills its tile image, against
the CPU oracle on each expert's routed rows, and bit for bit against kq_gemm_tiles
run expert by expert on the same image rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from q8k_tiles import from_bsum_tiles, from_tiles
from quant_matmul_amd import torch_ops as ops
import quant_matmul_amd as kq

pytestmark = pytest.mark.gpu
TOL = 1e-5


def host(t):
    return t.detach().cpu().numpy()


class Moe:
    def __init__(self, fmt, tokens, experts, top, n, k, seed):
        self.fmt, self.n, self.k, self.E = fmt, n, k, experts
        self.x = synth.activations(tokens, k, seed)
        self.rows, self.tile_expert, self.starts, self.counts = synth.moe_routes(
            synth.router_logits(tokens, experts, seed + 1), top)
        self.recs = [synth.weights(fmt, n, k, seed + 10 + e) for e in range(experts)]
        self.planes, self.stride = ops.pack_experts(fmt, self.recs, n, k)
        self.xd = torch.from_numpy(self.x).cuda()
        self.rows_d = torch.from_numpy(self.rows).cuda()
        self.te_d = torch.from_numpy(self.tile_expert).cuda()
        self.q8t = ops.quantize_q8k_tiles_gather(self.xd, self.rows_d)
        self.m = len(self.rows)


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k", "q6_k"])
@pytest.mark.parametrize("tokens,experts,top,n,k", [(37, 5, 2, 96, 512), (64, 8, 3, 200, 768)])
def test_grouped_gemm_matches_oracle_and_per_expert(fmt, tokens, experts, top, n, k):
    c = Moe(fmt, tokens, experts, top, n, k, seed=70 + experts)
    # gathered image: row i is the Q8_K of token rows[i], padding rows zero
    xq, xs, xbs = c.q8t
    codes, bs, d8 = from_tiles(host(xq), c.m, k), from_bsum_tiles(host(xbs), c.m, k), host(xs)
    rq, rs, rbs = oracle.quantize_q8k(c.x)
    for i, tok in enumerate(c.rows):
        if tok < 0:
            assert not codes[i].any() and not bs[i].any() and not d8[i].any()
        else:
            assert np.array_equal(codes[i], rq[tok]) and np.array_equal(bs[i], rbs[tok])
            assert np.array_equal(d8[i].view(np.uint32), rs[tok].view(np.uint32))

    y = ops.gemm_grouped(fmt, c.planes, c.stride, experts, c.te_d, n, k, c.q8t)
    yh = host(y)
    nsb = k // 256
    for e in range(experts):
        s0, cnt = int(c.starts[e]), int(c.counts[e])
        if cnt == 0:
            continue
        toks = c.rows[s0:s0 + cnt]
        q = (rq[toks], rs[toks], rbs[toks])
        y_o = oracle.matmul(fmt, c.recs[e], *q)
        R = oracle.rowmag(fmt, c.recs[e], q[0], q[1])
        assert np.all(np.abs(yh[s0:s0 + cnt].astype(np.float64) - y_o) <= TOL * R), f"expert {e}"
        # the same rows through kq_gemm_tiles (32-token tile), expert by expert
        mp = -(-cnt // 32) * 32
        ye = torch.empty((mp, n), device="cuda")
        kq.kq_gemm_tiles(fmt, c.planes.data_ptr() + e * c.stride, n, k, xq.data_ptr() + s0 * k,
                   xs.data_ptr() + s0 * nsb * 4, xbs.data_ptr() + s0 * (k // 16) * 2, mp, ye)
        assert torch.equal(ye, y[s0:s0 + mp]), f"expert {e}: grouped and per-expert differ"


def test_grouped_gemm_skips_tiles_of_unknown_experts():
    c = Moe("q4_k", 40, 4, 2, 64, 256, seed=90)
    te = c.te_d.clone()
    te[0] = 99  # first tile names no expert
    y = torch.full((c.m, 64), float("nan"), device="cuda")
    ops.gemm_grouped("q4_k", c.planes, c.stride, 4, te, 64, 256, c.q8t, y=y)
    torch.cuda.synchronize()
    assert torch.isnan(y[:32]).all() and not torch.isnan(y[32:]).any()


def test_moe_c4_shape_sampled():
    # the C4 MoE shape: 128 experts of gate|up (2 x 768 = 1536 rows) x 2048,
    # 512 tokens, top-8; checked on a sample of experts
    fmt, n, k = "q4_k", 1536, 2048
    c = Moe(fmt, 512, 128, 8, n, k, seed=5)
    y = host(ops.gemm_grouped(fmt, c.planes, c.stride, 128, c.te_d, n, k, c.q8t))
    rq, rs, rbs = oracle.quantize_q8k(c.x)
    rows = [0, 1, 767, 768, 1535] + list(range(100, n, 311))
    for e in (0, 1, 63, 127):
        s0, cnt = int(c.starts[e]), int(c.counts[e])
        toks = c.rows[s0:s0 + cnt]
        q = (rq[toks], rs[toks], rbs[toks])
        y_o = oracle.matmul(fmt, c.recs[e][rows], *q)
        R = oracle.rowmag(fmt, c.recs[e][rows], q[0], q[1])
        assert np.all(np.abs(y[s0:s0 + cnt][:, rows].astype(np.float64) - y_o) <= TOL * R), f"expert {e}"
