"""GPU tier: the remaining workload shapes, checked on sampled rows against
the CPU oracle -- the Qwen3-4B-shaped layer set (q, k, v, o, gate/up, down
with their formats), the same layer's merged matrices that share an input
(q|k 5120 x 2560 and gate|up 19456 x 2560), and the large dense projections
(17408 x 5120 and 5120 x 17408, each in Q4_K and Q6_K), each at decode
batch 1 (GEMV) and 512-token prefill (GEMM: the row image through kq_gemm,
bit-identical to the tile image through kq_gemm_tiles).  The tolerance is
the per-output row-magnitude bound of the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import synth
from quant_matmul_amd import torch_ops as ops

pytestmark = pytest.mark.gpu
TOL = 1e-5

# (name, format, n, k): the Qwen3-4B layer (hidden 2560, 32 query heads and 8
# key/value heads of 128, FFN 9728) and the dense 17408-wide projections
LAYER = [("q", "q4_k", 4096, 2560), ("k", "q4_k", 1024, 2560), ("v", "q6_k", 1024, 2560),
         ("o", "q4_k", 2560, 4096), ("gate", "q4_k", 9728, 2560), ("down", "q6_k", 2560, 9728)]
MERGED = [("qk", "q4_k", 5120, 2560), ("gate_up", "q4_k", 19456, 2560)]
DENSE = [("dense_up", "q4_k", 17408, 5120), ("dense_down", "q6_k", 5120, 17408),
         ("dense_down_q4", "q4_k", 5120, 17408), ("dense_up_q6", "q6_k", 17408, 5120)]
ALL = LAYER + MERGED + DENSE


def rows_of(n):
    return sorted(set([0, 1, n // 3, n // 2, n - 2, n - 1] + list(range(11, n, 997))))


def check_rows(fmt, recs, x, y, rows):
    xq, xs, xbs = oracle.quantize_q8k(x)
    y_o = oracle.matmul(fmt, recs[rows], xq, xs, xbs)
    R = oracle.rowmag(fmt, recs[rows], xq, xs)
    yh = y.detach().cpu().numpy()[:, rows].astype(np.float64)
    assert np.all(np.isfinite(yh))
    err = np.abs(yh - y_o)
    assert np.all(err <= TOL * R), f"worst ratio {np.max(err / R):.3g}"


@pytest.mark.parametrize("idx", range(len(ALL)), ids=[s[0] for s in ALL])
@pytest.mark.parametrize("t", [1, 512])
def test_workload_shape_sampled(idx, t):
    name, fmt, n, k = ALL[idx]
    recs = synth.weights(fmt, n, k, synth.seed_for(3, idx))
    planes = ops.pack(fmt, ops.upload_records(recs), n, k)
    x = synth.activations(t, k, synth.seed_for(3, 200 + min(t, 2)))
    xd = torch.from_numpy(x).cuda()
    if t == 1:
        y = ops.gemv(fmt, planes, n, k, ops.quantize_q8k(xd))
        check_rows(fmt, recs, x, y, rows_of(n))
    else:
        y = ops.gemm_tiles(fmt, planes, n, k, ops.quantize_q8k_tiles(xd))
        # 64 sampled tokens keep the oracle's work small
        tok = list(range(0, t, 8))
        check_rows(fmt, recs, x[tok], y[tok], rows_of(n))
        assert torch.equal(ops.gemm(fmt, planes, n, k, ops.quantize_q8k(xd)), y)
