"""GPU tier: kq_gemm_noalloc, the GEMM for callers that cannot allocate --
its workspace is the library's own device array -- against kq_gemm with a
caller-owned workspace, on two calls in a row (the second smaller, so it
runs on what the first left in the array), each also within the oracle's
row-magnitude tolerance on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quant_matmul_amd as kq
from quant_matmul_amd import torch_ops as ops

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _case(fmt, n, k, m, seed):
    recs = synth.weights(fmt, n, k, seed)
    planes = ops.pack(fmt, ops.upload_records(recs), n, k)
    x = synth.activations(m, k, seed + 1)
    q8 = ops.quantize_q8k(torch.from_numpy(x).cuda())
    return recs, planes, x, q8


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k", "q6_k"])
def test_noalloc_matches_kq_gemm_on_two_calls(fmt):
    # first: W_down at 512 tokens (the 256-token tile, k split through the
    # array's counter words and partial tiles); second: a smaller call on the
    # 32-token tile, also split, over the first call's leftovers
    for n, k, m, seed in ((2560, 9728, 512, 51), (300, 2560, 64, 52)):
        assert kq.kq_gemm_workspace_bytes(fmt, n, k, m) <= kq.KQ_SCRATCH_BYTES
        recs, planes, x, q8 = _case(fmt, n, k, m, seed)
        y = torch.full((m, n), float("nan"), device="cuda")
        rc = kq.lib.kq_gemm_noalloc(kq.FORMATS[fmt], planes.data_ptr(), n, k, q8[0].data_ptr(), q8[1].data_ptr(),
                                    q8[2].data_ptr(), m, y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == kq.KQ_OK
        ref = ops.gemm(fmt, planes, n, k, q8)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"{fmt} {n}x{k} m={m}: differs from kq_gemm"
        rows = sorted(set([0, n // 2, n - 1] + list(range(5, n, 331))))
        tok = list(range(0, m, 7))
        xq, xs, xbs = oracle.quantize_q8k(x[tok])
        y_o = oracle.matmul(fmt, recs[rows], xq, xs, xbs)
        R = oracle.rowmag(fmt, recs[rows], xq, xs)
        yh = y.cpu().numpy()[tok][:, rows].astype(np.float64)
        assert np.all(np.abs(yh - y_o) <= TOL * R)
