"""The kq entry points under HIP graph capture: a captured quantise + GEMV +
GEMM sequence, replayed several times with eager work and synchronisation in
between, matches the eager results bitwise on every replay (the entry points
record no memset and allocate nothing)."""
import numpy as np
import pytest
import torch

import synth
import quant_matmul_amd as kq
from quant_matmul_amd import torch_ops as ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k"])
def test_graph_replays_match_eager(fmt):
    n, k, t, m = 300, 2560, 2, 200
    t8 = 8  # the matrix-core GEMV
    planes = ops.pack(fmt, ops.upload_records(synth.weights(fmt, n, k, 21)), n, k)
    x1 = torch.from_numpy(synth.activations(t, k, 22)).cuda()
    x8 = torch.from_numpy(synth.activations(t8, k, 25)).cuda()
    xm = torch.from_numpy(synth.activations(m, k, 23)).cuda()
    ms = 40  # the 32-token tile, also split along k
    xs_ = torch.from_numpy(synth.activations(ms, k, 24)).cuda()
    assert kq.kq_gemm_tile_tokens(fmt, n, k, m) == 256 and kq.kq_gemm_tile_tokens(fmt, n, k, ms) == 32
    q1, qm, qs = ops.q8k_buffers(t, k), ops.q8k_tile_buffers(m, k), ops.q8k_tile_buffers(ms, k)
    q8 = ops.q8k_buffers(t8, k)
    y8 = torch.empty((t8, n), device="cuda")
    # the row-image GEMM too: its re-lay and split share one workspace
    qr = ops.q8k_buffers(m, k)
    yr = torch.empty((m, n), device="cuda")
    wsr = ops.gemm_workspace(fmt, n, k, m)
    y1 = torch.empty((t, n), device="cuda")
    ym = torch.empty((m, n), device="cuda")
    ys = torch.empty((ms, n), device="cuda")
    wss = ops.gemm_tiles_workspace(fmt, n, k, ms)
    assert wss is not None
    # a grid this small splits k (10 tiles, 3 parts each): the parts meet
    # through counter words in the workspace, tagged per call -- a replay
    # reuses its captured tag
    ws = ops.gemm_tiles_workspace(fmt, n, k, m)
    assert ws is not None

    def seq():
        kq.kq_quantize_q8k(x1, t, k, *q1)
        kq.kq_gemv(fmt, planes, n, k, *q1, t, y1)
        kq.kq_quantize_q8k(x8, t8, k, *q8)
        kq.kq_gemv(fmt, planes, n, k, *q8, t8, y8)
        kq.kq_quantize_q8k_tiles(xm, m, k, *qm)
        kq.kq_gemm_tiles(fmt, planes, n, k, *qm, m, ym, ws)
        kq.kq_quantize_q8k_tiles(xs_, ms, k, *qs)
        kq.kq_gemm_tiles(fmt, planes, n, k, *qs, ms, ys, wss)
        kq.kq_quantize_q8k(xm, m, k, *qr)
        kq.kq_gemm(fmt, planes, n, k, *qr, m, yr, wsr)

    seq()
    torch.cuda.synchronize()
    ref = [a.clone() for a in (*q1, *qm, y1, ym, ys, yr, y8)]
    assert torch.equal(yr, ym)  # the same split over the same image

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        seq()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        seq()
    for rep in range(4):
        for a in (*q1, *qm, y1, ym, ys, yr, y8):
            a.zero_()  # eager work between replays
        if rep == 2:
            # an eager call (a new tag) on the same workspace between replays
            kq.kq_gemm_tiles(fmt, planes, n, k, *qm, m, ym, ws)
            ym.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((*q1, *qm, y1, ym, ys, yr, y8), ref):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
