#!/usr/bin/env python3
"""Benchmark of the K-quant x Q8_K matmul on one MI355X.

One step = the whole hot path over one batch of synthetic input:

  GEMV leg: for each of Q4_K, Q5_K, Q6_K and each Qwen3-4B FFN shape
            (W_up 9728 x 2560, W_down 2560 x 9728): quantise one f32
            activation row to Q8_K on device, then the decode GEMV (batch 1);
  GEMM leg: for the same six matrices: quantise 512 f32 activation rows to
            Q8_K on device, then the pp512 prefill GEMM.

Weights are seeded random ggml superblocks (d, dmin |N(0, 1e-3)| as f16,
every other byte uniform), activations f32 N(0, 1).  Each matrix exists in
enough distinct copies that one step's rotation reads over 1 GiB of weights,
so the 256 MB Infinity Cache cannot serve them from cache: every GEMV reads
its weights from HBM.

The GEMV leg runs kq_gemv_f32, the Q8_K quantisation inside the GEMV
kernel (one launch per matrix); the same leg as two launches per matrix
(kq_quantize_q8k, then kq_gemv on the image) is timed after the timed steps
as gemv_two_launch.

Printed: one JSON line.  Each leg is captured into HIP graphs: one per
weight copy (one step) and one per rotation over all the copies (a step per
copy, as a model captures a whole decode token of hundreds of launches in
one graph).  The timed region runs the GEMV leg of all steps back to back
(whole rotations, then single steps for the rest), then the GEMM leg of all
steps, one HIP-event pair around each phase.  `value` is the GEMV leg's
throughput in GB/s of algorithmic bytes (packed weights + f32 activation +
f32 output) over its phase's GPU time; `gemm` holds the GEMM leg's int8
TOPS (2*M*N*K useful ops), quantiser launches included in both.
`roofline` divides the same algorithmic bytes by the average duration of
back-to-back launches of the leg's one kernel (kq_gemv_f32), and
`roofline_gemv_image` does the same for the GEMV kernel on a resident Q8_K
image (kq_gemv; the image's 292 bytes per 256 activations in place of the
f32 activation); `roofline_gemm` the GEMM's int8 ops.  Each of those is a
graph of repeated launches between one pair of HIP events on the launch
stream, inside the timed region.

Two further measurements run after the timed steps, each in its own graphs:
`gemm_mid` (the 32-token tile: quantise 64 rows + kq_gemm on the same six
matrices; `gemm_m128` the same at 128 tokens, the low end of the prefill range) and `moe` (a mixture-of-experts layer: 128 Q4_K experts of gate|up
1536 x 2048 and down 2048 x 768, 512 tokens routed top-8 by seeded U(0,1)
logits, gather-quantise + kq_gemm_grouped for each projection).  Both are
bound by the weight bytes, so their rooflines are in GB/s of HBM.
`layers` runs every matmul of one decode token and of one 512-token prefill
through a 36-layer Qwen3-4B-shaped set (q, k, v, o, gate, up, down; 2.3 GB
of weights), both as seven matrices per layer and with q|k and gate|up packed
as one matrix each (`*_fused`), and `probes` measures this machine's achievable ceilings -- a
plain streaming read of the same plane buffers and a plain int8 MFMA loop --
which `roofline.achievable` / `roofline_gemm.achievable` set beside the
datasheet peaks.  `dense` runs the large dense projections (17408 x 5120 and
its transpose, Q4_K and Q6_K, 50-73 MB each) through the GEMV at batch 1 and
the GEMM at 512 tokens, beside a plain streaming read of the same buffers:
the same kernels at a size where a launch's fixed cost weighs less.
`gemv_batch` times the decode GEMV alone at batch 4 and 8 on the six FFN
matrices, with its own rooflines.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "kq GEMV GB/s (% HBM peak) bs=1; kq GEMM pp512 int8 TOPS (% MFMA peak)"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, 8 TB/s
MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POPS
FMTS = ("q4_k", "q5_k", "q6_k")
SHAPES = ((9728, 2560), (2560, 9728))  # (n, k): W_up, W_down
GEMM_M = 512
MID_M = 64
MOE = {"experts": 128, "tokens": 512, "top": 8, "hidden": 2048, "ffn": 768, "fmt": "q4_k"}
# the large dense projections (17408 x 5120 and its transpose) in Q4_K and Q6_K
DENSE = (("q4_k", 17408, 5120), ("q4_k", 5120, 17408), ("q6_k", 17408, 5120), ("q6_k", 5120, 17408))
BYTES = {"q4_k": 144, "q5_k": 176, "q6_k": 210}


# HBM traffic per launch, averaged over the six matrices of a step:
# FETCH_SIZE + WRITE_SIZE counter passes scaled by a plain-copy reference
# (profiles/kq_gemv_hbm_traffic_qwen3_4b_ffn.md,
# profiles/kq_gemm_hbm_traffic_qwen3_4b_ffn_pp512.md; the GEMM figure is one
# kq_gemm call, split-sum pass included).  Each holds only for the sources
# it was measured on; with any other sources the roofline reports null.
GEMV_F32_TRAFFIC = {"files": ("kq_gemv.hip", "kq_common.h"), "src_sha256_16": "f08f035fc554a12d",
                    "bytes_per_launch": 17591366}
GEMV_TRAFFIC = {"files": ("kq_gemv.hip", "kq_common.h"), "src_sha256_16": "f08f035fc554a12d",
                "bytes_per_launch": 17414023}
# the matrix-core GEMV at batch 8 (the gemv_batch leg's t8)
GEMV8_TRAFFIC = {"files": ("kq_gemv_mma.hip", "kq_common.h"), "src_sha256_16": "f324a75e3f91e773",
                 "bytes_per_launch": 17898683}
GEMM_TRAFFIC = {"files": ("kq_gemm.hip", "kq_digits.h", "kq_common.h"), "src_sha256_16": "9c27a56fa3c1d0a0",
                "bytes_per_launch": 74575427}
MID_TRAFFIC = {"files": ("kq_gemm_mid.hip", "kq_gemm.hip", "kq_digits.h", "kq_common.h"),
               "src_sha256_16": "19986ef945635242", "bytes_per_launch": 24398521}
MOE_TRAFFIC = {"files": ("kq_gemm_mid.hip", "kq_digits.h", "kq_common.h"),
               "src_sha256_16": "2a677adcde19b108", "bytes_per_launch": 232180308}


# Mean per-dispatch duration of the same kernels in the committed rocprofv3
# kernel trace of a full bench run (profiles/kq_gemv_gemm_qwen3_4b_ffn_trace.md,
# timed-region window), so the line carries the roofline fraction from both
# timers; tied to the sources like the traffic records.
GEMV_F32_TRACE = {"files": ("kq_gemv.hip", "kq_common.h"), "src_sha256_16": "f08f035fc554a12d", "avg_us": 6.95}
GEMV_TRACE = {"files": ("kq_gemv.hip", "kq_common.h"), "src_sha256_16": "f08f035fc554a12d", "avg_us": 6.2}
GEMM_TRACE = {"files": ("kq_gemm.hip", "kq_digits.h", "kq_common.h"), "src_sha256_16": "9c27a56fa3c1d0a0",
              "avg_us": 50.15}


def trace_us(rec):
    return rec["avg_us"] if src_hash(rec["files"]) == rec["src_sha256_16"] else None


def src_hash(files):
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "quant_matmul_amd", "csrc")
    data = b"".join(open(os.path.join(csrc, f), "rb").read() for f in files)
    return hashlib.sha256(data).hexdigest()[:16]


def measured_traffic(rec):
    return rec["bytes_per_launch"] if src_hash(rec["files"]) == rec["src_sha256_16"] else None


def gemv_bytes(fmt, n, k, t=1, fused=True):
    """Algorithmic bytes of one GEMV: packed weights + the activation as the
    call takes it (f32 for the fused entry, else the 292-byte-per-256 Q8_K
    image) + the f32 output."""
    nsb = k // 256
    act = 4 * t * k if fused else t * nsb * 292
    return n * nsb * BYTES[fmt] + act + 4 * t * n


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pool-gib", type=float, default=1.0,
                    help="minimum weight bytes read per rotation cycle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--legs", default="gemv,gemm,mid,moe,probes,layers,dense,batch", help="which legs to run")
    ap.add_argument("--side-reps", type=int, default=20,
                    help="replays of the gemm_mid / moe graphs (after the timed steps)")
    ap.add_argument("--profile-one", metavar="KIND:FMT:N:K:T",
                    help="instead of the benchmark, run one configuration --reps times (for "
                         "rocprofv3 counter passes): KIND gemv|gemv_f32|gemm|mid (T activation rows), "
                         "moe (the MoE layer; FMT:N:K:T ignored), copy (a plain 64 MiB device "
                         "copy, the counters' byte reference)")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--probe-sweep", action="store_true",
                    help="only sweep the streaming-read probe over buffer size, loads in flight and grid, "
                         "and print the curve as one JSON line")
    return ap.parse_args()


def cpu_info():
    """Cores this process may run on (sched_getaffinity) and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def _timed_reps(fn, reps):
    """Steady-state timing: one discarded run, then the median of `reps`."""
    fn()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2], ts


def cpu_baseline(seconds):
    """The CPU oracle (oracle/kq_oracle.c, unchanged) on bounded samples of the
    benchmark's workload, timed on this host: single-thread and on all the
    cores this process may use (threads over row slices, each calling the
    same scalar oracle; ctypes releases the GIL during the C call).  Each
    figure is the median of several back-to-back repetitions after one
    discarded run.  GEMV side: Q8_K quantise + GEMV at batch 1 over a row
    slice of each of the six FFN matrices (GB/s of the GEMV's algorithmic
    bytes).  GEMM side: the pp512 products of a row sample of W_up and W_down
    (GMAC/s)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synth

    cores, model = cpu_info()
    # the machine's CPU share for one GPU is 16 cores, whatever the affinity says
    workers = max(1, min(cores, 16))
    # GEMV sample: `rows` rows of every (format, shape) pair, one token; the
    # row count is scaled from a 64-row calibration so that one single-thread
    # repetition takes about seconds/8
    def gemv_sample(rows):
        items = []
        for fmt in FMTS:
            for i, (n, k) in enumerate(SHAPES):
                recs = synth.weights(fmt, rows, k, synth.seed_for(1, 100 + len(items)))
                x = synth.activations(1, k, synth.seed_for(1, 50 + i))
                items.append((fmt, k, recs, x))
        return items

    def gemv_once(items, lo, hi):
        for fmt, k, recs, x in items:
            xq, xs, xbs = oracle.quantize_q8k(x)
            oracle.matmul(fmt, recs[lo:hi], xq, xs, xbs)

    cal = gemv_sample(64)
    t0 = time.perf_counter()
    gemv_once(cal, 0, 64)
    rows = int(min(2560, max(64, 64 * (seconds / 8) / max(time.perf_counter() - t0, 1e-6)))) // 64 * 64
    gemv_items = gemv_sample(rows)
    gemv_bytes_per_rep = sum(gemv_bytes(f, rows, k, fused=False) for f, k, _, _ in gemv_items)

    def gemv_run(parts):
        def work(item_part):
            (fmt, k, recs, x), lo, hi = item_part
            xq, xs, xbs = oracle.quantize_q8k(x)
            oracle.matmul(fmt, recs[lo:hi], xq, xs, xbs)
        jobs = []
        for it in gemv_items:
            step = -(-rows // parts)
            jobs += [(it, lo, min(rows, lo + step)) for lo in range(0, rows, step)]
        if parts == 1:
            for j in jobs:
                work(j)
        else:
            with cf.ThreadPoolExecutor(parts) as ex:
                list(ex.map(work, jobs))

    # GEMM sample: 512 tokens against `grows` rows of Q4_K W_up and Q6_K
    # W_down, scaled so that one single-thread repetition takes about
    # seconds/16
    def gemm_sample(grows):
        items = []
        for fmt, (n, k) in (("q4_k", SHAPES[0]), ("q6_k", SHAPES[1])):
            recs = synth.weights(fmt, grows, k, synth.seed_for(2, 100 + len(items)))
            x = synth.activations(GEMM_M, k, synth.seed_for(2, 50 + len(items)))
            items.append((fmt, k, recs, oracle.quantize_q8k(x)))
        return items

    cal = gemm_sample(2)
    t0 = time.perf_counter()
    for fmt, k, recs, q8 in cal:
        oracle.matmul(fmt, recs, *q8)
    grows = int(min(512, max(2 * workers, 2 * (seconds / 16) / max(time.perf_counter() - t0, 1e-6))))
    grows = -(-grows // workers) * workers
    gemm_items = gemm_sample(grows)
    gemm_macs_per_rep = sum(GEMM_M * grows * k for _, k, _, _ in gemm_items)

    def gemm_run(parts):
        def work(job):
            (fmt, k, recs, q8), lo, hi = job
            oracle.matmul(fmt, recs[lo:hi], *q8)
        jobs = []
        for it in gemm_items:
            step = -(-grows // parts)
            jobs += [(it, lo, min(grows, lo + step)) for lo in range(0, grows, step)]
        if parts == 1:
            for j in jobs:
                work(j)
        else:
            with cf.ThreadPoolExecutor(parts) as ex:
                list(ex.map(work, jobs))

    t_start = time.perf_counter()
    g1, g1_all = _timed_reps(lambda: gemv_run(1), 3)
    gN, gN_all = _timed_reps(lambda: gemv_run(workers), 5)
    m1, _ = _timed_reps(lambda: gemm_run(1), 3)
    mN, _ = _timed_reps(lambda: gemm_run(workers), 5)
    spent = time.perf_counter() - t_start
    return {"value": gemv_bytes_per_rep / gN / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "cpu_model": model, "cores_available": cores,
            "single_thread": {"value": gemv_bytes_per_rep / g1 / 1e9, "unit": "GB/s", "cores": 1},
            "gemm": {"single_thread_GMACs": gemm_macs_per_rep / m1 / 1e9,
                     "all_cores_GMACs": gemm_macs_per_rep / mN / 1e9, "cores": workers,
                     "sample": f"512 tokens x {grows} rows of Q4_K 9728x2560 and of Q6_K 2560x9728 "
                               f"({gemm_macs_per_rep / 1e6:.0f} M MACs per repetition)"},
            "sample": f"Q8_K quantise + GEMV at batch 1 over {rows} rows of each of the six Q4_K/Q5_K/Q6_K "
                      f"W_up/W_down matrices ({gemv_bytes_per_rep / 1e6:.2f} MB of algorithmic bytes per "
                      f"repetition); median of 5 all-core and 3 single-thread repetitions after one "
                      f"discarded run; threads over row slices",
            "seconds": spent}


def bench_probes(mats, copies, stream, capture, ev):
    """Achievable ceilings on this machine (probes/kq_probe.h): a plain
    streaming read of each matrix's plane buffers, rotated over the same
    weight copies the GEMV reads, and a plain int8 32x32x32 MFMA loop."""
    import torch
    import quant_matmul_amd as kq
    import probes
    sink = torch.zeros(65536 * 256, dtype=torch.int32, device="cuda")
    reps = 8 * copies
    read = []
    for fmt, n, k, pl in mats:
        nbytes = pl[0].numel()
        best = None
        # the configurations that win somewhere in the probe's size sweep
        # (profiles/probe_read_ceiling_vs_size.md)
        for unroll, grid in ((1, 2048), (1, 4096), (1, 8192), (2, 4096), (4, 1024), (4, 2048)):
            def run(grid=grid, unroll=unroll):
                for r in range(reps):
                    probes.kq_probe_read_u(pl[r % copies], nbytes, sink, grid, unroll)
            g = capture(run)
            g.replay()
            a, b = ev(), ev()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            if best is None or us < best[0]:
                best = (us, grid, unroll)
        read.append({"matrix": f"{fmt}_{n}x{k}", "bytes": nbytes, "us": best[0], "grid": best[1],
                     "loads_in_flight": best[2], "GBps": nbytes / (best[0] * 1e-6) / 1e9})
    read_gbps = sum(r["bytes"] for r in read) / (sum(r["us"] for r in read) * 1e-6) / 1e9
    mfma = []
    iters = 2048
    for grid in (512, 1024, 2048):
        def run(grid=grid):
            for _ in range(4):
                probes.kq_probe_mfma_i8(iters, grid, sink)
        g = capture(run)
        g.replay()
        a, b = ev(), ev()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / 4
        ops = grid * 4 * iters * 4 * 65536
        mfma.append({"grid": grid, "waves_per_simd": grid // 256, "us": us, "TOPS": ops / (us * 1e-6) / 1e12})
    return {"read_GBps": read_gbps, "read_per_matrix": read,
            "mfma_i8_TOPS": max(m["TOPS"] for m in mfma), "mfma_i8_runs": mfma}


def bench_mid(mats, copies, reps, stream, capture, ev, tokens=MID_M):
    """The 32-token tile: quantise `tokens` rows to the tile image + kq_gemm,
    per matrix, rotating the weight copies; HBM-bound at 64 tokens.  At 128
    tokens (the low end of the prefill range) kq_gemm also runs the 32-token
    tile, its four tiles paired."""
    import torch

    import synth
    import quant_matmul_amd as kq
    from quant_matmul_amd import torch_ops as ops

    res, kb_total, kus_total = {}, 0, 0.0
    for j, (fmt, n, k, pl) in enumerate(mats):
        x = torch.from_numpy(synth.activations(tokens, k, synth.seed_for(3, 50 + j))).cuda()
        q = ops.q8k_tile_buffers(tokens, k)
        y = torch.empty((tokens, n), device="cuda")
        ws = ops.gemm_tiles_workspace(fmt, n, k, tokens)

        def leg(c, kernel_only=False):
            if not kernel_only:
                kq.kq_quantize_q8k_tiles(x, tokens, k, *q)
            kq.kq_gemm_tiles(fmt, pl[c], n, k, *q, tokens, y, ws)

        kq.kq_quantize_q8k_tiles(x, tokens, k, *q)
        g_leg = [capture(leg, c) for c in range(copies)]
        g_k = capture(lambda: [leg(r % copies, True) for r in range(copies)])
        for g in g_leg:
            g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for r in range(reps):
            g_leg[r % copies].replay()
        b.record(stream)
        c_, d_ = ev(), ev()
        c_.record(stream)
        for r in range(max(1, reps // copies)):
            g_k.replay()
        d_.record(stream)
        torch.cuda.synchronize()
        leg_us = a.elapsed_time(b) * 1e3 / reps
        kus = c_.elapsed_time(d_) * 1e3 / (max(1, reps // copies) * copies)
        wb = n * (k // 256) * BYTES[fmt]
        byts = wb + tokens * (k // 256) * 292 + 4 * tokens * n
        res[f"{fmt}_{n}x{k}"] = {"us": kus, "leg_us": leg_us, "GBps": byts / (kus * 1e-6) / 1e9,
                                 "TOPS": 2 * tokens * n * k / (kus * 1e-6) / 1e12, "split_k": ws is not None}
        kb_total += byts
        kus_total += kus
    ach = kb_total / (kus_total * 1e-6) / 1e9
    return {"tokens": tokens, "per_matrix": res,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBPS, "traffic": measured_traffic(MID_TRAFFIC) if tokens == MID_M else None,
                         "algorithmic_bytes_per_launch": kb_total / len(mats),
                         "kernel": "kq::gemm_mid_kp_kernel / gemm_mid_lds_kernel (Q4_K, Q5_K), kq::gemm_mid_kernel (Q6_K) (kq_gemm, 32-token tile)",
                         "avg_launch_us": kus_total / len(mats)}}


def bench_batch(mats, copies, reps, stream, capture, ev, batches=(4, 8)):
    """The decode GEMV at batch 4 and 8 on the six FFN matrices (kq_gemv,
    the Q8_K image quantised once beforehand), back-to-back launches over the
    rotating weight copies: the kernel alone, as `roofline` times batch 1."""
    import torch

    import synth
    import quant_matmul_amd as kq
    from quant_matmul_amd import torch_ops as ops

    res = {}
    for t in batches:
        per, tb, tus = {}, 0, 0.0
        for j, (fmt, n, k, pl) in enumerate(mats):
            x = torch.from_numpy(synth.activations(t, k, synth.seed_for(5, 10 * t + j))).cuda()
            q = ops.quantize_q8k(x)
            y = torch.empty((t, n), device="cuda")

            def run():
                for r in range(copies):
                    kq.kq_gemv(fmt, pl[r], n, k, *q, t, y)

            g = capture(run)
            g.replay()
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / (reps * copies)
            byts = gemv_bytes(fmt, n, k, t, fused=False)
            per[f"{fmt}_{n}x{k}"] = {"us": us, "GBps": byts / (us * 1e-6) / 1e9}
            tb += byts
            tus += us
        ach = tb / (tus * 1e-6) / 1e9
        res[f"t{t}"] = {"per_matrix": per,
                        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                     "frac": ach / HBM_PEAK_GBPS,
                                     "traffic": measured_traffic(GEMV8_TRAFFIC) if t == 8 else None,
                                     "algorithmic_bytes_per_launch": tb / len(mats),
                                     "kernel": f"kq::gemv_mma_kernel (kq_gemv, batch {t}, matrix cores)",
                                     "avg_launch_us": tus / len(mats)}}
    return res


def bench_dense(pool_gib, reps, stream, capture, ev):
    """The large dense projections at decode batch 1 (GEMV) and 512-token
    prefill (GEMM), each matrix in enough copies that a rotation reads more
    than the 256 MB last-level cache holds, beside a plain streaming read of
    the same plane buffers.  At 50-73 MB per matrix the fixed cost of a
    launch weighs far less than on the 14-20 MB FFN matrices."""
    import torch

    import synth
    import quant_matmul_amd as kq
    import probes
    from quant_matmul_amd import torch_ops as ops

    sink = torch.zeros(65536 * 256, dtype=torch.int32, device="cuda")
    res = {}
    tot = {"gemv_bytes": 0, "gemv_us": 0.0, "read_us": 0.0, "gemm_ops": 0, "gemm_us": 0.0}
    for j, (fmt, n, k) in enumerate(DENSE):
        planes = ops.pack(fmt, ops.upload_records(synth.weights(fmt, n, k, synth.seed_for(4, j))), n, k)
        wb = n * (k // 256) * BYTES[fmt]
        copies = max(2, -(-int(pool_gib * (1 << 30)) // wb))
        pl = [planes] + [planes.clone() for _ in range(copies - 1)]
        x1 = torch.from_numpy(synth.activations(1, k, synth.seed_for(4, 50 + j))).cuda()
        xm = torch.from_numpy(synth.activations(GEMM_M, k, synth.seed_for(4, 60 + j))).cuda()
        q1, qm = ops.quantize_q8k(x1), ops.quantize_q8k_tiles(xm)
        y1 = torch.empty((1, n), device="cuda")
        ym = torch.empty((GEMM_M, n), device="cuda")
        ws = ops.gemm_tiles_workspace(fmt, n, k, GEMM_M)
        nbytes = pl[0].numel()

        def gemv_run():
            for r in range(copies):
                kq.kq_gemv(fmt, pl[r], n, k, *q1, 1, y1)

        def read_run():
            for r in range(copies):
                probes.kq_probe_read(pl[r], nbytes, sink, 4096)

        def gemm_run():
            for r in range(copies):
                kq.kq_gemm_tiles(fmt, pl[r], n, k, *qm, GEMM_M, ym, ws)

        out = {}
        for name, fn in (("gemv", gemv_run), ("read", read_run), ("gemm", gemm_run)):
            g = capture(fn)
            g.replay()
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            out[name] = a.elapsed_time(b) * 1e3 / (reps * copies)
        gbytes = wb + (k // 256) * 292 + 4 * n
        ops_ = 2 * GEMM_M * n * k
        res[f"{fmt}_{n}x{k}"] = {"gemv_us": out["gemv"], "gemv_GBps": gbytes / (out["gemv"] * 1e-6) / 1e9,
                                 "read_us": out["read"], "read_GBps": nbytes / (out["read"] * 1e-6) / 1e9,
                                 "gemm_us": out["gemm"], "gemm_TOPS": ops_ / (out["gemm"] * 1e-6) / 1e12,
                                 "weight_copies": copies}
        tot["gemv_bytes"] += gbytes
        tot["gemv_us"] += out["gemv"]
        tot["read_us"] += out["read"]
        tot["gemm_ops"] += ops_
        tot["gemm_us"] += out["gemm"]
        del pl, planes
        torch.cuda.empty_cache()
    ach = tot["gemv_bytes"] / (tot["gemv_us"] * 1e-6) / 1e9
    gem = tot["gemm_ops"] / (tot["gemm_us"] * 1e-6) / 1e12
    return {"per_matrix": res,
            "gemv_roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": ach / HBM_PEAK_GBPS, "kernel": "kq::gemv_kernel (kq_gemv, batch 1)",
                              "avg_launch_us": tot["gemv_us"] / len(DENSE)},
            "gemm_roofline": {"bound": "mfma", "achieved": gem, "peak": MFMA_I8_PEAK_TOPS, "unit": "TOPS",
                              "frac": gem / MFMA_I8_PEAK_TOPS, "kernel": "kq::gemm_kernel (kq_gemm, 512 tokens)",
                              "avg_launch_us": tot["gemm_us"] / len(DENSE)}}


def bench_moe(reps, stream, capture, ev):
    """A mixture-of-experts layer: gather-quantise the routed token rows,
    grouped gate|up, gather-quantise the (synthetic) hidden rows, grouped
    down -- all 128 experts per launch."""
    import torch

    import synth
    import quant_matmul_amd as kq
    from quant_matmul_amd import torch_ops as ops

    E, T, top, H, F, fmt = (MOE[x] for x in ("experts", "tokens", "top", "hidden", "ffn", "fmt"))
    rows, tile_expert, starts, counts = synth.moe_routes(synth.router_logits(T, E, synth.seed_for(4, 0)), top)
    m = len(rows)
    rows_d, te_d = torch.from_numpy(rows).cuda(), torch.from_numpy(tile_expert).cuda()
    up, up_stride = ops.pack_experts(fmt, [synth.weights(fmt, 2 * F, H, synth.seed_for(4, 10 + e))
                                           for e in range(E)], 2 * F, H)
    dn, dn_stride = ops.pack_experts(fmt, [synth.weights(fmt, H, F, synth.seed_for(4, 300 + e))
                                           for e in range(E)], H, F)
    layer_bytes = E * (2 * F * (H // 256) + H * (F // 256)) * BYTES[fmt]
    copies = max(2, -(-(1 << 30) // layer_bytes))  # > 1 GiB per rotation: past the 256 MB cache
    ups, dns = [up] + [up.clone() for _ in range(copies - 1)], [dn] + [dn.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.activations(T, H, synth.seed_for(4, 1))).cuda()
    h = torch.from_numpy(synth.activations(T, F, synth.seed_for(4, 2))).cuda()
    qx, qh = ops.q8k_tile_buffers(m, H), ops.q8k_tile_buffers(m, F)
    y1, y2 = torch.empty((m, 2 * F), device="cuda"), torch.empty((m, H), device="cuda")

    def layer(c):
        kq.kq_quantize_q8k_tiles_gather(x, T, H, rows_d, m, *qx)
        kq.kq_gemm_grouped(fmt, ups[c], up_stride, E, te_d, 2 * F, H, *qx, m, y1)
        kq.kq_quantize_q8k_tiles_gather(h, T, F, rows_d, m, *qh)
        kq.kq_gemm_grouped(fmt, dns[c], dn_stride, E, te_d, H, F, *qh, m, y2)

    def grouped_only(c):
        kq.kq_gemm_grouped(fmt, ups[c], up_stride, E, te_d, 2 * F, H, *qx, m, y1)
        kq.kq_gemm_grouped(fmt, dns[c], dn_stride, E, te_d, H, F, *qh, m, y2)

    gl = [capture(layer, c) for c in range(copies)]
    gk = [capture(grouped_only, c) for c in range(copies)]
    for g in gl:
        g.replay()
    torch.cuda.synchronize()
    a, b, c_, d_ = ev(), ev(), ev(), ev()
    a.record(stream)
    for r in range(reps):
        gl[r % copies].replay()
    b.record(stream)
    c_.record(stream)
    for r in range(reps):
        gk[r % copies].replay()
    d_.record(stream)
    torch.cuda.synchronize()
    layer_us = a.elapsed_time(b) * 1e3 / reps
    gemm_us = c_.elapsed_time(d_) * 1e3 / reps
    routed = int(counts.sum())
    useful = 2 * routed * (2 * F * H + H * F)
    nsb_h, nsb_f = H // 256, F // 256
    alg = layer_bytes + routed * (nsb_h + nsb_f) * 292 + 4 * routed * (2 * F + H)
    ach = alg / (gemm_us * 1e-6) / 1e9
    return {"config": {"experts": E, "tokens": T, "top": top, "hidden": H, "expert_ffn": F, "format": fmt,
                       "gate_up_rows": 2 * F, "routed_rows": routed, "image_rows_padded": m,
                       "weight_bytes": layer_bytes, "weight_copies": copies},
            "layer_us": layer_us, "grouped_gemms_us": gemm_us,
            "weight_GBps": layer_bytes / (gemm_us * 1e-6) / 1e9,
            "useful_TOPS": useful / (gemm_us * 1e-6) / 1e12,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBPS, "traffic": measured_traffic(MOE_TRAFFIC),
                         "algorithmic_bytes_per_launch": alg / 2,
                         "kernel": "kq::gemm_mid_lds_kernel (kq_gemm_grouped), gate|up + down launches",
                         "avg_launch_us": gemm_us / 2}}


# The Qwen3-4B-shaped layer set: (name, format, n, k, input), 36 layers.
# Matrices with the same input read one shared Q8_K image, as a model does.
LAYER_SET = [("q", "q4_k", 4096, 2560, "attn"), ("k", "q4_k", 1024, 2560, "attn"),
             ("v", "q6_k", 1024, 2560, "attn"), ("o", "q4_k", 2560, 4096, "o"),
             ("gate", "q4_k", 9728, 2560, "ffn"), ("up", "q4_k", 9728, 2560, "ffn"),
             ("down", "q6_k", 2560, 9728, "down")]
LAYER_INPUTS = {"attn": 2560, "o": 4096, "ffn": 2560, "down": 9728}
N_LAYERS = 36


def bench_layers(reps, stream, capture, ev):
    """Every matmul of one decode token (batch 1) and of one 512-token
    prefill through the 36-layer Qwen3-4B-shaped set, in order on one stream:
    per layer four quantisations (attention input, o input, FFN input, down
    input) and seven GEMVs / GEMMs.  Only the matmuls run -- no attention,
    norms or activation functions; the inputs are fixed seeded rows.  One
    seeded layer is packed and copied to 36 distinct buffers (2.3 GB), so
    the weights stream from HBM as in a real model."""
    import numpy as np
    import torch

    import synth
    import quant_matmul_amd as kq
    from quant_matmul_amd import torch_ops as ops

    layer = []
    for i, (name, fmt, n, k, inp) in enumerate(LAYER_SET):
        planes = ops.pack(fmt, ops.upload_records(synth.weights(fmt, n, k, synth.seed_for(3, i))), n, k)
        layer.append((name, fmt, n, k, inp, [planes] + [planes.clone() for _ in range(N_LAYERS - 1)]))
    torch.cuda.synchronize()
    x1 = {inp: torch.from_numpy(synth.activations(1, k, synth.seed_for(3, 100 + j))).cuda()
          for j, (inp, k) in enumerate(LAYER_INPUTS.items())}
    xm = {inp: torch.from_numpy(synth.activations(GEMM_M, k, synth.seed_for(3, 110 + j))).cuda()
          for j, (inp, k) in enumerate(LAYER_INPUTS.items())}
    q1 = {inp: ops.q8k_buffers(1, k) for inp, k in LAYER_INPUTS.items()}
    qm = {inp: ops.q8k_tile_buffers(GEMM_M, k) for inp, k in LAYER_INPUTS.items()}
    y1 = [torch.empty((1, n), device="cuda") for _, _, n, _, _, _ in layer]
    ym = [torch.empty((GEMM_M, n), device="cuda") for _, _, n, _, _, _ in layer]
    wss = [ops.gemm_tiles_workspace(fmt, n, k, GEMM_M) for _, fmt, n, k, _, _ in layer]

    def decode():
        for L in range(N_LAYERS):
            for j, (name, fmt, n, k, inp, pl) in enumerate(layer):
                if j == 0 or inp != layer[j - 1][4]:
                    kq.kq_quantize_q8k(x1[inp], 1, k, *q1[inp])
                kq.kq_gemv(fmt, pl[L], n, k, *q1[inp], 1, y1[j])

    def prefill():
        for L in range(N_LAYERS):
            for j, (name, fmt, n, k, inp, pl) in enumerate(layer):
                if j == 0 or inp != layer[j - 1][4]:
                    kq.kq_quantize_q8k_tiles(xm[inp], GEMM_M, k, *qm[inp])
                kq.kq_gemm_tiles(fmt, pl[L], n, k, *qm[inp], GEMM_M, ym[j], wss[j])

    # The same token as a model would lay it out: q|k and gate|up, which
    # share an input and a format, packed as one matrix each (rows
    # concatenated), and the quantisation fused into every GEMV
    # (kq_gemv_f32).  5 launches per layer instead of 11.
    names = [e[0] for e in LAYER_SET]

    def cat(parts_names):
        parts = [layer[names.index(nm)] for nm in parts_names]
        fmt, k = parts[0][1], parts[0][3]
        recs = np.concatenate([synth.weights(fmt, e[2], k, synth.seed_for(3, names.index(e[0]))) for e in parts])
        n = sum(e[2] for e in parts)
        planes = ops.pack(fmt, ops.upload_records(recs), n, k)
        return (fmt, n, k, [planes] + [planes.clone() for _ in range(N_LAYERS - 1)])

    def single(nm):
        e = layer[names.index(nm)]
        return (e[1], e[2], e[3], e[5])

    fused_layer = [cat(["q", "k"]), single("v"), single("o"), cat(["gate", "up"]), single("down")]
    fused_in = ["attn", "attn", "o", "ffn", "down"]
    yf = [torch.empty((1, n), device="cuda") for _, n, _, _ in fused_layer]
    ymf = [torch.empty((GEMM_M, n), device="cuda") for _, n, _, _ in fused_layer]
    wsf = [ops.gemm_tiles_workspace(fmt, n, k, GEMM_M) for fmt, n, k, _ in fused_layer]
    torch.cuda.synchronize()

    def decode_fused():
        for L in range(N_LAYERS):
            for j, ((fmt, n, k, pl), inp) in enumerate(zip(fused_layer, fused_in)):
                kq.kq_gemv_f32(fmt, pl[L], n, k, x1[inp], 1, yf[j])

    # the prefill over the same merged matrices (q|k: 5120 rows, gate|up:
    # 19456 rows), one quantisation per distinct input
    def prefill_fused():
        for L in range(N_LAYERS):
            for j, ((fmt, n, k, pl), inp) in enumerate(zip(fused_layer, fused_in)):
                if j == 0 or inp != fused_in[j - 1]:
                    kq.kq_quantize_q8k_tiles(xm[inp], GEMM_M, k, *qm[inp])
                kq.kq_gemm_tiles(fmt, pl[L], n, k, *qm[inp], GEMM_M, ymf[j], wsf[j])

    res = {}
    for kind, fn, nrep in (("decode", decode, reps), ("decode_fused", decode_fused, reps),
                           ("prefill", prefill, max(2, reps // 4)),
                           ("prefill_fused", prefill_fused, max(2, reps // 4))):
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(nrep):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        res[kind] = a.elapsed_time(b) * 1e3 / nrep  # us per pass
    wbytes = N_LAYERS * sum(n * (k // 256) * BYTES[fmt] for _, fmt, n, k, _, _ in layer)
    ops_prefill = N_LAYERS * sum(2 * GEMM_M * n * k for _, _, n, k, _, _ in layer)
    dec_alg = wbytes + N_LAYERS * (sum(292 * k // 256 for k in LAYER_INPUTS.values())
                                   + 4 * sum(n for _, _, n, _, _, _ in layer))
    return {"config": {"layers": N_LAYERS, "matrices": [[nm, f, n, k] for nm, f, n, k, _, _ in layer],
                       "weight_bytes": wbytes, "prefill_tokens": GEMM_M},
            "decode_us_per_token": res["decode"],
            "decode_GBps": dec_alg / (res["decode"] * 1e-6) / 1e9,
            "decode_frac_hbm": dec_alg / (res["decode"] * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "decode_launches_per_token": N_LAYERS * (len(layer) + len(LAYER_INPUTS)),
            "decode_fused_us_per_token": res["decode_fused"],
            "decode_fused_GBps": dec_alg / (res["decode_fused"] * 1e-6) / 1e9,
            "decode_fused_launches_per_token": N_LAYERS * len(fused_layer),
            "prefill_us": res["prefill"],
            "prefill_TOPS": ops_prefill / (res["prefill"] * 1e-6) / 1e12,
            "prefill_frac_mfma": ops_prefill / (res["prefill"] * 1e-6) / 1e12 / MFMA_I8_PEAK_TOPS,
            "prefill_fused_us": res["prefill_fused"],
            "prefill_fused_TOPS": ops_prefill / (res["prefill_fused"] * 1e-6) / 1e12,
            "prefill_fused_launches": N_LAYERS * (len(fused_layer) + len(LAYER_INPUTS))}


def profile_one(spec, reps):
    """One kq configuration `reps` times on fixed seeded inputs, nothing else
    timed: the workload of a rocprofv3 counter pass."""
    import torch

    import synth
    import quant_matmul_amd as kq
    from quant_matmul_amd import torch_ops as ops

    kind, *rest = spec.split(":")
    if kind == "copy":
        src = torch.empty(16 << 20, dtype=torch.float32, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(reps):
            dst.copy_(src)
    elif kind == "moe":
        # the bench's MoE layer, replayed
        bench_moe(reps, torch.cuda.current_stream(), lambda fn, *a: _Eager(fn, *a),
                  lambda: torch.cuda.Event(enable_timing=True))
    else:
        fmt, n, k, t = rest[0], int(rest[1]), int(rest[2]), int(rest[3])
        planes = ops.pack(fmt, ops.upload_records(synth.weights(fmt, n, k, synth.seed_for(1, 0))), n, k)
        x = torch.from_numpy(synth.activations(t, k, synth.seed_for(1, 50))).cuda()
        y = torch.empty((t, n), device="cuda")
        if kind == "gemv":
            q = ops.quantize_q8k(x)
            for _ in range(reps):
                kq.kq_gemv(fmt, planes, n, k, *q, t, y)
        elif kind == "gemv_f32":
            for _ in range(reps):
                kq.kq_gemv_f32(fmt, planes, n, k, x, t, y)
        else:
            q = ops.quantize_q8k_tiles(x)
            ws = ops.gemm_tiles_workspace(fmt, n, k, t)
            for _ in range(reps):
                kq.kq_gemm_tiles(fmt, planes, n, k, *q, t, y, ws)
    torch.cuda.synchronize()
    print(json.dumps({"profile_one": spec, "reps": reps}), flush=True)
    return 0


class _Eager:
    """Stands in for a captured graph: replay() runs the function eagerly."""

    def __init__(self, fn, *a):
        self.fn, self.a = fn, a

    def replay(self):
        self.fn(*self.a)


def probe_sweep():
    """Best plain streaming read on this machine per buffer size: the probe
    (probes/kq_probe.h) over sizes from the FFN matrices to 1 GiB, 1-16 loads
    in flight per thread and 512-16384 workgroups; small sizes rotate over
    copies that together exceed the 256 MB Infinity Cache, each launch timed
    back to back inside one HIP graph."""
    import torch

    import probes

    torch.cuda.set_device(0)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sizes_mb = (14, 17, 20, 50, 73, 128, 256, 512, 1024)
    out = {"probe_sweep": [], "unit": "GB/s", "peak": HBM_PEAK_GBPS}
    for mb in sizes_mb:
        nbytes = mb * (1 << 20)
        copies = max(1, -(-(1 << 30) // nbytes)) if mb < 512 else 1
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
        reps = max(copies, 16 if mb < 256 else 4)
        best = None
        rows = []
        for unroll in (1, 2, 4, 8, 16):
            for grid in (512, 1024, 2048, 4096, 8192, 16384):
                g = torch.cuda.CUDAGraph()
                s_ = torch.cuda.Stream()
                with torch.cuda.stream(s_):
                    probes.kq_probe_read_u(bufs[0], nbytes, sink, grid, unroll, stream=s_)
                torch.cuda.synchronize()
                with torch.cuda.graph(g):
                    for r in range(reps):
                        probes.kq_probe_read_u(bufs[r % copies], nbytes, sink, grid, unroll)
                g.replay()
                torch.cuda.synchronize()
                ts = []
                for _ in range(5):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    e1.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3 / reps)
                us = sorted(ts)[2]
                gbps = nbytes / (us * 1e-6) / 1e9
                rows.append([unroll, grid, round(us, 3), round(gbps, 1)])
                if best is None or gbps > best[3]:
                    best = [unroll, grid, us, gbps]
                del g
        out["probe_sweep"].append({"MiB": mb, "copies": copies, "best": {"unroll": best[0], "grid": best[1],
                                   "us": round(best[2], 3), "GBps": round(best[3], 1),
                                   "frac_of_peak": round(best[3] / HBM_PEAK_GBPS, 4)}, "all": rows})
        print(f"[sweep] {mb} MiB best {best}", file=sys.stderr, flush=True)
        del bufs
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)
    return 0


def main():
    args = parse()
    if args.probe_sweep:
        return probe_sweep()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the kq path is a single-GPU kernel library; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        return 2
    legs = set(args.legs.split(","))
    if args.profile_one:
        return profile_one(args.profile_one, args.reps)

    import numpy as np
    import torch

    import synth
    import quant_matmul_amd as kq
    from quant_matmul_amd import torch_ops as ops

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)

    # ---------------------------------------------------------- inputs ---
    mats = []  # (fmt, n, k, [plane copies])
    tensor = 0
    for fmt in FMTS:
        for n, k in SHAPES:
            recs = synth.weights(fmt, n, k, synth.seed_for(1, tensor))
            tensor += 1
            planes = ops.pack(fmt, ops.upload_records(recs), n, k)
            mats.append([fmt, n, k, [planes]])
    cycle_bytes = sum(m[1] * (m[2] // 256) * BYTES[m[0]] for m in mats)
    copies = max(1, -(-int(args.pool_gib * (1 << 30)) // cycle_bytes))
    for m in mats:
        m[3] += [m[3][0].clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()

    acts = {}
    for i, (n, k) in enumerate(SHAPES):
        x1 = torch.from_numpy(synth.activations(1, k, synth.seed_for(1, 50 + i))).cuda()
        xm = torch.from_numpy(synth.activations(GEMM_M, k, synth.seed_for(2, 50 + i))).cuda()
        acts[k] = (x1, ops.q8k_buffers(1, k), xm, ops.q8k_tile_buffers(GEMM_M, k))
    ys = [(torch.empty((1, m[1]), device="cuda"), torch.empty((GEMM_M, m[1]), device="cuda"))
          for m in mats]
    # kq_gemm workspaces (zero-filled once; each call leaves them reusable)
    wss = [ops.gemm_tiles_workspace(fmt, n, k, GEMM_M) for fmt, n, k, _ in mats]

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # Every leg is captured once per weight copy into a HIP graph and
    # replayed, so the GPU runs the launches back to back instead of
    # waiting on Python's launch rate.
    def gemv_leg(c):
        # decode: the f32 activation quantised to Q8_K inside the GEMV kernel
        for j, (fmt, n, k, pl) in enumerate(mats):
            kq.kq_gemv_f32(fmt, pl[c], n, k, acts[k][0], 1, ys[j][0])

    def gemv_leg_two(c):
        # the same as two launches: the quantiser, then the GEMV on the image
        for j, (fmt, n, k, pl) in enumerate(mats):
            x1, (xq, xs, xbs), _, _ = acts[k]
            kq.kq_quantize_q8k(x1, 1, k, xq, xs, xbs)
            kq.kq_gemv(fmt, pl[c], n, k, xq, xs, xbs, 1, ys[j][0])

    def gemm_leg(c):
        for j, (fmt, n, k, pl) in enumerate(mats):
            _, _, xm, (xq, xs, xbs) = acts[k]
            kq.kq_quantize_q8k_tiles(xm, GEMM_M, k, xq, xs, xbs)
            kq.kq_gemm_tiles(fmt, pl[c], n, k, xq, xs, xbs, GEMM_M, ys[j][1], wss[j])

    def kernel_only(kind, j, reps):
        fmt, n, k, pl = mats[j]
        x1, q1, xm, qm = acts[k]
        for r in range(reps):
            c = r % copies
            if kind == "gemv_f32":
                kq.kq_gemv_f32(fmt, pl[c], n, k, x1, 1, ys[j][0])
            elif kind == "gemv":
                kq.kq_gemv(fmt, pl[c], n, k, *q1, 1, ys[j][0])
            else:
                kq.kq_gemm_tiles(fmt, pl[c], n, k, *qm, GEMM_M, ys[j][1], wss[j])

    def capture(fn, *a):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(*a)  # eager run on the capture's side stream first
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            fn(*a)
        return g

    # one graph per step (weight copy c), and one per whole rotation over
    # the copies (`copies` steps in one replay, as a model captures a whole
    # decode token of hundreds of launches); a phase of K steps replays
    # whole rotations, then single steps for the rest
    def rotation(leg):
        for c in range(copies):
            leg(c)

    graphs, rgraphs = {}, {}
    legfns = {}
    if "gemv" in legs:
        legfns["gemv"], legfns["gemv2"] = gemv_leg, gemv_leg_two
    if "gemm" in legs:
        legfns["gemm"] = gemm_leg
    for kind, fn in legfns.items():
        graphs[kind] = [capture(fn, c) for c in range(copies)]
        rgraphs[kind] = capture(rotation, fn)
    # activations quantised once for the kernel-only graphs
    for k in acts:
        x1, q1, xm, qm = acts[k]
        kq.kq_quantize_q8k(x1, 1, k, *q1)
        kq.kq_quantize_q8k_tiles(xm, GEMM_M, k, *qm)
    reps = {"gemv_f32": 8 * copies, "gemv": 8 * copies, "gemm": copies}
    kinds = (("gemv_f32", "gemv") if "gemv" in graphs else ()) + (("gemm",) if "gemm" in graphs else ())
    kgraphs = {kind: [capture(kernel_only, kind, j, reps[kind]) for j in range(len(mats))] for kind in kinds}
    torch.cuda.synchronize()

    def phase(kind, nsteps):
        # nsteps passes of one leg back to back, one event pair around them
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(nsteps // copies):
            rgraphs[kind].replay()
        for i in range(nsteps % copies):
            graphs[kind][i].replay()
        b.record(stream)
        return a, b

    for kind in graphs:
        phase(kind, args.warmup)
    torch.cuda.synchronize()

    # ------------------------------------------------------ timed region --
    # every step's GEMV leg, then every step's GEMM leg: args.steps passes
    # of the whole path
    rec, krec = {}, {kind: [] for kind in kgraphs}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = ev()
    start.record(stream)
    for kind in ("gemv", "gemm"):
        if kind in graphs:
            rec[kind] = phase(kind, args.steps)
    end = ev()
    end.record(stream)
    for kind in kgraphs:  # kernel-only replays: the roofline's launch durations
        for j in range(len(mats)):
            a, b = ev(), ev()
            a.record(stream)
            kgraphs[kind][j].replay()
            b.record(stream)
            krec[kind].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    # the two-launch GEMV leg, after the timed region
    if "gemv2" in graphs:
        rec["gemv2"] = phase("gemv2", args.steps)
        torch.cuda.synchronize()

    def ms(pair):
        return pair[0].elapsed_time(pair[1])

    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": total_ms / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": "kq v2 decode GEMV batch 1 + prefill GEMM pp512, Q8_K activations "
                                  "quantised on device, Qwen3-4B FFN shapes",
                      "formats": list(FMTS), "shapes_nk": [list(s) for s in SHAPES],
                      "gemv_batch": 1, "gemm_tokens": GEMM_M,
                      "weight_copies": copies, "weight_bytes_per_rotation": cycle_bytes * copies,
                      "seeds": {"weights": [synth.seed_for(1, t) for t in range(len(mats))],
                                "gemv_x": [synth.seed_for(1, 50 + i) for i in range(len(SHAPES))],
                                "gemm_x": [synth.seed_for(2, 50 + i) for i in range(len(SHAPES))],
                                "generator": "numpy PCG64 (synth/)"}},
           "device": props.name, "host_wall_s": wall}
    per = {}
    if "gemv" in graphs:
        leg_ms = ms(rec["gemv"])
        leg_bytes = args.steps * sum(gemv_bytes(f, n, k, fused=True) for f, n, k, _ in mats)
        out["value"] = leg_bytes / (leg_ms * 1e-3) / 1e9
        out["gemv_leg_ms_per_step"] = leg_ms / args.steps
        leg2_ms = ms(rec["gemv2"])
        leg2_bytes = args.steps * sum(gemv_bytes(f, n, k, fused=False) for f, n, k, _ in mats)
        out["gemv_two_launch"] = {"value": leg2_bytes / (leg2_ms * 1e-3) / 1e9, "unit": "GB/s",
                                  "leg_ms_per_step": leg2_ms / args.steps,
                                  "note": "kq_quantize_q8k then kq_gemv, two launches per matrix; algorithmic "
                                          "bytes count the Q8_K image in place of the f32 activation"}

        def roof(kind, fused, label, traffic_rec, trace_rec):
            kb = sum(reps[kind] * gemv_bytes(f, n, k, fused=fused) for f, n, k, _ in mats)
            kms = sum(ms(p) for p in krec[kind])
            ach = kb / (kms * 1e-3) / 1e9
            alg = kb / (reps[kind] * len(mats))
            tus = trace_us(trace_rec)
            for j, (f, n, k, _) in enumerate(mats):
                us = ms(krec[kind][j]) * 1e3 / reps[kind]
                per.setdefault(f"{f}_{n}x{k}", {})[kind] = {
                    "us": us, "GBps": gemv_bytes(f, n, k, fused=fused) / (us * 1e-6) / 1e9}
            return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBPS, "traffic": measured_traffic(traffic_rec),
                    "algorithmic_bytes_per_launch": alg, "kernel": label,
                    "avg_launch_us": kms * 1e3 / (reps[kind] * len(mats)),
                    "timer": "HIP events around graph replays of back-to-back launches",
                    "trace_avg_us": tus,
                    "frac_trace": None if tus is None else alg / (tus * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        out["roofline"] = roof("gemv_f32", True, "kq::gemv_kernel, quantiser fused (kq_gemv_f32, batch 1)",
                               GEMV_F32_TRAFFIC, GEMV_F32_TRACE)
        out["roofline_gemv_image"] = roof("gemv", False, "kq::gemv_kernel on a resident Q8_K image (kq_gemv, batch 1)",
                                          GEMV_TRAFFIC, GEMV_TRACE)
    if "gemm" in graphs:
        leg_ms = ms(rec["gemm"])
        ops_step = sum(2 * GEMM_M * n * k for _, n, k, _ in mats)
        kms = sum(ms(p) for p in krec["gemm"])
        ach = reps["gemm"] * ops_step / (kms * 1e-3) / 1e12
        out["gemm"] = {"value": args.steps * ops_step / (leg_ms * 1e-3) / 1e12, "unit": "TOPS",
                       "leg_ms_per_step": leg_ms / args.steps}
        gemm_alg = sum(n * (k // 256) * BYTES[f] + GEMM_M * (k + k // 64 + k // 8) + 4 * GEMM_M * n
                       for f, n, k, _ in mats) / len(mats)
        tus = trace_us(GEMM_TRACE)
        ops_launch = ops_step / len(mats)
        out["roofline_gemm"] = {"bound": "mfma", "achieved": ach, "peak": MFMA_I8_PEAK_TOPS, "unit": "TOPS",
                                "frac": ach / MFMA_I8_PEAK_TOPS, "traffic": measured_traffic(GEMM_TRAFFIC),
                                "algorithmic_bytes_per_launch": gemm_alg,
                                "kernel": "kq::gemm_kernel (W_down split along k, parts added in-kernel)",
                                "avg_launch_us": kms * 1e3 / (reps["gemm"] * len(mats)),
                                "timer": "HIP events around graph replays of back-to-back launches",
                                "trace_avg_us": tus,
                                "frac_trace": None if tus is None else
                                ops_launch / (tus * 1e-6) / 1e12 / MFMA_I8_PEAK_TOPS}
        for j, (f, n, k, _) in enumerate(mats):
            us = ms(krec["gemm"][j]) * 1e3 / reps["gemm"]
            per.setdefault(f"{f}_{n}x{k}", {})["gemm"] = {
                "us": us, "TOPS": 2 * GEMM_M * n * k / (us * 1e-6) / 1e12}
    out["per_matrix"] = per
    if "probes" in legs:
        pr = bench_probes(mats, copies, stream, capture, ev)
        out["probes"] = pr
        for key in ("roofline", "roofline_gemv_image"):
            if key in out:
                out[key]["achievable"] = {
                    "value": pr["read_GBps"], "unit": "GB/s", "frac": out[key]["achieved"] / pr["read_GBps"],
                    "probe": "kq_probe_read_u: plain 16-byte streaming read of the same plane buffers, best of "
                             "six launch shapes"}
        if "roofline_gemm" in out:
            t = pr["mfma_i8_TOPS"]
            out["roofline_gemm"]["achievable"] = {
                "value": t, "unit": "TOPS", "frac": out["roofline_gemm"]["achieved"] / t,
                "useful_ceiling_two_digit_passes": t / 2,
                "probe": "kq_probe_mfma_i8: independent v_mfma_i32_32x32x32_i8 chains"}
    if "layers" in legs:
        out["layers"] = bench_layers(args.side_reps, stream, capture, ev)
    if "mid" in legs:
        out["gemm_mid"] = bench_mid(mats, copies, args.side_reps, stream, capture, ev)
        out["gemm_m128"] = bench_mid(mats, copies, args.side_reps, stream, capture, ev, tokens=128)
    if "moe" in legs:
        out["moe"] = bench_moe(args.side_reps, stream, capture, ev)
    if "batch" in legs:
        out["gemv_batch"] = bench_batch(mats, copies, max(2, args.side_reps // 4), stream, capture, ev)
    if "dense" in legs:
        out["dense"] = bench_dense(args.pool_gib, max(2, args.side_reps // 4), stream, capture, ev)
    if out["value"] is None and "gemm" in out:
        out["value"], out["unit"] = out["gemm"]["value"], "TOPS"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
