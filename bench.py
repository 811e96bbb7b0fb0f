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

The GEMV leg runs kq_quantize_q8k then kq_gemv; the fused entry point
kq_gemv_f32 (Q8_K quantisation inside the GEMV kernel, one launch) is timed
beside it as gemv_fused.

Printed: one JSON line.  Each leg is captured into a HIP graph (one per
weight copy) and replayed, so the GPU runs its launches back to back.
`value` is the GEMV leg's throughput in GB/s of algorithmic bytes (packed
weights + Q8_K image + f32 output) over the leg's GPU time (HIP events
around the replay), quantiser launches included; `gemm` holds the GEMM leg's
int8 TOPS (2*M*N*K useful ops).  `roofline` / `roofline_gemm` divide the
same algorithmic work by the average duration of back-to-back launches of
the GEMV / GEMM kernel alone (a graph of repeated launches between one pair
of HIP events on the launch stream, inside the timed region).
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
BYTES = {"q4_k": 144, "q5_k": 176, "q6_k": 210}


# HBM traffic of kq_gemv per launch, averaged over the six matrices of a
# step: FETCH_SIZE + WRITE_SIZE counter passes scaled by a plain-copy
# reference (profiles/kq_gemv_hbm_traffic_qwen3_4b_ffn.md).  It holds only
# for the GEMV sources it was measured on; with any other sources the
# roofline reports traffic as null.
GEMV_TRAFFIC = {"src_sha256_16": "c32ca253a2f82f95", "bytes_per_launch": 17422080}


def gemv_src_hash():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "quant_matmul_amd", "csrc")
    data = b"".join(open(os.path.join(csrc, f), "rb").read() for f in ("kq_gemv.hip", "kq_common.h"))
    return hashlib.sha256(data).hexdigest()[:16]


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
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--legs", default="gemv,gemm", help="which legs to run")
    return ap.parse_args()


def cpu_baseline(seconds):
    """The CPU oracle (oracle/kq_oracle.c, single thread) on a bounded sample:
    Q8_K quantise + GEMV at batch 1 over row slices of the six matrices."""
    import numpy as np

    import oracle
    import synth

    done_bytes, t_used, matrices = 0, 0.0, 0
    rows = 512
    start = time.perf_counter()
    while t_used < seconds:
        for fmt in FMTS:
            for i, (n, k) in enumerate(SHAPES):
                recs = synth.weights(fmt, rows, k, synth.seed_for(1, 100 + matrices))
                x = synth.activations(1, k, synth.seed_for(1, 50 + i))
                t0 = time.perf_counter()
                xq, xs, xbs = oracle.quantize_q8k(x)
                oracle.matmul(fmt, recs, xq, xs, xbs)
                t_used += time.perf_counter() - t0
                done_bytes += gemv_bytes(fmt, rows, k, fused=False)
                matrices += 1
        if time.perf_counter() - start > 4 * seconds:
            break
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{matrices} GEMV calls at batch 1, each 512 rows of one of the six "
                      f"Q4_K/Q5_K/Q6_K W_up/W_down matrices (Q8_K quantise included), "
                      f"{t_used:.1f} s of single-thread CPU time",
            "seconds": t_used}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the kq path is a single-GPU kernel library; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        return 2
    legs = set(args.legs.split(","))

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
    wss = [ops.gemm_workspace(fmt, n, k, GEMM_M) for fmt, n, k, _ in mats]

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # Every leg is captured once per weight copy into a HIP graph and
    # replayed, so the GPU runs the launches back to back instead of
    # waiting on Python's launch rate.
    def gemv_leg(c):
        # decode: quantise the f32 activation to Q8_K, then the GEMV
        for j, (fmt, n, k, pl) in enumerate(mats):
            x1, (xq, xs, xbs), _, _ = acts[k]
            kq.kq_quantize_q8k(x1, 1, k, xq, xs, xbs)
            kq.kq_gemv(fmt, pl[c], n, k, xq, xs, xbs, 1, ys[j][0])

    def gemv_leg_fused(c):
        # the same with the quantiser fused into the GEMV (kq_gemv_f32)
        for j, (fmt, n, k, pl) in enumerate(mats):
            kq.kq_gemv_f32(fmt, pl[c], n, k, acts[k][0], 1, ys[j][0])

    def gemm_leg(c):
        for j, (fmt, n, k, pl) in enumerate(mats):
            _, _, xm, (xq, xs, xbs) = acts[k]
            kq.kq_quantize_q8k_tiles(xm, GEMM_M, k, xq, xs, xbs)
            kq.kq_gemm(fmt, pl[c], n, k, xq, xs, xbs, GEMM_M, ys[j][1], wss[j])

    def kernel_only(kind, j, reps):
        fmt, n, k, pl = mats[j]
        x1, q1, xm, qm = acts[k]
        for r in range(reps):
            c = r % copies
            if kind == "gemv":
                kq.kq_gemv(fmt, pl[c], n, k, *q1, 1, ys[j][0])
            else:
                kq.kq_gemm(fmt, pl[c], n, k, *qm, GEMM_M, ys[j][1], wss[j])

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

    graphs = {}
    if "gemv" in legs:
        graphs["gemv"] = [capture(gemv_leg, c) for c in range(copies)]
        graphs["gemv2"] = [capture(gemv_leg_fused, c) for c in range(copies)]
    if "gemm" in legs:
        graphs["gemm"] = [capture(gemm_leg, c) for c in range(copies)]
    # activations quantised once for the kernel-only graphs
    for k in acts:
        x1, q1, xm, qm = acts[k]
        kq.kq_quantize_q8k(x1, 1, k, *q1)
        kq.kq_quantize_q8k_tiles(xm, GEMM_M, k, *qm)
    reps = {"gemv": 8 * copies, "gemm": copies}
    kgraphs = {kind: [capture(kernel_only, kind, j, reps[kind]) for j in range(len(mats))]
               for kind in ("gemv", "gemm") if kind in graphs}
    torch.cuda.synchronize()

    def run_steps(nsteps, rec):
        for i in range(nsteps):
            c = i % copies
            for kind in ("gemv", "gemv2", "gemm"):
                if kind in graphs:
                    a, b = ev(), ev()
                    a.record(stream)
                    graphs[kind][c].replay()
                    b.record(stream)
                    rec[kind].append((a, b))

    run_steps(args.warmup, {"gemv": [], "gemv2": [], "gemm": []})
    torch.cuda.synchronize()

    # ------------------------------------------------------ timed region --
    rec = {"gemv": [], "gemv2": [], "gemm": []}
    krec = {kind: [] for kind in kgraphs}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = ev()
    start.record(stream)
    run_steps(args.steps, rec)
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

    def ms(ps):
        return sum(a.elapsed_time(b) for a, b in ps)

    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": total_ms / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": "kq v2 decode GEMV batch 1 + prefill GEMM pp512, Q8_K activations "
                                  "quantised on device, Qwen3-4B FFN shapes",
                      "formats": list(FMTS), "shapes_nk": [list(s) for s in SHAPES],
                      "gemv_batch": 1, "gemm_tokens": GEMM_M,
                      "weight_copies": copies, "weight_bytes_per_rotation": cycle_bytes * copies},
           "device": props.name, "host_wall_s": wall}
    per = {}
    if "gemv" in graphs:
        leg_ms = ms(rec["gemv"])
        leg_bytes = args.steps * sum(gemv_bytes(f, n, k, fused=False) for f, n, k, _ in mats)
        out["value"] = leg_bytes / (leg_ms * 1e-3) / 1e9
        out["gemv_leg_ms_per_step"] = leg_ms / args.steps
        leg2_ms = ms(rec["gemv2"])
        leg2_bytes = args.steps * sum(gemv_bytes(f, n, k, fused=True) for f, n, k, _ in mats)
        out["gemv_fused"] = {"value": leg2_bytes / (leg2_ms * 1e-3) / 1e9, "unit": "GB/s",
                             "note": "kq_gemv_f32: Q8_K quantisation inside the GEMV, one launch per matrix"}
        kb = sum(reps["gemv"] * gemv_bytes(f, n, k, fused=False) for f, n, k, _ in mats)
        kms = ms(krec["gemv"])
        ach = kb / (kms * 1e-3) / 1e9
        traffic = (GEMV_TRAFFIC["bytes_per_launch"]
                   if gemv_src_hash() == GEMV_TRAFFIC["src_sha256_16"] else None)
        out["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBPS, "traffic": traffic,
                           "algorithmic_bytes_per_launch": kb / (reps["gemv"] * len(mats)),
                           "kernel": "kq::gemv_kernel (kq_gemv)",
                           "avg_launch_us": kms * 1e3 / (reps["gemv"] * len(mats))}
        for j, (f, n, k, _) in enumerate(mats):
            us = krec["gemv"][j][0].elapsed_time(krec["gemv"][j][1]) * 1e3 / reps["gemv"]
            per.setdefault(f"{f}_{n}x{k}", {})["gemv"] = {
                "us": us, "GBps": gemv_bytes(f, n, k, fused=False) / (us * 1e-6) / 1e9}
    if "gemm" in graphs:
        leg_ms = ms(rec["gemm"])
        ops_step = sum(2 * GEMM_M * n * k for _, n, k, _ in mats)
        kms = ms(krec["gemm"])
        ach = reps["gemm"] * ops_step / (kms * 1e-3) / 1e12
        out["gemm"] = {"value": args.steps * ops_step / (leg_ms * 1e-3) / 1e12, "unit": "TOPS",
                       "leg_ms_per_step": leg_ms / args.steps}
        out["roofline_gemm"] = {"bound": "mfma", "achieved": ach, "peak": MFMA_I8_PEAK_TOPS, "unit": "TOPS",
                                "frac": ach / MFMA_I8_PEAK_TOPS, "traffic": None, "kernel": "kq::gemm_kernel",
                                "avg_launch_us": kms * 1e3 / (reps["gemm"] * len(mats))}
        for j, (f, n, k, _) in enumerate(mats):
            us = krec["gemm"][j][0].elapsed_time(krec["gemm"][j][1]) * 1e3 / reps["gemm"]
            per.setdefault(f"{f}_{n}x{k}", {})["gemm"] = {
                "us": us, "TOPS": 2 * GEMM_M * n * k / (us * 1e-6) / 1e12}
    out["per_matrix"] = per
    if out["value"] is None and "gemm" in out:
        out["value"], out["unit"] = out["gemm"]["value"], "TOPS"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
