"""Writes tests/golden/c0_oracle.json: a regression record of the small
single-GEMV workload (Q4_K, 256 x 2560, batch 1) as the CPU oracle computes
it.  It calls only the synthetic-input generator and the oracle.  These are
self-generated values, not values printed on the K-quant kernel arc page
(the page prints none); they pin the generator's byte stream and guard the
oracle against unintended change.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def record():
    out = {}
    for fmt in ("q4_k", "q5_k", "q6_k"):
        w = synth.weights(fmt, 256, 2560, synth.seed_for(0, 1))
        x = synth.activations(1, 2560, synth.seed_for(0, 2))
        xq, xs, xbs = oracle.quantize_q8k(x)
        P, M = oracle.partials(fmt, w, xq, xbs)
        y = oracle.matmul(fmt, w, xq, xs, xbs)
        out[fmt] = {
            "weights_sha256": sha(w),
            "x_sha256": sha(x),
            "q8k_sha256": [sha(xq), sha(xs), sha(xbs)],
            "partials_sha256": [sha(P), sha(M)],
            "y_first8": [float(v) for v in y[0, :8]],
        }
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c0_oracle.json")
    with open(path, "w") as f:
        json.dump(record(), f, indent=1)
    print("wrote", path)
