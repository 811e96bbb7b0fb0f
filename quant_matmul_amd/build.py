"""Build libkq.so (the kq C ABI + its gfx950 kernels) in-tree with hipcc,
and the benchmark's measurement probes (probes/libkq_probe.so, not part of
the matmul library).

    python quant_matmul_amd/build.py

(run as a script, not `-m`: importing the package loads the library.)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkq.so")
SOURCES = ["kq_api.hip", "kq_quantize.hip", "kq_pack.hip", "kq_gemv.hip", "kq_gemv_mma.hip", "kq_gemm.hip", "kq_gemm_mid.hip"]
PROBE_DIR = os.path.join(ROOT, "probes")
PROBE_SRC = os.path.join(PROBE_DIR, "kq_probe.hip")
PROBE_LIB = os.path.join(PROBE_DIR, "libkq_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # keep hipcc from forming packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # export only the entry points include/kq.h declares
    "-fvisibility=hidden",
]


def _compile(src: str) -> str:
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(OBJ, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-I" + PROBE_DIR, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + [PROBE_SRC]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, srcs))
    for lib, parts in ((LIB, objs[:-1]), (PROBE_LIB, objs[-1:])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *parts]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
