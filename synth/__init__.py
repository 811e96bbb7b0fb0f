"""Seeded synthetic inputs for the K-quant x Q8_K matmul.

This module only draws random bytes and numbers and writes them into the
ggml superblock byte records; it holds none of the matmul's arithmetic
(no decode, no dequantisation, no quantisation).  Both the CPU oracle and
the HIP path read the exact bytes it returns.

Workload recipe (from the workload description of the K-quant kernel arc
and its Qwen3-4B measurements, "Results" section of the K-quant kernel arc
page):

* superblocks: every byte drawn uniformly at random (scales, mins, quant
  bits, Q6_K's signed per-16 scales, -128 included), except the f16 scale
  fields d (and dmin for Q4_K/Q5_K), which are |N(0, sigma=1e-3)| drawn in
  float64, rounded to float32 and then to float16 (round to nearest even);
* activations: float32 N(0, 1);
* the router for the MoE shape: float32 U(0, 1) logits, and the routing
  tables (top-k experts per token, ties to the lower id) built from them.

The bit generator is numpy's PCG64 with the given integer seed.
"""
from __future__ import annotations

import numpy as np

# byte size of one 256-weight superblock record, and where its f16 scale
# fields sit inside the record (the ggml K-quant record layouts)
BLOCK_BYTES = {"q4_k": 144, "q5_k": 176, "q6_k": 210}
_F16_FIELDS = {"q4_k": (0, 2), "q5_k": (0, 2), "q6_k": (208,)}
QK = 256  # weights per superblock

SEED_BASE = 0x6B71000000000000


def seed_for(config: int, tensor: int) -> int:
    """Seed of tensor `tensor` of workload configuration `config`."""
    return SEED_BASE + 256 * config + tensor


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weights(fmt: str, n: int, k: int, seed: int) -> np.ndarray:
    """ggml superblock records of an n x k weight matrix, row-major.

    Returns uint8 of shape (n, k // 256, BLOCK_BYTES[fmt]).
    """
    if fmt not in BLOCK_BYTES:
        raise ValueError(f"unknown format {fmt!r}")
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nsb = k // QK
    rng = _rng(seed)
    rec = rng.integers(0, 256, size=(n, nsb, BLOCK_BYTES[fmt]), dtype=np.uint8)
    for off in _F16_FIELDS[fmt]:
        v = np.abs(rng.normal(0.0, 1e-3, size=(n, nsb))).astype(np.float32)
        h = v.astype(np.float16).view(np.uint8).reshape(n, nsb, 2)
        rec[:, :, off:off + 2] = h
    return rec


def activations(t: int, k: int, seed: int) -> np.ndarray:
    """float32 N(0, 1) activations of shape (t, k)."""
    return _rng(seed).standard_normal(size=(t, k), dtype=np.float32)


def router_logits(tokens: int, experts: int, seed: int) -> np.ndarray:
    """float32 U(0, 1) router logits of shape (tokens, experts)."""
    return _rng(seed).random(size=(tokens, experts), dtype=np.float32)



def moe_routes(logits: np.ndarray, top: int, tile: int = 32):
    """Routing tables of a mixture-of-experts layer from router logits.

    Each token goes to its `top` experts of highest logit (ties to the lower
    expert id).  Returns (rows, tile_expert, starts, counts): `rows` lists,
    expert after expert, the tokens routed to it in token order, each
    expert's list padded with -1 to a multiple of `tile`; `tile_expert[i]`
    is the expert of rows[i*tile:(i+1)*tile]; `starts[e]` / `counts[e]` are
    the first row and the number of real rows of expert e.
    """
    tokens, experts = logits.shape
    # a stable sort of the negated logits keeps the lower id first among ties
    chosen = np.argsort(-logits, axis=1, kind="stable")[:, :top]
    rows, tile_expert, starts, counts = [], [], [], []
    for e in range(experts):
        toks = np.nonzero((chosen == e).any(axis=1))[0]
        starts.append(len(rows))
        counts.append(len(toks))
        padded = -(-len(toks) // tile) * tile
        rows.extend(toks.tolist() + [-1] * (padded - len(toks)))
        tile_expert.extend([e] * (padded // tile))
    return (np.asarray(rows, dtype=np.int32), np.asarray(tile_expert, dtype=np.int32),
            np.asarray(starts, dtype=np.int64), np.asarray(counts, dtype=np.int64))
