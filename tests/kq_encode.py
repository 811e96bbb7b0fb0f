"""Test helper: build ggml K-quant superblock records FROM known integer
fields (the inverse of decoding), so the oracle's decoder can be pinned
against field values that were never produced by a decoder.

Record layouts (ggml K-quant, fixed sizes 144/176/210 B):

* Q4_K: f16 d | f16 dmin | 12 B scale/min packing | 128 B nibbles
* Q5_K: as Q4_K, then 32 B of fifth bits, then 128 B nibbles
* Q6_K: 128 B low nibbles | 64 B high bit pairs | 16 int8 scales | f16 d

Scale/min packing (eight 6-bit scales sc and mins m): bytes 0..3 carry sc
0..3 in their low 6 bits and the top 2 bits of sc 4..7; bytes 4..7 carry
m 0..3 and the top 2 bits of m 4..7; bytes 8..11 carry the low nibbles of
sc 4..7 (low half) and of m 4..7 (high half).
"""
from __future__ import annotations

import numpy as np


def _f16_bytes(v) -> np.ndarray:
    return np.array([v], dtype=np.float16).view(np.uint8)


def pack_scale_min(sc, m) -> np.ndarray:
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    assert all(0 <= v < 64 for v in sc + m)
    out = np.zeros(12, np.uint8)
    for j in range(4):
        out[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        out[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        out[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return out


def encode_q4k(d, dmin, sc, m, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() < 16
    rec = np.zeros(144, np.uint8)
    rec[0:2] = _f16_bytes(d)
    rec[2:4] = _f16_bytes(dmin)
    rec[4:16] = pack_scale_min(sc, m)
    # weights 64p..64p+31 are the low nibbles and 64p+32..64p+63 the high
    # nibbles of bytes 32p..32p+31
    for p in range(4):
        lo = q[64 * p: 64 * p + 32]
        hi = q[64 * p + 32: 64 * p + 64]
        rec[16 + 32 * p: 16 + 32 * p + 32] = (lo | (hi << 4)).astype(np.uint8)
    return rec


def encode_q5k(d, dmin, sc, m, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() < 32
    rec = np.zeros(176, np.uint8)
    rec[0:2] = _f16_bytes(d)
    rec[2:4] = _f16_bytes(dmin)
    rec[4:16] = pack_scale_min(sc, m)
    low = q & 15
    for p in range(4):
        lo = low[64 * p: 64 * p + 32]
        hi = low[64 * p + 32: 64 * p + 64]
        rec[48 + 32 * p: 48 + 32 * p + 32] = (lo | (hi << 4)).astype(np.uint8)
    # fifth bit of weight 32j + l is bit j of byte l of the high-bit array
    five = (q >> 4) & 1
    for l in range(32):
        byte = 0
        for j in range(8):
            byte |= int(five[32 * j + l]) << j
        rec[16 + l] = byte
    return rec


def encode_q6k(d, sc, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    sc = np.asarray(sc, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() < 64
    assert sc.shape == (16,) and sc.min() >= -128 and sc.max() < 128
    rec = np.zeros(210, np.uint8)
    # weight i = 128h + 32t + l: low nibble in byte 64h + l + 32(t%2) of the
    # low array (low half for t < 2, high half otherwise), high two bits in
    # bits 2t..2t+1 of byte 32h + l of the high array
    for h in range(2):
        for t in range(4):
            for l in range(32):
                v = int(q[128 * h + 32 * t + l])
                b = 64 * h + l + 32 * (t % 2)
                rec[b] |= (v & 15) << (0 if t < 2 else 4)
                rec[128 + 32 * h + l] |= (v >> 4) << (2 * t)
    rec[192:208] = sc.astype(np.int8).view(np.uint8)
    rec[208:210] = _f16_bytes(d)
    return rec


def random_fields(fmt: str, rng: np.random.Generator) -> dict:
    if fmt in ("q4_k", "q5_k"):
        return {
            "d": np.float16(abs(rng.normal(0, 1e-3))),
            "dmin": np.float16(abs(rng.normal(0, 1e-3))),
            "sc": rng.integers(0, 64, size=8),
            "m": rng.integers(0, 64, size=8),
            "q": rng.integers(0, 16 if fmt == "q4_k" else 32, size=256),
        }
    return {
        "d": np.float16(abs(rng.normal(0, 1e-3))),
        "sc": rng.integers(-128, 128, size=16),
        "q": rng.integers(0, 64, size=256),
    }


def encode(fmt: str, f: dict) -> np.ndarray:
    if fmt == "q4_k":
        return encode_q4k(f["d"], f["dmin"], f["sc"], f["m"], f["q"])
    if fmt == "q5_k":
        return encode_q5k(f["d"], f["dmin"], f["sc"], f["m"], f["q"])
    return encode_q6k(f["d"], f["sc"], f["q"])


def dequant_fields(fmt: str, f: dict) -> np.ndarray:
    """w (256,) float64 straight from the format's definition."""
    q = np.asarray(f["q"], np.float64)
    d = float(f["d"])
    if fmt == "q6_k":
        sc = np.repeat(np.asarray(f["sc"], np.float64), 16)
        return d * sc * (q - 32)
    sc = np.repeat(np.asarray(f["sc"], np.float64), 32)
    m = np.repeat(np.asarray(f["m"], np.float64), 32)
    return d * sc * q - float(f["dmin"]) * m
