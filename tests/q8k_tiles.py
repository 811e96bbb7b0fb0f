"""Host re-lay of a Q8_K image between the row layout (xq[t][k] int8,
xbs[t][k/16] int16) and the GEMM's tile image (include/kq.h,
kq_quantize_q8k_tiles): test-side marshalling of the oracle's image, written
from the layout's index formulas."""
import numpy as np


def _pad(a: np.ndarray, rows: int) -> np.ndarray:
    out = np.zeros((rows,) + a.shape[1:], dtype=a.dtype)
    out[:a.shape[0]] = a
    return out


def to_tiles(xq: np.ndarray) -> np.ndarray:
    """xq[t][k] int8 -> flat code tiles; tokens past t padded with zeros."""
    t, k = xq.shape
    tp = (t + 31) // 32 * 32
    # token 32g + r, code 32c + 16q + e  ->  [g][c][q][r][e]
    return np.ascontiguousarray(_pad(xq, tp).reshape(tp // 32, 32, k // 32, 2, 16).transpose(0, 2, 3, 1, 4)).reshape(-1)


def bsum_tiles(xbs: np.ndarray) -> np.ndarray:
    """xbs[t][k/16] int16 -> flat f16 bsum tiles; tokens past t zero."""
    t, kb = xbs.shape
    tp = (t + 31) // 32 * 32
    # token 32g + r, bsum 16s + 8q + e  ->  [g][s][q][r][e]
    a = _pad(xbs, tp).reshape(tp // 32, 32, kb // 16, 2, 8).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(a).reshape(-1).astype(np.float16)


def from_tiles(tiles: np.ndarray, t: int, k: int) -> np.ndarray:
    """Inverse of to_tiles: the (t rounded up to 32) x k row image."""
    tp = (t + 31) // 32 * 32
    return np.ascontiguousarray(tiles.reshape(tp // 32, k // 32, 2, 32, 16).transpose(0, 3, 1, 2, 4)).reshape(tp, k)


def from_bsum_tiles(tiles: np.ndarray, t: int, k: int) -> np.ndarray:
    """Inverse of bsum_tiles: (t rounded up to 32) x k/16, as float64."""
    tp = (t + 31) // 32 * 32
    a = tiles.astype(np.float64).reshape(tp // 32, k // 256, 2, 32, 8).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(a).reshape(tp, k // 16)
