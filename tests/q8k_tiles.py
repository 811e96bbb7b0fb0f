"""Host re-lay of Q8_K codes between the row image xq[t][k] and the GEMM's
tile image (include/kq.h, kq_quantize_q8k_tiles): test-side marshalling of
the oracle's image, written from the layout's index formula."""
import numpy as np


def to_tiles(xq: np.ndarray) -> np.ndarray:
    """xq[t][k] int8 -> flat tile image; tokens past t padded with zeros."""
    t, k = xq.shape
    tp = (t + 15) // 16 * 16
    pad = np.zeros((tp, k), dtype=np.int8)
    pad[:t] = xq
    # token 16g + r, code 64c + 16q + e  ->  [g][c][q][r][e]
    return np.ascontiguousarray(pad.reshape(tp // 16, 16, k // 64, 4, 16).transpose(0, 2, 3, 1, 4)).reshape(-1)


def from_tiles(tiles: np.ndarray, t: int, k: int) -> np.ndarray:
    """Inverse of to_tiles: the (t rounded up to 16) x k row image."""
    tp = (t + 15) // 16 * 16
    return np.ascontiguousarray(tiles.reshape(tp // 16, k // 64, 4, 16, 16).transpose(0, 3, 1, 2, 4)).reshape(tp, k)
