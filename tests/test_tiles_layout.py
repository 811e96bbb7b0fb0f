"""CPU tier: the tile-image re-lay used to feed the oracle's Q8_K image to
the GEMM agrees with the layout's index formulas, element by element."""
import numpy as np

from q8k_tiles import bsum_tiles, from_bsum_tiles, from_tiles, to_tiles


def test_tiles_match_index_formulas():
    rng = np.random.default_rng(5)
    for t, k in ((1, 256), (32, 256), (37, 512), (70, 768)):
        xq = rng.integers(-127, 128, size=(t, k), dtype=np.int8)
        xbs = rng.integers(-2032, 2033, size=(t, k // 16), dtype=np.int16)
        tiles, bt = to_tiles(xq), bsum_tiles(xbs)
        tp = (t + 31) // 32 * 32
        assert tiles.shape == (tp * k,) and bt.shape == (tp * k // 16,) and bt.dtype == np.float16
        C, nsb = k // 32, k // 256
        for tok in range(tp):
            g, r = divmod(tok, 32)
            for code in range(k):
                c, rest = divmod(code, 32)
                q, e = divmod(rest, 16)
                want = xq[tok, code] if tok < t else 0
                assert tiles[((g * C + c) * 64 + q * 32 + r) * 16 + e] == want
            for j in range(k // 16):
                s, rest = divmod(j, 16)
                q, e = divmod(rest, 8)
                want = xbs[tok, j] if tok < t else 0
                assert bt[((g * nsb + s) * 64 + q * 32 + r) * 8 + e] == want  # exact in f16
        back = from_tiles(tiles, t, k)
        assert np.array_equal(back[:t], xq) and not back[t:].any()
        bback = from_bsum_tiles(bt, t, k)
        assert np.array_equal(bback[:t], xbs.astype(np.float64)) and not bback[t:].any()
