"""CPU tier: the tile-image re-lay used to feed the oracle's codes to the
GEMM agrees with the layout's index formula, element by element."""
import numpy as np

from q8k_tiles import from_tiles, to_tiles


def test_to_tiles_matches_index_formula():
    rng = np.random.default_rng(5)
    for t, k in ((1, 256), (16, 256), (21, 512), (40, 768)):
        xq = rng.integers(-127, 128, size=(t, k), dtype=np.int8)
        tiles = to_tiles(xq)
        tp = (t + 15) // 16 * 16
        assert tiles.shape == (tp * k,)
        C = k // 64
        for tok in range(tp):
            g, r = divmod(tok, 16)
            for code in range(k):
                c, rest = divmod(code, 64)
                q, e = divmod(rest, 16)
                want = xq[tok, code] if tok < t else 0
                assert tiles[(((g * C + c) * 4 + q) * 16 + r) * 16 + e] == want
        back = from_tiles(tiles, t, k)
        assert np.array_equal(back[:t], xq) and not back[t:].any()
