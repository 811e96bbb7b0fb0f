"""CPU tier: the MoE routing tables of the synthetic workload (top-k with
ties to the lower expert id, per-expert lists padded to 32-row tiles)."""
import numpy as np

import synth


def test_routes_structure():
    logits = synth.router_logits(200, 16, 3)
    rows, tile_expert, starts, counts = synth.moe_routes(logits, 4)
    assert counts.sum() == 200 * 4
    assert len(rows) == 32 * len(tile_expert)
    for e in range(16):
        seg = rows[starts[e]:starts[e] + counts[e]]
        assert np.all(np.diff(seg) > 0)  # token order, no repeats
        pad = -(-counts[e] // 32) * 32
        assert np.all(rows[starts[e] + counts[e]:starts[e] + pad] == -1)
        assert np.all(tile_expert[starts[e] // 32:(starts[e] + pad) // 32] == e)
        # every listed token has e among its 4 largest logits
        for tok in seg:
            assert (logits[tok] > logits[tok, e]).sum() < 4


def test_routes_ties_go_to_lower_id():
    logits = np.zeros((3, 6), dtype=np.float32)
    logits[1, 4] = 1.0
    rows, tile_expert, starts, counts = synth.moe_routes(logits, 2)
    # all-equal rows pick experts 0 and 1; row 1 picks 4, then 0
    assert counts.tolist() == [3, 2, 0, 0, 1, 0]
    assert rows[starts[4]] == 1 and list(tile_expert) == [0, 1, 4]
