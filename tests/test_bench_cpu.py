"""Host-side pieces of bench.py: the visible-pair counts that turn a step
time into useful FLOP/s, checked against the oracle's mask predicate."""
import numpy as np
import pytest

import bench


@pytest.mark.parametrize("L,M,W,tc", [(16, 4, 0, False), (24, 4, 0, True), (16, 4, 3, False), (32, 8, 5, False),
                                      (16, 1, 4, True), (16, 16, 5, False), (24, 4, 9, True), (16, 4, 40, False)])
def test_visible_pairs_match_oracle_mask(orc, L, M, W, tc):
    p = orc.problem(1, L, M, 1, 1, 4, token_causal=tc, window=W)
    n = sum(orc.visible(p, i, j) for i in range(2 * L) for j in range(2 * L))
    assert bench.visible_pairs(L, M, W, tc) == n


@pytest.mark.parametrize("L,M,blocks,clean", [(32, 4, [0, 7, 3], [(4, 9)]), (64, 8, [1, 2, 6], [(0, 8), (56, 64)])])
def test_share_pairs_match_oracle_mask(orc, L, M, blocks, clean):
    p = orc.problem(1, L, M, 1, 1, 4)
    rows = [t for lo, hi in clean for t in range(lo, hi)] + [L + b * M + i for b in blocks for i in range(M)]
    n = sum(orc.visible(p, i, j) for i in rows for j in range(2 * L))
    assert bench.share_pairs(L, M, sorted(blocks), clean) == n
