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


@pytest.mark.parametrize("L,M", [(256, 32), (384, 16), (512, 64)])
def test_tile_counts_brute_force(L, M):
    """Visited (128-row, 64-key) tile pairs of the whole block-causal mask,
    against a pair-by-pair scan of the mask."""
    import bench

    def seen(qa, ka):
        for r in range(qa, min(qa + 128, 2 * L)):
            for k in range(ka, min(ka + 64, 2 * L)):
                if r < L:
                    if k < L and k // M <= r // M:
                        return True
                elif (k < L and k // M < (r - L) // M) or (k >= L and (k - L) // M == (r - L) // M):
                    return True
        return False

    vis = sum(seen(qa, ka) for qa in range(0, 2 * L, 128) for ka in range(0, 2 * L, 64))
    assert bench.tile_counts(L, M) == (vis, (2 * L // 128) * (2 * L // 64))


def test_traffic_record_only_for_its_workload():
    """The committed HBM byte counts belong to the workload they were taken
    on: a bench line of another workload carries none."""
    import json
    with open(bench.TRAFFIC_FILE) as f:
        recs = json.load(f)
    for kernel, rec in recs.items():
        assert bench.measured_traffic(kernel, rec["workload"] + "_other") is None
        got = bench.measured_traffic(kernel, rec["workload"])
        assert got is None or (isinstance(got, int) and got > 0)
