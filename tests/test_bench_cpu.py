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


@pytest.mark.parametrize("L,M,W", [(256, 32, 100), (384, 16, 130), (512, 32, 64), (256, 32, 33), (384, 16, 17)])
def test_tile_counts_window_brute_force(orc, L, M, W):
    """Visited tile pairs under a clean-key window of at least M + 1 tokens,
    against a pair-by-pair scan of the oracle's mask predicate."""
    p = orc.problem(1, L, M, 1, 1, 4, window=W)

    def seen(qa, ka):
        return any(orc.visible(p, r, k) for r in range(qa, min(qa + 128, 2 * L))
                   for k in range(ka, min(ka + 64, 2 * L)))

    vis = sum(seen(qa, ka) for qa in range(0, 2 * L, 128) for ka in range(0, 2 * L, 64))
    assert bench.tile_counts(L, M, window=W) == (vis, (2 * L // 128) * (2 * L // 64))


def test_cpu_baseline_row_counts_match_oracle_mask(orc):
    """The CPU baseline prices each sampled row by its visible keys: the same
    count as the oracle's predicate, with and without a window."""
    L, M = 96, 8
    for W in (0, 20):
        p = orc.problem(1, L, M, 1, 1, 4, window=W)
        pos = np.arange(2 * L)
        t = np.where(pos < L, pos, pos - L)
        blk = t // M
        lo = np.maximum(0, t - W + 1) if W > 0 else np.zeros_like(t)
        clean_hi = np.where(pos < L, (blk + 1) * M, blk * M)
        nvis = np.maximum(0, clean_hi - lo) + np.where(pos < L, 0, M)
        ref = [sum(orc.visible(p, i, j) for j in range(2 * L)) for i in range(2 * L)]
        assert list(nvis) == ref


def test_whole_workload_window_field():
    for name, work in bench.WORKLOADS.items():
        w = bench.whole_workload(work)
        assert len(w) == 7 and w[6] == (1024 if name.endswith("window1024") else 0)


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
