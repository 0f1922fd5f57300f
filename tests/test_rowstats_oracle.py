"""Pins of the batched fp64 oracle route (oracle/rowstats.py) against the
per-pair C oracle, which the pins of test_oracle_pins.py fix against the
pages' definitions: the visible ranges pair by pair, row statistics, and
dK/dV of single keys over the whole mask and over CSBP shares (owned
blocks plus clean query ranges), for both clean masks, with and without a
window, MHA and GQA.  Agreement is to fp64 rounding (1e-10 relative)."""
import numpy as np
import pytest

from oracle import rowstats as RS
from tests.common import share_positions


def _inputs(seed, L, hq, hkv, d):
    rng = np.random.default_rng(seed)

    def bf16(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do

    n2 = 2 * L
    return bf16((1, n2, hq, d)), bf16((1, n2, hkv, d)), bf16((1, n2, hkv, d)), bf16((1, n2, hq, d))


@pytest.mark.parametrize("L,M,tc,W", [(32, 4, False, 0), (32, 4, True, 0), (48, 8, False, 5), (24, 1, False, 0),
                                      (40, 8, True, 11)])
def test_key_ranges_match_predicate(orc, L, M, tc, W):
    p = orc.problem(1, L, M, 2, 1, 8, token_causal=tc, window=W)
    for i in range(2 * L):
        lo, hi, clo, chi = RS.key_ranges(p, i)
        got = np.zeros(2 * L, dtype=bool)
        got[lo:hi] = True
        got[clo:chi] = True
        ref = np.array([orc.visible(p, i, j) for j in range(2 * L)], dtype=bool)
        assert np.array_equal(got, ref), i


@pytest.mark.parametrize("L,M,hq,hkv,tc,W", [(64, 8, 4, 2, False, 0), (64, 4, 2, 2, True, 0),
                                             (96, 16, 6, 2, False, 20)])
def test_row_stats_match_c_oracle(orc, L, M, hq, hkv, tc, W):
    d = 16
    q, k, v, do = _inputs(L + M, L, hq, hkv, d)
    p = orc.problem(1, L, M, hq, hkv, d, token_causal=tc, bf16=True, window=W)
    G = hq // hkv
    rows = np.arange(2 * L)
    for g in range(hkv):
        lse, D = RS.row_stats(p, q, k, v, do, 0, g, rows)
        n = rows.size * G
        h = np.tile(np.arange(g * G, (g + 1) * G), rows.size)
        i = np.repeat(rows, G)
        _, o, rl = orc.dq_rows(p, orc.keys(), orc.keys(), q, k, v, do, np.zeros(n, np.int32), h, i)
        dof = (do.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rD = (dof[0, i, h] * o).sum(-1)
        np.testing.assert_allclose(lse.reshape(-1), rl, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(D.reshape(-1), rD, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("share_kind", ["whole", "csbp", "csbp_clean"])
@pytest.mark.parametrize("tc,W", [(False, 0), (True, 0), (False, 13)])
def test_dkdv_keys_match_c_oracle(orc, share_kind, tc, W):
    L, M, hq, hkv, d = 64, 8, 4, 2, 16
    q, k, v, do = _inputs(7 + W, L, hq, hkv, d)
    p = orc.problem(1, L, M, hq, hkv, d, token_causal=tc, bf16=True, window=W)
    if share_kind == "whole":
        sh = orc.share()
        rows = np.arange(2 * L)
    else:
        blocks = [0, 1, 6, 7]
        clean_q = [(0, 8), (56, 64)] if share_kind == "csbp_clean" else []
        sh = orc.share(L, M, clean=clean_q, blocks=blocks)
        rows = share_positions(L, M, blocks, clean_q)
    keys = np.array([0, 1, 7, 8, 20, 31, 32, 47, 55, 63, L, L + 3, L + 8, 2 * L - 1])
    for g in range(hkv):
        lse, D = RS.row_stats(p, q, k, v, do, 0, g, rows)
        dk, dv = RS.dkdv_keys(p, q, k, v, do, 0, g, keys, rows, lse, D)
        rdk, rdv = orc.dkdv_rows(p, sh, orc.keys(), orc.keys(), q, k, v, do, np.zeros(keys.size, np.int32),
                                 np.full(keys.size, g, np.int32), keys)
        scale = max(1.0, np.abs(rdk).max(), np.abs(rdv).max())
        np.testing.assert_allclose(dk, rdk, rtol=0, atol=1e-10 * scale)
        np.testing.assert_allclose(dv, rdv, rtol=0, atol=1e-10 * scale)
