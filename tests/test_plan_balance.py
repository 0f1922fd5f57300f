"""Work orders of the two kernel families, checked on the host:

* the key-major (dK/dV) order bdattn_plan_order_keys, bit-exact against an
  independent statement of it, as the query-major order is in
  test_abi_cpu.py;
* the load-balancing rule both orders apply ("CSBP 完全拆解", section
  "负载均衡：为什么要首尾块配对": pairing an early block with a late one gives
  every pair identical work): at the benchmark workloads, every workgroup
  that holds two tiles carries the same number of visible (query, key)
  pairs.  The pairs are counted here from the mask definition, row by row
  (query tiles) or key by key (key tiles), with no use of the library's
  planner."""
import numpy as np
import pytest

from block_diffusion_lm_bdlm_amd import bdattn as B
from tests import workloads as W

BQ, BKB = 128, 128  # query rows per query tile, keys per key tile


def _xcd_order(logical):
    N = len(logical)
    per, rem = divmod(N, 8)
    sizes = [per + (1 if x < rem else 0) for x in range(8)]
    starts = np.cumsum([0] + sizes[:-1])
    return np.array([logical[starts[w % 8] + w // 8] for w in range(N)], dtype=np.int32)


def _key_order_reference(batch, hkv, clean_tiles, local_tiles):
    """Logical index = (b*hkv + g)*npairs + pair; clean pair p holds tiles
    (p, nc-1-p), -1 when they coincide; local tiles follow singly.  XCD x =
    w % 8 runs a contiguous block of logical indices and hands it out
    longest first: the block's clean pairs in order, then its local tiles."""
    nc = clean_tiles
    pairs = [(p, -1 if p == nc - 1 - p else nc - 1 - p) for p in range((nc + 1) // 2)]
    pairs += [(nc + t, -1) for t in range(local_tiles)]
    logical = [(b, g, a, c) for b in range(batch) for g in range(hkv) for a, c in pairs]
    N = len(logical)
    per, rem = divmod(N, 8)
    sizes = [per + (1 if x < rem else 0) for x in range(8)]
    starts = np.cumsum([0] + sizes[:-1])
    queues = []
    for x in range(8):
        block = logical[starts[x]:starts[x] + sizes[x]]
        longs = [it for it in block if it[2] < nc]
        queues.append(longs + [it for it in block if it[2] >= nc])
    return np.array([queues[w % 8][w // 8] for w in range(N)], dtype=np.int32)


def _calls(name):
    """(problem, share, key sets, row token structure) of a benchmark workload."""
    if name in W.WHOLE:
        w = W.WHOLE[name]
        L, M = w["L"], w["M"]
        p = B.problem(w["batch"], L, M, w["hq"], w["hkv"], w["d"])
        return p, B.share(range(L // M), [(0, L)]), [B.kv([(0, L)], True)], list(range(L // M)), [(0, L)]
    w = W.CSBP[name]
    L, M = w["L"], w["M"]
    blocks, shards = W.assign(L, M, w["P"], w["r"])
    clean_q = shards[w["r"]] if w["clean_queries"] else []
    p = B.problem(1, L, M, w["hq"], w["hkv"], w["d"])
    kvs = [B.kv([], True)] + [B.kv(s, False) for s in shards]
    return p, B.share(blocks, clean_q), kvs, blocks, clean_q


def _rows(L, M, blocks, clean_q):
    """Share rows in row order: (is corrupted, token t, block)."""
    kind, tok = [], []
    for lo, hi in clean_q:
        kind.append(np.zeros(hi - lo, bool))
        tok.append(np.arange(lo, hi))
    bl = np.asarray(blocks, np.int64)
    kind.append(np.ones(bl.size * M, bool))
    tok.append((bl[:, None] * M + np.arange(M)[None, :]).reshape(-1))
    return np.concatenate(kind), np.concatenate(tok)


def _row_keys_in_call(M, corr, tok, kv):
    """Visible keys of each row within one call (block-causal mask, no
    window): clean keys of the call's ranges below the row's clean bound,
    plus the own block when the call includes the local keys."""
    hi = np.where(corr, (tok // M) * M, (tok // M + 1) * M)
    n = np.zeros(tok.size, np.int64)
    for r in range(kv.n):
        lo_r, hi_r = kv.lo[r], kv.hi[r]
        n += np.clip(hi, lo_r, hi_r) - lo_r
    if kv.include_local:
        n += np.where(corr, M, 0)
    return n


def _tile_rows(M, corr, tok, clean_q):
    """Row index ranges of the query tiles: segments (clean ranges, runs of
    consecutive blocks) padded to tiles of BQ rows."""
    segs, start = [], 0
    for lo, hi in clean_q:
        segs.append((start, start + hi - lo))
        start += hi - lo
    n = corr.size
    i = start
    while i < n:
        j = i + M
        while j < n and tok[j] == tok[j - 1] + 1:
            j += M
        segs.append((i, j))
        i = j
    tiles = []
    for a, b in segs:
        tiles += [(t, min(t + BQ, b)) for t in range(a, b, BQ)]
    return tiles


@pytest.mark.parametrize("name", list(W.WHOLE) + list(W.CSBP))
def test_query_major_pairs_carry_equal_work(name):
    p, sh, kvs, blocks, clean_q = _calls(name)
    corr, tok = _rows(p.L, p.M, blocks, clean_q)
    tiles = _tile_rows(p.M, corr, tok, clean_q)
    for kv in kvs:
        per_row = _row_keys_in_call(p.M, corr, tok, kv)
        work = np.array([per_row[a:b].sum() for a, b in tiles])
        order = B.bdattn_plan_order(p, sh, kv)
        # pairs are formed within each kind of query tile (clean, corrupted)
        n_clean_tiles = sum(1 for a, _ in tiles if not corr[a])
        for kind in (False, True):
            paired = [work[a] + work[c] for _, _, a, c in order if c >= 0 and (a >= n_clean_tiles) == kind]
            if not paired:
                continue
            assert min(paired) == max(paired), (name, kv.lo[0], kv.include_local, kind, min(paired), max(paired))


@pytest.mark.parametrize("name", list(W.WHOLE) + list(W.CSBP))
def test_key_major_pairs_carry_equal_work(name):
    p, sh, kvs, blocks, clean_q = _calls(name)
    corr, tok = _rows(p.L, p.M, blocks, clean_q)
    hi = np.sort(np.where(corr, (tok // p.M) * p.M, (tok // p.M + 1) * p.M))
    G = p.hq // p.hkv
    for kv in kvs:
        # clean key tiles of the call: each range cut into tiles of BKB keys
        ktiles = []
        for r in range(kv.n):
            ktiles += [(t, min(t + BKB, kv.hi[r])) for t in range(kv.lo[r], kv.hi[r], BKB)]
        # rows seeing clean key j: rows whose clean bound exceeds j
        work = []
        for a, b in ktiles:
            j = np.arange(a, b)
            work.append(int((hi.size - np.searchsorted(hi, j, side="right")).sum()) * G)
        order = B.bdattn_plan_order_keys(p, sh, kv)
        nc = len(ktiles)
        paired = [work[a] + work[c] for _, _, a, c in order if c >= 0 and a < nc]
        if kv.n == 0:
            # local keys only: single tiles, each key seen by its block's rows
            assert all(c < 0 for _, _, _, c in order)
            continue
        assert len(paired) > 0
        assert min(paired) == max(paired), (name, kv.lo[0], min(paired), max(paired))


@pytest.mark.parametrize("name", list(W.WHOLE) + list(W.CSBP))
def test_key_major_order_bit_exact(name):
    p, sh, kvs, blocks, _ = _calls(name)
    for kv in kvs:
        nclean = sum((kv.hi[r] - kv.lo[r] + BKB - 1) // BKB for r in range(kv.n))
        nlocal = (len(blocks) * p.M + BKB - 1) // BKB if kv.include_local else 0
        got = B.bdattn_plan_order_keys(p, sh, kv)
        ref = _key_order_reference(p.batch, p.hkv, nclean, nlocal)
        assert np.array_equal(got, ref)


def test_key_major_order_covers_every_tile_once():
    p, sh, kvs, blocks, _ = _calls("bdlm_L8K_M32_b2_h16kv8_d128")
    got = B.bdattn_plan_order_keys(p, sh, kvs[0])
    seen = set()
    for b, g, a, c in got:
        for t in (a, c):
            if t >= 0:
                assert (b, g, t) not in seen
                seen.add((b, g, t))
    ntiles = (p.L + BKB - 1) // BKB + (len(blocks) * p.M + BKB - 1) // BKB
    assert len(seen) == p.batch * p.hkv * ntiles
