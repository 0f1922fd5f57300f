"""Pins for the CPU oracle: each check ties it to something other than itself.

 * hand-written golden fixtures from the pages (tests/golden/);
 * an independent dense formulation: the 2L x 2L mask built from Kronecker
   block products (not from the oracle's per-pair predicate) and the masked
   softmax, logsumexp and autograd gradients of torch in float64;
 * special cases that reduce to torch's scaled_dot_product_attention;
 * closed forms (visible-pair counts, K = 0, constant V, the merge example);
 * identities the pages state exactly: block-separable loss (BP), exact LSE
   merge over any split of the keys (CSBP), corrupted K/V read only by their
   own block;
 * central finite differences of the oracle's own forward.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers
def window_band(L, W):
    """Clean-key sliding window as a band: entry (t, j) kept when j >= t - W + 1
    (np.triu with offset -(W - 1)); W = 0 keeps everything."""
    if W <= 0:
        return np.ones((L, L), dtype=bool)
    return np.triu(np.ones((L, L), dtype=bool), -(W - 1))


def dense_mask(L, M, token_causal=False, window=0):
    """Doubled-input mask from block products: clean rows over the clean copy
    (block lower-triangular of ones, or token lower-triangular), corrupted
    block b over clean blocks < b (strict block lower-triangular) and its own
    corrupted block (block diagonal).  A window cuts both clean-key blocks
    with the same band (the corrupted copy's rows are the same token
    positions as the clean copy's)."""
    B = L // M
    E = np.ones((M, M), dtype=bool)
    if token_causal:
        cc = np.tril(np.ones((L, L), dtype=bool))
    else:
        cc = np.kron(np.tril(np.ones((B, B), dtype=bool)), E)
    xc = np.kron(np.tril(np.ones((B, B), dtype=bool), -1), E)
    band = window_band(L, window)
    cc, xc = cc & band, xc & band
    xx = np.kron(np.eye(B, dtype=bool), E)
    top = np.concatenate([cc, np.zeros((L, L), dtype=bool)], 1)
    bot = np.concatenate([xc, xx], 1)
    return np.concatenate([top, bot], 0)


def dense_attention(q, k, v, mask, scale):
    """torch float64 masked attention: q [b,n,hq,d], k/v [b,n,hkv,d]."""
    G = q.shape[2] // k.shape[2]
    kk = k.repeat_interleave(G, dim=2)
    vv = v.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) * scale
    m = torch.as_tensor(mask)
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.exp(s - lse[..., None])
    p = torch.nan_to_num(p, nan=0.0)
    o = torch.einsum("bhij,bjhd->bihd", p, vv)
    return o, lse.permute(0, 2, 1)


def rand_inputs(batch, L, hq, hkv, d, seed, bf16=False):
    g = np.random.default_rng(seed)
    n2 = 2 * L
    arrs = [g.standard_normal((batch, n2, h, d)).astype(np.float32)
            for h in (hq, hkv, hkv, hq)]
    if bf16:
        arrs = [torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                for a in arrs]
    return arrs


def as_f64(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(a).double()


SHAPES = [
    # batch, L, M, hq, hkv, d, token_causal
    (1, 8, 2, 1, 1, 4, False),
    (2, 16, 4, 4, 2, 8, False),
    (1, 16, 4, 3, 1, 8, True),
    (1, 12, 3, 2, 2, 6, False),
    (1, 16, 1, 2, 1, 4, False),
    (1, 16, 16, 2, 2, 4, False),
]


# ---------------------------------------------------------------- mask pins
def test_mask_matches_golden(orc):
    rows = [ln.strip() for ln in open(os.path.join(GOLD, "mask_L8_M2.txt"))
            if ln.strip() and not ln.startswith("#")]
    gold = np.array([[c == "1" for c in r] for r in rows])
    p = orc.problem(1, 8, 2, 1, 1, 4)
    got = np.array([[orc.visible(p, i, j) for j in range(16)] for i in range(16)], dtype=bool)
    assert gold.shape == (16, 16)
    assert (got == gold).all()
    assert gold.sum() == 8 * (8 + 2)


@pytest.mark.parametrize("L,M", [(8, 2), (12, 3), (16, 1), (16, 16), (24, 4), (32, 8)])
@pytest.mark.parametrize("token_causal", [False, True])
def test_mask_counts_closed_form(orc, L, M, token_causal):
    p = orc.problem(1, L, M, 1, 1, 4, token_causal=token_causal)
    vis = np.array([[orc.visible(p, i, j) for j in range(2 * L)] for i in range(2 * L)], dtype=bool)
    assert (vis == dense_mask(L, M, token_causal)).all()
    for i in range(L):
        n = i + 1 if token_causal else (i // M + 1) * M
        assert vis[i].sum() == n
    for t in range(L):
        b = t // M
        assert vis[L + t].sum() == (b + 1) * M
    total = L * L + L * M // 2 + L // 2 if token_causal else L * (L + M)
    if token_causal:
        # clean part is L(L+1)/2, corrupted part L*M/2 + L*L/2 ... as a sum
        assert vis.sum() == L * (L + 1) // 2 + sum((t // M + 1) * M for t in range(L))
        if M == 1:
            assert vis.sum() == total
    else:
        assert vis.sum() == total


# ---------------------------------------------------------------- forward pins
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
def test_fwd_matches_dense(orc, shape, bf16):
    batch, L, M, hq, hkv, d, tc = shape
    q, k, v, _ = rand_inputs(batch, L, hq, hkv, d, seed=L * 7 + M, bf16=bf16)
    p = orc.problem(batch, L, M, hq, hkv, d, token_causal=tc, bf16=bf16)
    o, lse = orc.fwd(p, orc.keys(), q, k, v)
    ro, rlse = dense_attention(as_f64(q), as_f64(k), as_f64(v), dense_mask(L, M, tc), p.scale)
    np.testing.assert_allclose(o, ro.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES[:4])
def test_bwd_matches_autograd(orc, shape):
    batch, L, M, hq, hkv, d, tc = shape
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=11 + L)
    p = orc.problem(batch, L, M, hq, hkv, d, token_causal=tc)
    dq, dk, dv = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    tq, tk, tv = (as_f64(x).requires_grad_(True) for x in (q, k, v))
    o, _ = dense_attention(tq, tk, tv, dense_mask(L, M, tc), p.scale)
    (o * as_f64(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def test_sdpa_special_cases(orc):
    """M = L: each copy reduces to plain non-causal attention over itself
    (the corrupted copy is one block with no clean prefix).  M = 1: the clean
    copy is standard causal attention and block-causal equals token-causal."""
    F = torch.nn.functional
    batch, L, hq, d = 2, 16, 2, 8
    q, k, v, _ = rand_inputs(batch, L, hq, hq, d, seed=5)
    tq, tk, tv = (as_f64(x).transpose(1, 2) for x in (q, k, v))  # [b,h,n,d]
    p = orc.problem(batch, L, L, hq, hq, d)
    o, _ = orc.fwd(p, orc.keys(), q, k, v)
    ref_c = F.scaled_dot_product_attention(tq[:, :, :L], tk[:, :, :L], tv[:, :, :L])
    ref_x = F.scaled_dot_product_attention(tq[:, :, L:], tk[:, :, L:], tv[:, :, L:])
    np.testing.assert_allclose(o[:, :L], ref_c.transpose(1, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(o[:, L:], ref_x.transpose(1, 2).numpy(), atol=1e-12)
    p1 = orc.problem(batch, L, 1, hq, hq, d)
    p1t = orc.problem(batch, L, 1, hq, hq, d, token_causal=True)
    o1, l1 = orc.fwd(p1, orc.keys(), q, k, v)
    o1t, l1t = orc.fwd(p1t, orc.keys(), q, k, v)
    ref = F.scaled_dot_product_attention(tq[:, :, :L], tk[:, :, :L], tv[:, :, :L], is_causal=True)
    np.testing.assert_allclose(o1[:, :L], ref.transpose(1, 2).numpy(), atol=1e-12)
    assert np.array_equal(o1, o1t) and np.array_equal(l1, l1t)


def test_zero_keys_and_constant_values(orc):
    """K = 0: every visible logit is 0, so LSE_i = ln(n_i) and O_i is the mean
    of the visible V rows.  V constant: O equals that constant."""
    batch, L, M, hq, d = 1, 16, 4, 2, 4
    q, k, v, _ = rand_inputs(batch, L, hq, hq, d, seed=9)
    k0 = np.zeros_like(k)
    p = orc.problem(batch, L, M, hq, hq, d)
    o, lse = orc.fwd(p, orc.keys(), q, k0, v)
    mask = dense_mask(L, M)
    n = mask.sum(1)
    np.testing.assert_allclose(lse[0], np.log(n)[:, None].repeat(hq, 1), atol=1e-14)
    vm = (mask[:, :, None, None] * v[0][None].astype(np.float64)).sum(1) / n[:, None, None]
    np.testing.assert_allclose(o[0], vm, atol=1e-12)
    vc = np.full_like(v, 0.375)
    oc, _ = orc.fwd(p, orc.keys(), q, k, vc)
    np.testing.assert_allclose(oc, 0.375, atol=1e-14)


def test_softmax_invariants(orc):
    """max s <= LSE <= max s + ln n_i and O inside the per-column hull of the
    visible V rows."""
    batch, L, M, hq, d = 1, 16, 4, 1, 8
    q, k, v, _ = rand_inputs(batch, L, hq, hq, d, seed=21)
    p = orc.problem(batch, L, M, hq, hq, d)
    o, lse = orc.fwd(p, orc.keys(), q, k, v)
    mask = dense_mask(L, M)
    s = np.einsum("id,jd->ij", q[0, :, 0].astype(np.float64), k[0, :, 0].astype(np.float64)) * p.scale
    s[~mask] = -np.inf
    smax = s.max(1)
    assert (lse[0, :, 0] >= smax - 1e-12).all()
    assert (lse[0, :, 0] <= smax + np.log(mask.sum(1)) + 1e-12).all()
    for i in range(2 * L):
        vis = v[0, mask[i], 0].astype(np.float64)
        assert (o[0, i, 0] >= vis.min(0) - 1e-12).all() and (o[0, i, 0] <= vis.max(0) + 1e-12).all()


# ---------------------------------------------------------------- GQA
def test_gqa_equals_repeated_mha(orc):
    batch, L, M, hq, hkv, d = 1, 16, 4, 6, 2, 4
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=3)
    G = hq // hkv
    kr, vr = (np.ascontiguousarray(np.repeat(x, G, axis=2)) for x in (k, v))
    pg = orc.problem(batch, L, M, hq, hkv, d)
    pm = orc.problem(batch, L, M, hq, hq, d)
    og, lg = orc.fwd(pg, orc.keys(), q, k, v)
    om, lm = orc.fwd(pm, orc.keys(), q, kr, vr)
    np.testing.assert_allclose(og, om, atol=1e-14)
    np.testing.assert_allclose(lg, lm, atol=1e-14)
    _, dkg, dvg = orc.bwd(pg, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    _, dkm, dvm = orc.bwd(pm, orc.share(), orc.keys(), orc.keys(), q, kr, vr, do)
    np.testing.assert_allclose(dkg, dkm.reshape(batch, 2 * L, hkv, G, d).sum(3), atol=1e-12)
    np.testing.assert_allclose(dvg, dvm.reshape(batch, 2 * L, hkv, G, d).sum(3), atol=1e-12)


# ---------------------------------------------------------------- BP identity
def test_bp_identity_forward(orc):
    """Block b alone, Attn(Q_b, [K_b; K^clean_<b], [V_b; V^clean_<b]) ("CSBP
    完全拆解", CSBP forward equation), computed by plain SDPA on the
    concatenated keys, equals the monolithic masked rows."""
    F = torch.nn.functional
    batch, L, M, hq, d = 1, 16, 4, 2, 8
    q, k, v, _ = rand_inputs(batch, L, hq, hq, d, seed=13)
    p = orc.problem(batch, L, M, hq, hq, d)
    o, lse = orc.fwd(p, orc.keys(), q, k, v)
    tq, tk, tv = (as_f64(x).transpose(1, 2) for x in (q, k, v))
    for b in range(L // M):
        rows = slice(L + b * M, L + (b + 1) * M)
        kb = torch.cat([tk[:, :, rows], tk[:, :, : b * M]], dim=2)
        vb = torch.cat([tv[:, :, rows], tv[:, :, : b * M]], dim=2)
        ob = F.scaled_dot_product_attention(tq[:, :, rows], kb, vb)
        np.testing.assert_allclose(o[:, rows], ob.transpose(1, 2).numpy(), atol=1e-12)
        # the same rows from the row API
        bi = np.zeros(M * hq, np.int32)
        hi = np.tile(np.arange(hq, dtype=np.int32), M)
        ii = np.repeat(np.arange(rows.start, rows.stop), hq)
        orow, lrow = orc.fwd_rows(p, orc.keys(), q, k, v, bi, hi, ii)
        np.testing.assert_array_equal(orow.reshape(M, hq, d), o[0, rows])
        np.testing.assert_array_equal(lrow.reshape(M, hq), lse[0, rows])


def test_bp_identity_gradients(orc):
    """L = sum_b L_b and sum_r grad L_r = grad L ("CSBP 完全拆解", section
    "BP：把损坏块留在本地", gradient-sum equation): per-block shares plus the
    clean rows' share sum to the monolithic gradient."""
    batch, L, M, hq, hkv, d = 1, 16, 4, 4, 2, 4
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=17)
    p = orc.problem(batch, L, M, hq, hkv, d)
    full = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    acc = [np.zeros_like(x) for x in full]
    shares = [orc.share(L, M, blocks=[b]) for b in range(L // M)]
    shares.append(orc.share(L, M, clean=[(0, L)]))
    for sh in shares:
        part = orc.bwd(p, sh, orc.keys(), orc.keys(), q, k, v, do)
        for a, x in zip(acc, part):
            a += x
    for a, x in zip(acc, full):
        np.testing.assert_allclose(a, x, atol=1e-12)


# ---------------------------------------------------------------- CSBP identity
def test_merge_golden(orc):
    line = [ln for ln in open(os.path.join(GOLD, "merge_closed_form.txt")) if not ln.startswith("#")][0]
    a, b, c = (np.array([float(x) for x in part.split()]) for part in line.split("|"))
    o, z = orc.merge(a[None, :2], a[None, 2:], b[None, :2], b[None, 2:])
    np.testing.assert_allclose(o[0], c[:2], atol=1e-15)
    np.testing.assert_allclose(z[0], c[2], atol=1e-15)
    assert abs(c[2] - math.log(4.0)) < 1e-15


def test_merge_identity_and_extremes(orc):
    g = np.random.default_rng(0)
    o1 = g.standard_normal((5, 3))
    z1 = np.array([-np.inf, 0.5, 120.0, -300.0, 2.0])
    zero = np.zeros_like(o1)
    ninf = np.full(5, -np.inf)
    o, z = orc.merge(o1, z1, zero, ninf)
    np.testing.assert_array_equal(o[1:], o1[1:])
    np.testing.assert_array_equal(z, z1)
    np.testing.assert_array_equal(o[0], 0.0)
    o, z = orc.merge(zero, ninf, zero, ninf)
    assert np.all(o == 0) and np.all(z == -np.inf)
    o, z = orc.merge(o1, z1, o1, z1 + 1.0)
    assert np.isfinite(o[1:]).all() and np.isfinite(z[1:]).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_csbp_merge_equals_unsharded(orc, seed):
    """LSE merge over any split of the clean keys equals the unsharded result
    ("CSBP 完全拆解", section "在线 softmax 合并": exact, not an
    approximation).  The local corrupted part is merged first, then pieces."""
    g = np.random.default_rng(seed)
    batch, L, M, hq, hkv, d = 1, 32, 4, 4, 2, 8
    q, k, v, _ = rand_inputs(batch, L, hq, hkv, d, seed=100 + seed)
    p = orc.problem(batch, L, M, hq, hkv, d)
    o_ref, l_ref = orc.fwd(p, orc.keys(), q, k, v)
    cuts = np.sort(g.choice(np.arange(1, L), size=5, replace=False))
    edges = [0, *cuts.tolist(), L]
    pieces = [(edges[t], edges[t + 1]) for t in range(len(edges) - 1)]
    g.shuffle(pieces)
    o_acc, l_acc = orc.fwd(p, orc.keys([], local=True), q, k, v)
    # pieces of two ranges each (like zigzag shards), plus an empty piece
    groups = [pieces[t:t + 2] for t in range(0, len(pieces), 2)] + [[]]
    for grp in groups:
        o_s, l_s = orc.fwd(p, orc.keys(grp, local=False), q, k, v)
        o_acc, l_acc = orc.merge(o_acc, l_acc, o_s, l_s)
    np.testing.assert_allclose(o_acc, o_ref, atol=1e-12)
    np.testing.assert_allclose(l_acc, l_ref, atol=1e-12)


def test_csbp_sharded_backward_sums(orc):
    """Per-shard backward with the final LSE (softmax over every key, pairs
    restricted to the shard) sums to the unsharded gradient."""
    batch, L, M, hq, hkv, d = 1, 32, 4, 4, 2, 4
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=23)
    p = orc.problem(batch, L, M, hq, hkv, d)
    P = 4
    full = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    calls = [orc.keys([], local=True)] + [orc.keys(orc.clean_shard(L, P, s), local=False) for s in range(P)]
    acc = [np.zeros_like(x) for x in full]
    for kg in calls:
        part = orc.bwd(p, orc.share(), orc.keys(), kg, q, k, v, do)
        for a, x in zip(acc, part):
            a += x
    for a, x in zip(acc, full):
        np.testing.assert_allclose(a, x, atol=1e-12)


def test_row_apis_match_full(orc):
    """dq_rows / dkdv_rows on a share equal the matching rows of orc_bwd."""
    batch, L, M, hq, hkv, d = 2, 16, 4, 4, 2, 4
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=29)
    p = orc.problem(batch, L, M, hq, hkv, d)
    sh = orc.share(L, M, clean=[(4, 8), (12, 16)], blocks=[0, 3])
    kn, kg = orc.keys(), orc.keys([(0, 4), (8, 12)], local=True)
    dq, dk, dv = orc.bwd(p, sh, kn, kg, q, k, v, do)
    rows = [(0, 1, 5), (1, 3, L + 13), (0, 0, L + 1), (1, 2, 13)]
    b, h, i = (np.array(c) for c in zip(*rows))
    dqr, _, _ = orc.dq_rows(p, kn, kg, q, k, v, do, b, h, i)
    np.testing.assert_allclose(dqr, dq[b, i, h], atol=1e-13)
    keys = [(0, 0, 1), (1, 1, 9), (0, 1, L + 2), (1, 0, L + 14), (0, 0, 5)]
    b, g_, j = (np.array(c) for c in zip(*keys))
    dkr, dvr = orc.dkdv_rows(p, sh, kn, kg, q, k, v, do, b, g_, j)
    np.testing.assert_allclose(dkr, dk[b, j, g_], atol=1e-13)
    np.testing.assert_allclose(dvr, dv[b, j, g_], atol=1e-13)


# ---------------------------------------------------------------- isolation
def test_corrupted_kv_isolation(orc):
    """Corrupted K/V of block j are read only by block j's queries (Turbo-dLLM
    page, "Method"): perturbing them leaves every other row bitwise equal."""
    batch, L, M, hq, hkv, d = 1, 16, 4, 2, 1, 8
    q, k, v, _ = rand_inputs(batch, L, hq, hkv, d, seed=31)
    p = orc.problem(batch, L, M, hq, hkv, d)
    o, lse = orc.fwd(p, orc.keys(), q, k, v)
    jb = 2
    rows = slice(L + jb * M, L + (jb + 1) * M)
    k2, v2 = k.copy(), v.copy()
    k2[:, rows] += 3.0
    v2[:, rows] -= 5.0
    o2, lse2 = orc.fwd(p, orc.keys(), q, k2, v2)
    keep = np.ones(2 * L, dtype=bool)
    keep[rows] = False
    assert np.array_equal(o[:, keep], o2[:, keep]) and np.array_equal(lse[:, keep], lse2[:, keep])
    assert not np.array_equal(o[:, rows], o2[:, rows])


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("tc", [False, True])
def test_finite_differences(orc, tc):
    batch, L, M, hq, hkv, d = 1, 32, 4, 4, 2, 8
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=37 + tc)
    p = orc.problem(batch, L, M, hq, hkv, d, token_causal=tc)
    dq, dk, dv = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    eps = 2.0 ** -14  # exact in float32 for these magnitudes
    do64 = do.astype(np.float64)

    def loss(qq, kk, vv):
        o, _ = orc.fwd(p, orc.keys(), qq, kk, vv)
        return float((o * do64).sum())

    g = np.random.default_rng(41)
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(4):
            base = {"q": q, "k": k, "v": v}
            arr = base[which]
            idx = tuple(int(g.integers(0, s)) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            assert plus[idx] - arr[idx] == np.float32(eps)
            bp = dict(base, **{which: plus})
            bm = dict(base, **{which: minus})
            fd = (loss(bp["q"], bp["k"], bp["v"]) - loss(bm["q"], bm["k"], bm["v"])) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


# ---------------------------------------------------------------- sliding window
WINDOWS = [(16, 4, 1), (16, 4, 3), (16, 4, 4), (16, 4, 7), (24, 4, 9), (32, 8, 5), (16, 1, 4),
           (16, 16, 5), (16, 4, 40)]


@pytest.mark.parametrize("L,M,W", WINDOWS)
@pytest.mark.parametrize("token_causal", [False, True])
def test_window_mask_counts_closed_form(orc, L, M, W, token_causal):
    """Per-row visible counts under a clean-key window of W tokens, derived by
    hand: clean block-causal row t sees (t//M + 1) M - max(0, t - W + 1),
    clean token-causal row t sees min(t + 1, W), corrupted row (block b,
    offset i) sees M + max(0, min(b M, W - 1 - i))."""
    p = orc.problem(1, L, M, 1, 1, 4, token_causal=token_causal, window=W)
    vis = np.array([[orc.visible(p, i, j) for j in range(2 * L)] for i in range(2 * L)], dtype=bool)
    assert (vis == dense_mask(L, M, token_causal, W)).all()
    for t in range(L):
        n = min(t + 1, W) if token_causal else (t // M + 1) * M - max(0, t - W + 1)
        assert vis[t].sum() == n
        b, i = divmod(t, M)
        assert vis[L + t].sum() == M + max(0, min(b * M, W - 1 - i))


WSHAPES = [
    # batch, L, M, hq, hkv, d, token_causal, window
    (1, 16, 4, 2, 1, 8, False, 6),
    (2, 16, 4, 4, 2, 4, True, 5),
    (1, 24, 3, 2, 2, 6, False, 2),
    (1, 16, 8, 2, 1, 4, False, 9),
]


@pytest.mark.parametrize("shape", WSHAPES)
def test_window_fwd_bwd_match_dense(orc, shape):
    batch, L, M, hq, hkv, d, tc, W = shape
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=51 + W)
    p = orc.problem(batch, L, M, hq, hkv, d, token_causal=tc, window=W)
    o, lse = orc.fwd(p, orc.keys(), q, k, v)
    dq, dk, dv = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    tq, tk, tv = (as_f64(x).requires_grad_(True) for x in (q, k, v))
    ro, rlse = dense_attention(tq, tk, tv, dense_mask(L, M, tc, W), p.scale)
    np.testing.assert_allclose(o, ro.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse.detach().numpy(), rtol=0, atol=1e-12)
    (ro * as_f64(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def test_window_sdpa_special_case(orc):
    """M = 1, token-causal: the clean copy is standard causal sliding-window
    attention; torch's SDPA with a banded causal mask (tril, then triu)."""
    F = torch.nn.functional
    batch, L, hq, d, W = 2, 16, 2, 8, 5
    q, k, v, _ = rand_inputs(batch, L, hq, hq, d, seed=57)
    tq, tk, tv = (as_f64(x).transpose(1, 2) for x in (q, k, v))
    p = orc.problem(batch, L, 1, hq, hq, d, token_causal=True, window=W)
    o, _ = orc.fwd(p, orc.keys(), q, k, v)
    band = torch.ones(L, L, dtype=torch.bool).tril().triu(-(W - 1))
    ref = F.scaled_dot_product_attention(tq[:, :, :L], tk[:, :, :L], tv[:, :, :L], attn_mask=band)
    np.testing.assert_allclose(o[:, :L], ref.transpose(1, 2).numpy(), atol=1e-12)


def test_window_wide_is_none(orc):
    """A window at least as long as the sequence changes nothing, bit for bit."""
    batch, L, M, hq, hkv, d = 1, 16, 4, 2, 1, 8
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=59)
    p0 = orc.problem(batch, L, M, hq, hkv, d)
    pw = orc.problem(batch, L, M, hq, hkv, d, window=L)
    for a, b in zip(orc.fwd(p0, orc.keys(), q, k, v), orc.fwd(pw, orc.keys(), q, k, v)):
        assert np.array_equal(a, b)
    for a, b in zip(orc.bwd(p0, orc.share(), orc.keys(), orc.keys(), q, k, v, do),
                    orc.bwd(pw, orc.share(), orc.keys(), orc.keys(), q, k, v, do)):
        assert np.array_equal(a, b)


def test_window_csbp_identities(orc):
    """Under a window the LSE merge over zigzag shards still equals the
    unsharded forward, and the per-shard backward still sums to the full
    gradient (shards far outside a row's window contribute the identity)."""
    batch, L, M, hq, hkv, d, W, P = 1, 32, 4, 4, 2, 4, 7, 4
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=61)
    p = orc.problem(batch, L, M, hq, hkv, d, window=W)
    o_ref, l_ref = orc.fwd(p, orc.keys(), q, k, v)
    o_acc, l_acc = orc.fwd(p, orc.keys([], local=True), q, k, v)
    calls = [orc.keys(orc.clean_shard(L, P, s), local=False) for s in range(P)]
    for kg in calls:
        o_s, l_s = orc.fwd(p, kg, q, k, v)
        o_acc, l_acc = orc.merge(o_acc, l_acc, o_s, l_s)
    np.testing.assert_allclose(o_acc, o_ref, atol=1e-12)
    np.testing.assert_allclose(l_acc, l_ref, atol=1e-12)
    full = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    acc = [np.zeros_like(x) for x in full]
    for kg in [orc.keys([], local=True)] + calls:
        for a, x in zip(acc, orc.bwd(p, orc.share(), orc.keys(), kg, q, k, v, do)):
            a += x
    for a, x in zip(acc, full):
        np.testing.assert_allclose(a, x, atol=1e-12)


def test_window_finite_differences(orc):
    batch, L, M, hq, hkv, d, W = 1, 16, 4, 2, 1, 4, 6
    q, k, v, do = rand_inputs(batch, L, hq, hkv, d, seed=67)
    p = orc.problem(batch, L, M, hq, hkv, d, window=W)
    dq, dk, dv = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), q, k, v, do)
    eps = 2.0 ** -14
    do64 = do.astype(np.float64)
    g = np.random.default_rng(71)
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(4):
            base = {"q": q, "k": k, "v": v}
            idx = tuple(int(g.integers(0, s)) for s in base[which].shape)
            vals = []
            for sgn in (1, -1):
                a = base[which].copy()
                a[idx] += sgn * eps
                bb = dict(base, **{which: a})
                o, _ = orc.fwd(p, orc.keys(), bb["q"], bb["k"], bb["v"])
                vals.append(float((o * do64).sum()))
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


# ---------------------------------------------------------------- assignment
def test_assignment_golden(orc):
    for ln in open(os.path.join(GOLD, "assign_B16_P4.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        r, ids = ln.split(":")
        assert orc.assign_blocks(16, 4, int(r)).tolist() == [int(x) for x in ids.split()]


@pytest.mark.parametrize("B,P", [(16, 4), (64, 8), (8192, 8), (32768, 16), (6, 3), (2, 1)])
def test_assignment_partition_and_balance(orc, B, P):
    seen = np.zeros(B, dtype=int)
    c = B // (2 * P)
    for r in range(P):
        br = orc.assign_blocks(B, P, r)
        assert len(br) == B // P and (np.diff(br) > 0).all()
        # independent formulation: 2P equal chunks, rank r takes chunk r and chunk 2P-1-r
        chunks = np.arange(B).reshape(2 * P, c)
        assert np.array_equal(br, np.concatenate([chunks[r], chunks[2 * P - 1 - r]]))
        # every rank carries the same total prefix length
        assert br.sum() == (B // P) * (B - 1) // 2
        seen[br] += 1
    assert (seen == 1).all()
    with pytest.raises(ValueError):
        orc.assign_blocks(B + 1, P, 0)


@pytest.mark.parametrize("L,P,M", [(64, 4, 4), (262144, 8, 32), (524288, 16, 16)])
def test_clean_shards(orc, L, P, M):
    cover = np.zeros(L, dtype=np.int8) if L <= 65536 else None
    works = []
    for s in range(P):
        rng = orc.clean_shard(L, P, s)
        assert len(rng) == 2 and all(hi - lo == L // (2 * P) for lo, hi in rng)
        if cover is not None:
            for lo, hi in rng:
                cover[lo:hi] += 1
        # block-causal clean-query work of the shard: sum over tokens of (t//M + 1) M
        w = 0
        for lo, hi in rng:
            b0, b1 = lo // M, hi // M
            w += M * M * ((b1 * (b1 + 1) - b0 * (b0 + 1)) // 2)
        works.append(w)
    if cover is not None:
        assert (cover == 1).all()
    assert len(set(works)) == 1
