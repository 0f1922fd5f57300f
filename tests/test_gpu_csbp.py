"""GPU parity of the CSBP per-rank form: a rank's dual-end block share (plus
its zigzag clean shard of query rows) attended against its own corrupted keys
and then the clean key shards one at a time, merged by log-sum-exp; backward
with the final O/LSE per call.

Virtual ranks: all P shares are run on one GPU; the union of their rows must
match the oracle's whole-mask rows, the sum of their clean dK/dV partials
(the stand-in for the owner reduce-scatter) the oracle's whole-mask clean
dK/dV, and their corrupted dK/dV the oracle's rows of those blocks.
Bar: O (fp32 merged) max|err| <= 2e-2, LSE <= 1e-3, gradients rel-L2 <= 1e-2.
"""
import numpy as np
import pytest
import torch

from tests.common import (TOL_GRAD, TOL_LSE, TOL_O, csbp_inputs, doubled_host, host_bits, max_abs,
                          rel_l2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdattn
    bdattn.lib()
    return torch.device("cuda:0")


def _rank(dev, L, M, hq, hkv, d, P, r, clean_queries, seed, window=0):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    blocks = B.bdattn_assign_blocks(L // M, P, r).tolist()
    cs = B.bdattn_clean_shard(L, P, r)
    clean_q = [(cs.lo[0], cs.hi[0]), (cs.lo[1], cs.hi[1])] if clean_queries else []
    shards = []
    for s in range(P):
        k = B.bdattn_clean_shard(L, P, s)
        shards.append([(k.lo[0], k.hi[0]), (k.lo[1], k.hi[1])])
    t = csbp_inputs(seed, L, M, hq, hkv, d, blocks, clean_q, device=dev)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, shards, window=window)
    o32, lse, obf = sh.fwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"])
    grads = sh.bwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"],
                   o32, lse, t["do"])
    torch.cuda.synchronize()
    return blocks, clean_q, t, o32, lse, obf, grads


@pytest.mark.parametrize("L,M,hq,hkv,d,P,W", [(1024, 16, 4, 2, 128, 4, 0), (768, 32, 2, 1, 64, 3, 0),
                                              (512, 8, 4, 4, 128, 2, 0), (1024, 16, 4, 2, 128, 4, 200)])
def test_virtual_ranks(dev, orc, L, M, hq, hkv, d, P, W):
    """W > 0: the same under a clean-key sliding window of W tokens (most
    shards are then outside most rows' windows and contribute the identity)."""
    seed = 100 + L
    # every rank uses the same clean K/V (shared context) and its own corrupted / query rows:
    # build the oracle's doubled input from all ranks' pieces
    ranks = [_rank(dev, L, M, hq, hkv, d, P, r, True, seed, window=W) for r in range(P)]
    qh = np.zeros((1, 2 * L, hq, d), np.uint16)
    doh = np.zeros_like(qh)
    kh = np.zeros((1, 2 * L, hkv, d), np.uint16)
    vh = np.zeros_like(kh)
    for blocks, clean_q, t, *_ in ranks:
        q_, k_, v_, do_, pos = doubled_host(L, hq, hkv, d, t, blocks, clean_q, M)
        qh[0, pos] = q_[0, pos]
        doh[0, pos] = do_[0, pos]
        kh[0, :L] = k_[0, :L]
        vh[0, :L] = v_[0, :L]
        kx = pos[len(pos) - len(blocks) * M:]
        kh[0, kx] = k_[0, kx]
        vh[0, kx] = v_[0, kx]
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True, window=W)
    o_ref, lse_ref = orc.fwd(p, orc.keys(), qh, kh, vh)
    dq_ref, dk_ref, dv_ref = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), qh, kh, vh, doh)
    dkc = np.zeros((L, hkv, d))
    dvc = np.zeros((L, hkv, d))
    covered = np.zeros(2 * L, dtype=int)
    for blocks, clean_q, t, o32, lse, obf, grads in ranks:
        from tests.common import share_positions
        pos = share_positions(L, M, blocks, clean_q)
        covered[pos] += 1
        assert max_abs(o32.cpu().numpy()[0], o_ref[0, pos]) <= TOL_O
        assert max_abs(obf.float().cpu().numpy()[0], o_ref[0, pos]) <= TOL_O
        assert max_abs(lse.cpu().numpy()[0], lse_ref[0, pos]) <= TOL_LSE
        dq, gkc, gvc, gkx, gvx, _ = grads
        assert rel_l2(dq.cpu().numpy()[0], dq_ref[0, pos]) <= TOL_GRAD
        kx = pos[len(pos) - len(blocks) * M:]
        assert rel_l2(gkx.cpu().numpy()[0], dk_ref[0, kx]) <= TOL_GRAD
        assert rel_l2(gvx.cpu().numpy()[0], dv_ref[0, kx]) <= TOL_GRAD
        dkc += gkc.cpu().numpy()[0]
        dvc += gvc.cpu().numpy()[0]
    assert (covered == 1).all()  # the shares partition every query row
    assert rel_l2(dkc, dk_ref[0, :L]) <= TOL_GRAD
    assert rel_l2(dvc, dv_ref[0, :L]) <= TOL_GRAD


def test_shard_merge_kernel(dev, orc):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    g = torch.Generator().manual_seed(5)
    rows, d = 1000, 128
    o1 = torch.randn(rows, d, generator=g)
    o2 = torch.randn(rows, d, generator=g)
    z1 = torch.randn(rows, generator=g) * 30
    z2 = torch.randn(rows, generator=g) * 30
    z1[:50] = float("-inf")
    o1[:50] = 0
    z2[25:75] = float("-inf")
    o2[25:75] = 0
    z2[100:110] = z1[100:110]  # ties
    ref_o, ref_z = orc.merge(o1.numpy(), z1.numpy(), o2.numpy(), z2.numpy())
    acc, lacc = o1.to(dev), z1.to(dev)
    obf = torch.empty(rows, d, dtype=torch.bfloat16, device=dev)
    B.bdattn_shard_merge(rows, d, acc, lacc, o2.to(dev), z2.to(dev), obf)
    torch.cuda.synchronize()
    assert max_abs(acc.cpu().numpy(), ref_o) <= 1e-5
    assert max_abs(lacc.cpu().numpy(), ref_z) <= 1e-5
    assert torch.isinf(lacc[25:50]).all() and (acc[25:50] == 0).all()
    assert max_abs(obf.float().cpu().numpy(), ref_o) <= 2e-2


@pytest.mark.parametrize("seed", [0, 1])
def test_random_key_splits(dev, orc, seed):
    """Whole share, clean keys split into random pieces (two ranges per call),
    merged by LSE: equals the oracle's unsharded result."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    rng = np.random.default_rng(seed)
    L, M, hq, hkv, d = 640, 16, 4, 2, 128
    cuts = np.sort(rng.choice(np.arange(1, L), size=5, replace=False)).tolist()
    edges = [0, *cuts, L]
    pieces = [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]
    rng.shuffle(pieces)
    shards = [sorted(pieces[i:i + 2]) for i in range(0, len(pieces), 2)]
    blocks = list(range(L // M))
    t = csbp_inputs(200 + seed, L, M, hq, hkv, d, blocks, [(0, L)], device=dev)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, [(0, L)], shards)
    o32, lse, _ = sh.fwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"])
    torch.cuda.synchronize()
    q, k, v, do, pos = doubled_host(L, hq, hkv, d, t, blocks, [(0, L)], M)
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True)
    o_ref, lse_ref = orc.fwd(p, orc.keys(), q, k, v)
    assert max_abs(o32.cpu().numpy()[0], o_ref[0, pos]) <= TOL_O
    assert max_abs(lse.cpu().numpy()[0], lse_ref[0, pos]) <= TOL_LSE


def test_empty_rows_in_a_shard(dev):
    """Early blocks see nothing in late shards: those calls give (0, -inf)
    rows and the merge keeps the accumulator unchanged."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    L, M, hq, hkv, d = 512, 32, 2, 1, 128
    blocks = [0, 1, 14, 15]
    t = csbp_inputs(300, L, M, hq, hkv, d, blocks, [], device=dev)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, [], [[(256, 512)]])
    o = torch.empty(1, sh.R, hq, d, dtype=torch.float32, device=dev)
    lse = torch.empty(1, sh.R, hq, dtype=torch.float32, device=dev)
    ws = sh.workspace(False, dev)
    B.bdattn_fwd(sh.prob, sh.share, sh.kv_shards[0], t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"],
                 t["k_corr"], t["v_corr"], o, B.BDATTN_F32, lse, ws)
    torch.cuda.synchronize()
    early = slice(0, 2 * M)  # blocks 0, 1 see only clean keys < 64: none in [256, 512)
    assert torch.isinf(lse[:, early]).all() and (lse[:, early] < 0).all()
    assert (o[:, early] == 0).all()
    assert torch.isfinite(lse[:, 2 * M:]).all()
