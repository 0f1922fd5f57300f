"""GPU parity on seeded random problems: combinations of batch, head size,
GQA group, block size (odd ones included), sequence length, clean-copy mask
and sliding window that the fixed shapes do not pair up.  Whole-mask cases
and single-rank CSBP shares (random P, rank, clean query shard and window),
forward and backward, checked element by element against the oracle.

Bar: bf16 O max|err| <= 2e-2, LSE <= 1e-3, dQ/dK/dV relative L2 <= 1e-2.
"""
import numpy as np
import pytest
import torch

from tests.common import TOL_GRAD, TOL_LSE, TOL_O, doubled_inputs, host_bits, max_abs, rel_l2

pytestmark = pytest.mark.gpu

N_CASES = 32


def _case(i):
    """Parameters of case i, from a generator seeded by i alone."""
    rng = np.random.default_rng(7000 + i)
    batch = int(rng.choice([1, 2]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 5]))
    M = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 32, 48, 64, 100, 128]))
    nb = int(rng.integers(1, max(2, 600 // M) + 1))
    L = M * nb
    token_causal = bool(rng.integers(0, 2))
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 2 * L + 1))
    return batch, L, M, hkv * G, hkv, d, token_causal, window


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdattn
    bdattn.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_whole_mask(dev, orc, i):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    batch, L, M, hq, hkv, d, tc, W = _case(i)
    print(f"\n[case {i}] batch={batch} L={L} M={M} hq={hq} hkv={hkv} d={d} token_causal={tc} window={W}",
          flush=True)
    q, k, v, do = doubled_inputs(8000 + i, batch, L, hq, hkv, d, device=dev)
    wm = WholeMask(batch, L, M, hq, hkv, d, B.BDATTN_BF16,
                   B.BDATTN_CLEAN_TOKEN_CAUSAL if tc else B.BDATTN_CLEAN_BLOCK_CAUSAL, window=W)
    o, lse = wm.fwd(q, k, v, o_dtype=torch.float32)
    dq, dk, dv = wm.bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    p = orc.problem(batch, L, M, hq, hkv, d, token_causal=tc, bf16=True, window=W)
    hq_, hk_, hv_, hdo = (host_bits(x) for x in (q, k, v, do))
    o_ref, lse_ref = orc.fwd(p, orc.keys(), hq_, hk_, hv_)
    assert max_abs(o.cpu().numpy(), o_ref) <= TOL_O
    assert max_abs(lse.cpu().numpy(), lse_ref) <= TOL_LSE
    dq_ref, dk_ref, dv_ref = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), hq_, hk_, hv_, hdo)
    assert rel_l2(dq.cpu().numpy(), dq_ref) <= TOL_GRAD
    assert rel_l2(dk.cpu().numpy(), dk_ref) <= TOL_GRAD
    assert rel_l2(dv.cpu().numpy(), dv_ref) <= TOL_GRAD


def _share_case(i):
    rng = np.random.default_rng(9000 + i)
    P = int(rng.integers(1, 5))
    M = int(rng.choice([4, 8, 16, 32]))
    nb = 2 * P * int(rng.integers(1, max(2, 512 // (2 * P * M)) + 1))
    L = M * nb
    r = int(rng.integers(0, P))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 5]))
    clean_queries = bool(rng.integers(0, 2))
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 2 * L + 1))
    return L, M, hkv * G, hkv, d, P, r, clean_queries, window


@pytest.mark.parametrize("i", range(16))
def test_random_csbp_share(dev, orc, i):
    """One rank's share: local call, P clean shards streamed and merged,
    backward per call; its rows, its clean dK/dV partial and its corrupted
    dK/dV against the oracle's share-restricted results."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    from tests.common import csbp_inputs, doubled_host, share_positions
    L, M, hq, hkv, d, P, r, cq, W = _share_case(i)
    print(f"\n[share case {i}] L={L} M={M} hq={hq} hkv={hkv} d={d} P={P} r={r} clean_q={cq} window={W}", flush=True)
    blocks = B.bdattn_assign_blocks(L // M, P, r).tolist()
    cs = B.bdattn_clean_shard(L, P, r)
    clean_q = [(cs.lo[0], cs.hi[0]), (cs.lo[1], cs.hi[1])] if cq else []
    shards = []
    for s in range(P):
        k = B.bdattn_clean_shard(L, P, s)
        shards.append([(k.lo[0], k.hi[0]), (k.lo[1], k.hi[1])])
    t = csbp_inputs(9500 + i, L, M, hq, hkv, d, blocks, clean_q, device=dev)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, shards, window=W)
    ins = (t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"])
    o32, lse, _ = sh.fwd(*ins)
    dq, dkc, dvc, dkx, dvx, _ = sh.bwd(*ins, o32, lse, t["do"])
    torch.cuda.synchronize()
    qh, kh, vh, doh, pos = doubled_host(L, hq, hkv, d, t, blocks, clean_q, M)
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True, window=W)
    owned = orc.share(L, M, clean=clean_q, blocks=blocks)
    o_ref, lse_ref = orc.fwd(p, orc.keys(), qh, kh, vh)
    dq_ref, dk_ref, dv_ref = orc.bwd(p, owned, orc.keys(), orc.keys(), qh, kh, vh, doh)
    assert np.array_equal(pos, share_positions(L, M, blocks, clean_q))
    assert max_abs(o32[0].cpu().numpy(), o_ref[0, pos]) <= TOL_O
    assert max_abs(lse[0].cpu().numpy(), lse_ref[0, pos]) <= TOL_LSE
    assert rel_l2(dq[0].cpu().numpy(), dq_ref[0, pos]) <= TOL_GRAD
    n_clean = sum(hi - lo for lo, hi in clean_q)
    kx = pos[n_clean:]  # the share's corrupted positions, packed order
    assert rel_l2(dkc[0].cpu().numpy(), dk_ref[0, :L]) <= TOL_GRAD
    assert rel_l2(dvc[0].cpu().numpy(), dv_ref[0, :L]) <= TOL_GRAD
    assert rel_l2(dkx[0].cpu().numpy(), dk_ref[0, kx]) <= TOL_GRAD
    assert rel_l2(dvx[0].cpu().numpy(), dv_ref[0, kx]) <= TOL_GRAD


@pytest.mark.parametrize("i", range(12))
def test_random_whole_mask_overwrite(dev, orc, i):
    """The whole-mask backward with BDATTN_BWD_OVERWRITE on gradients
    pre-filled with NaN: every element must be written (an element left
    alone stays NaN and fails), and the values must match the oracle."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    batch, L, M, hq, hkv, d, tc, W = _case(i)
    print(f"\n[overwrite case {i}] batch={batch} L={L} M={M} hq={hq} hkv={hkv} d={d} token_causal={tc} window={W}",
          flush=True)
    q, k, v, do = doubled_inputs(8000 + i, batch, L, hq, hkv, d, device=dev)
    wm = WholeMask(batch, L, M, hq, hkv, d, B.BDATTN_BF16,
                   B.BDATTN_CLEAN_TOKEN_CAUSAL if tc else B.BDATTN_CLEAN_BLOCK_CAUSAL, window=W)
    o, lse = wm.fwd(q, k, v, o_dtype=torch.float32)
    grads = wm.alloc_grads(dev)
    for g_ in grads[:5]:
        g_.fill_(float("nan"))
    dq, dk, dv = wm.bwd(q, k, v, o, lse, do, grads=grads, overwrite=True)
    torch.cuda.synchronize()
    assert not torch.isnan(dq).any() and not torch.isnan(dk).any() and not torch.isnan(dv).any()
    p = orc.problem(batch, L, M, hq, hkv, d, token_causal=tc, bf16=True, window=W)
    hq_, hk_, hv_, hdo = (host_bits(x) for x in (q, k, v, do))
    dq_ref, dk_ref, dv_ref = orc.bwd(p, orc.share(), orc.keys(), orc.keys(), hq_, hk_, hv_, hdo)
    assert rel_l2(dq.cpu().numpy(), dq_ref) <= TOL_GRAD
    assert rel_l2(dk.cpu().numpy(), dk_ref) <= TOL_GRAD
    assert rel_l2(dv.cpu().numpy(), dv_ref) <= TOL_GRAD
