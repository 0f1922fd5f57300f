"""The five benchmark workloads at full size, in the launch configuration the
benchmark uses, checked against the oracle on sampled outputs the oracle can
compute one at a time, and on identities that hold at any size.

 1. fp32 forward, L=1024, M=16, 4 heads MHA, d=64: every output (oracle full).
 2. bf16 fwd+bwd, L=8192, M=32, batch 2, 16/8 heads, d=128, inputs /sqrt(d).
 3. bf16 fwd+bwd, L=65536, M=32, 40/8 heads, d=128 (the headline workload).
 4. CSBP share, L=262144, P=8, rank 0 (1024 dual-end blocks), 32/8 heads,
    8 zigzag clean shards of 32768 tokens merged by LSE.
 5. CSBP share, L=524288, M=16, P=16, rank 0 (2048 blocks + its 32768-token
    clean shard of query rows), 32/4 heads, 1% of rows x8 (outlier logits).
 3w. workload 3 under a 1,024-token clean-key sliding window.

Sampled checks: O and LSE of random query rows; dQ of random query rows;
dK/dV of corrupted keys anywhere and of clean keys in the last blocks (few
rows see them, so the oracle can afford it).  Identities (any size): per KV
head, sum_j dV_j = sum over the group's share rows of dO_i; sum_j dK_j = 0;
sum_i q_i.dQ_i = sum_j k_j.dK_j.
Bar: fp32 O/LSE max|err| <= 1e-4; bf16 O <= 2e-2, LSE <= 1e-3,
gradients rel-L2 <= 1e-2 (the identities: relative 1e-2 of the summed norm).
"""
import numpy as np
import pytest
import torch

from tests.common import (TOL_F32, TOL_GRAD, TOL_LSE, TOL_O, csbp_inputs, doubled_host, doubled_inputs,
                          host_bits, max_abs, rel_l2, share_positions)

pytestmark = pytest.mark.gpu

SEED0 = 0x5EED0000


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdattn
    bdattn.lib()
    return torch.device("cuda:0")


def _identities(dq, dk, dv, q, k, v, do, G, hkv):
    """dq, q, do: [rows, hq, d] (share rows); dk, k, dv, v: [keys, hkv, d] (every key of the share)."""
    dq, dk, dv = (np.asarray(x, dtype=np.float64) for x in (dq, dk, dv))
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    for g in range(hkv):
        hs = slice(g * G, (g + 1) * G)
        sdv = dv[:, g].sum(0)
        sdo = do[:, hs].sum((0, 1))
        assert np.linalg.norm(sdv - sdo) <= 1e-2 * max(1.0, np.linalg.norm(sdo)), g
        sdk = dk[:, g].sum(0)
        assert np.linalg.norm(sdk) <= 1e-2 * max(1.0, np.abs(dk[:, g]).sum(0).max()), g
        qa = (q[:, hs] * dq[:, hs]).sum(-1)
        kb = (k[:, g] * dk[:, g]).sum(-1)
        a, b = float(qa.sum()), float(kb.sum())
        scale = max(1.0, float(np.abs(qa).sum()), float(np.abs(kb).sum()))
        assert abs(a - b) <= 1e-2 * scale, (g, a, b, scale)


def _whole(dev, orc, batch, L, M, hq, hkv, d, std, seed, n_rows=96, window=0):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    print(f"\n[config] whole mask batch={batch} L={L} M={M} hq={hq} hkv={hkv} d={d} window={window}", flush=True)
    q, k, v, do = doubled_inputs(seed, batch, L, hq, hkv, d, std=std, device=dev)
    wm = WholeMask(batch, L, M, hq, hkv, d, B.BDATTN_BF16, window=window)
    o, lse = wm.fwd(q, k, v, o_dtype=torch.bfloat16)
    dq, dk, dv = wm.bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    G = hq // hkv
    hq_, hk_, hv_, hdo = (host_bits(x) for x in (q, k, v, do))
    p = orc.problem(batch, L, M, hq, hkv, d, bf16=True, window=window)
    rng = np.random.default_rng(seed)
    b = rng.integers(0, batch, n_rows)
    h = rng.integers(0, hq, n_rows)
    i = np.concatenate([rng.integers(0, 2 * L, n_rows - 4), [0, L - 1, L, 2 * L - 1]])
    rdq, ro, rl = orc.dq_rows(p, orc.keys(), orc.keys(), hq_, hk_, hv_, hdo, b, h, i)
    assert max_abs(o[b, i, h].float().cpu().numpy(), ro) <= TOL_O
    assert max_abs(lse[b, i, h].cpu().numpy(), rl) <= TOL_LSE
    assert rel_l2(dq[b, i, h].cpu().numpy(), rdq) <= TOL_GRAD
    # keys: corrupted anywhere; clean in the last three blocks (few rows see
    # them), or anywhere when a window bounds the rows that see each key
    nk = 24
    kb = rng.integers(0, batch, nk)
    kg = rng.integers(0, hkv, nk)
    lo = 0 if window > 0 else L - 3 * M
    kj = np.concatenate([L + rng.integers(0, L, nk // 2), rng.integers(lo, L, nk - nk // 2)])
    rdk, rdv = orc.dkdv_rows(p, orc.share(), orc.keys(), orc.keys(), hq_, hk_, hv_, hdo, kb, kg, kj)
    assert rel_l2(dk[kb, kj, kg].cpu().numpy(), rdk) <= TOL_GRAD
    assert rel_l2(dv[kb, kj, kg].cpu().numpy(), rdv) <= TOL_GRAD
    for bb in range(batch):
        _identities(dq[bb].cpu().numpy(), dk[bb].cpu().numpy(), dv[bb].cpu().numpy(), q[bb].float().cpu().numpy(),
                    k[bb].float().cpu().numpy(), v[bb].float().cpu().numpy(), do[bb].float().cpu().numpy(), G, hkv)


def test_config1_fp32_forward(dev, orc):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    batch, L, M, hq, hkv, d = 1, 1024, 16, 4, 4, 64
    print(f"\n[config] fp32 forward L={L} M={M} heads={hq} d={d}", flush=True)
    q, k, v, _ = doubled_inputs(SEED0 + 0, batch, L, hq, hkv, d, dtype=torch.float32, device=dev)
    wm = WholeMask(batch, L, M, hq, hkv, d, B.BDATTN_F32)
    o, lse = wm.fwd(q, k, v)
    torch.cuda.synchronize()
    p = orc.problem(batch, L, M, hq, hkv, d)
    ro, rl = orc.fwd(p, orc.keys(), *(host_bits(x) for x in (q, k, v)))
    assert max_abs(o.cpu().numpy(), ro) <= TOL_F32
    assert max_abs(lse.cpu().numpy(), rl) <= TOL_F32


def test_config2_bf16_L8K(dev, orc):
    _whole(dev, orc, 2, 8192, 32, 16, 8, 128, std=128 ** -0.5, seed=SEED0 + 1)


def test_config3_bf16_L64K(dev, orc):
    _whole(dev, orc, 1, 65536, 32, 40, 8, 128, std=1.0, seed=SEED0 + 2, n_rows=64)


def test_config3_window1024(dev, orc):
    """The headline workload under a 1,024-token clean-key sliding window
    (the pages' hybrid models attend through such a window in most layers)."""
    _whole(dev, orc, 1, 65536, 32, 40, 8, 128, std=1.0, seed=SEED0 + 12, n_rows=64, window=1024)


def _csbp(dev, orc, L, M, hq, hkv, d, P, r, clean_queries, seed, outlier_frac=0.0, n_rows=64):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    blocks = B.bdattn_assign_blocks(L // M, P, r).tolist()
    ref_blocks = orc.assign_blocks(L // M, P, r).tolist()
    assert blocks == ref_blocks  # bit-exact block assignment
    cs = B.bdattn_clean_shard(L, P, r)
    assert [(cs.lo[0], cs.hi[0]), (cs.lo[1], cs.hi[1])] == orc.clean_shard(L, P, r)
    clean_q = [(cs.lo[0], cs.hi[0]), (cs.lo[1], cs.hi[1])] if clean_queries else []
    shards = []
    for s in range(P):
        kk = B.bdattn_clean_shard(L, P, s)
        shards.append([(kk.lo[0], kk.hi[0]), (kk.lo[1], kk.hi[1])])
    print(f"\n[config] CSBP share L={L} M={M} P={P} r={r} blocks={len(blocks)} clean_q={clean_q} "
          f"hq={hq} hkv={hkv}", flush=True)
    t = csbp_inputs(seed, L, M, hq, hkv, d, blocks, clean_q, device=dev, outlier_frac=outlier_frac)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, shards)
    o32, lse, obf = sh.fwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"])
    dq, dkc, dvc, dkx, dvx, _ = sh.bwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"],
                                       t["v_corr"], o32, lse, t["do"])
    torch.cuda.synchronize()
    qh, kh, vh, doh, pos = doubled_host(L, hq, hkv, d, t, blocks, clean_q, M)
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True)
    owned = orc.share(L, M, clean=clean_q, blocks=blocks)
    rng = np.random.default_rng(seed)
    R = len(pos)
    rows = np.concatenate([rng.integers(0, R, n_rows - 2), [0, R - 1]])
    h = rng.integers(0, hq, n_rows)
    rdq, ro, rl = orc.dq_rows(p, orc.keys(), orc.keys(), qh, kh, vh, doh, np.zeros(n_rows, np.int32), h, pos[rows])
    assert max_abs(o32[0, rows, h].cpu().numpy(), ro) <= TOL_O
    assert max_abs(lse[0, rows, h].cpu().numpy(), rl) <= TOL_LSE
    assert max_abs(obf[0, rows, h].float().cpu().numpy(), ro) <= TOL_O + np.abs(ro).max() * 2.0 ** -9
    assert rel_l2(dq[0, rows, h].cpu().numpy(), rdq) <= TOL_GRAD
    # corrupted keys of owned blocks, clean keys near the end (seen by the late blocks only)
    n_clean = sum(hi - lo for lo, hi in clean_q)
    nk = 16
    kx = rng.integers(0, len(blocks) * M, nk)
    kc = rng.integers(L - 2 * M, L, nk)
    kg = rng.integers(0, hkv, 2 * nk)
    kj = np.concatenate([pos[n_clean + kx], kc])
    rdk, rdv = orc.dkdv_rows(p, owned, orc.keys(), orc.keys(), qh, kh, vh, doh, np.zeros(2 * nk, np.int32), kg, kj)
    gdk = np.concatenate([dkx[0, kx, kg[:nk]].cpu().numpy(), dkc[0, kc, kg[nk:]].cpu().numpy()])
    gdv = np.concatenate([dvx[0, kx, kg[:nk]].cpu().numpy(), dvc[0, kc, kg[nk:]].cpu().numpy()])
    assert rel_l2(gdk, rdk) <= TOL_GRAD
    assert rel_l2(gdv, rdv) <= TOL_GRAD
    # identities over the share: every key the share sees
    qf = torch.cat([t["q_clean"][0], t["q_corr"][0]]).float().cpu().numpy()
    kf = torch.cat([t["k_clean"][0], t["k_corr"][0]]).float().cpu().numpy()
    vf = torch.cat([t["v_clean"][0], t["v_corr"][0]]).float().cpu().numpy()
    dkf = torch.cat([dkc[0], dkx[0]]).cpu().numpy()
    dvf = torch.cat([dvc[0], dvx[0]]).cpu().numpy()
    _identities(dq[0].cpu().numpy(), dkf, dvf, qf, kf, vf, t["do"][0].float().cpu().numpy(), hq // hkv, hkv)


def test_config4_csbp_L256K(dev, orc):
    _csbp(dev, orc, 262144, 32, 32, 8, 128, P=8, r=0, clean_queries=False, seed=SEED0 + 3)


def test_config5_csbp_L512K_outliers(dev, orc):
    _csbp(dev, orc, 524288, 16, 32, 4, 128, P=16, r=0, clean_queries=True, seed=SEED0 + 4, outlier_frac=0.01)
