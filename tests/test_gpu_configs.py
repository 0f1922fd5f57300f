"""The five benchmark workloads at full size, in the launch configuration the
benchmark uses, checked against the oracle on sampled outputs the oracle can
compute one at a time, on stored oracle gradients of key rows across the
whole sequence, and on identities that hold at any size.

 1. fp32 forward, L=1024, M=16, 4 heads MHA, d=64: every output (oracle full).
 2. bf16 fwd+bwd, L=8192, M=32, batch 2, 16/8 heads, d=128, inputs /sqrt(d).
 3. bf16 fwd+bwd, L=65536, M=32, 40/8 heads, d=128 (the headline workload).
 4. CSBP share, L=262144, P=8, rank 0 (1024 dual-end blocks), 32/8 heads,
    8 zigzag clean shards of 32768 tokens merged by LSE.
 5. CSBP share, L=524288, M=16, P=16, rank 0 (2048 blocks + its 32768-token
    clean shard of query rows), 32/4 heads, 1% of rows x8 (outlier logits).
 3w. workload 3 under a 1,024-token clean-key sliding window.

The whole-mask workloads run the backward the benchmark times: gradients
written, not added (BDATTN_BWD_OVERWRITE), into buffers filled with NaN, so
an element left unwritten fails.

Checks:
 * O and LSE of random query rows; dQ of random query rows (oracle per row).
 * dK/dV of key rows spread over the whole sequence -- the first clean keys,
   seen by every later row, whose gradients are the longest sums -- against
   values stored under tests/golden/ by tests/golden/make_fullsize_keys.py
   (the batched fp64 oracle route, oracle/rowstats.py); inputs are drawn on
   the host so both sides see the same bits, and the stored fingerprints of
   the inputs are compared first.
 * dK/dV of keys near the end and of corrupted keys (oracle per key).
 * Identities at any size: per KV head, sum_j dV_j = sum over the group's
   share rows of dO_i; sum_j dK_j = 0; sum_i q_i.dQ_i = sum_j k_j.dK_j.
 * No input lies outside the fp16 range: each call's range flag is clear.
Bar: fp32 O/LSE max|err| <= 1e-4; bf16 O <= 2e-2, LSE <= 1e-3,
gradients rel-L2 <= 1e-2 (the identities: relative 1e-2 of the summed norm).
Every measured error is printed on an "[errors]" line.
"""
import json
import os

import numpy as np
import pytest
import torch

from tests import workloads as W
from tests.common import TOL_F32, TOL_GRAD, TOL_LSE, TOL_O, doubled_inputs, host_bits, max_abs, rel_l2

pytestmark = pytest.mark.gpu

SEED0 = W.SEED0
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdattn
    bdattn.lib()
    return torch.device("cuda:0")


def _report(name, errs):
    print(f"[errors] {name} " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


def _golden(name, host, b):
    """Stored oracle dK/dV of `name`, after checking the input fingerprints."""
    path = os.path.join(GOLDEN, f"fullsize_keys_{name}.npz")
    z = np.load(path, allow_pickle=False)
    qh, kh, _, doh = host
    keys, g = z["keys"], int(z["g"])
    assert int(z["b"]) == b
    fr = z["fp_rows"]
    assert np.array_equal(z["fp_k"], kh[b, keys, g]), "inputs differ from the stored values' inputs (K)"
    assert np.array_equal(z["fp_q"], qh[b, fr]), "inputs differ from the stored values' inputs (Q)"
    assert np.array_equal(z["fp_do"], doh[b, fr]), "inputs differ from the stored values' inputs (dO)"
    return keys, g, z["dk"], z["dv"], json.loads(str(z["meta"]))


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


def _whole(dev, orc, name, n_rows=96, window=0, golden=True):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    w = W.WHOLE[name]
    batch, L, M, hq, hkv, d = (w[x] for x in ("batch", "L", "M", "hq", "hkv", "d"))
    seed = w["seed"] + (10 if window else 0)
    print(f"\n[config] {name} whole mask batch={batch} L={L} M={M} hq={hq} hkv={hkv} d={d} window={window}",
          flush=True)
    if window:
        q, k, v, do = doubled_inputs(seed, batch, L, hq, hkv, d, std=w["std"], device="cpu")
        host = tuple(host_bits(x) for x in (q, k, v, do))
    else:
        (q, k, v, do), host = W.whole_host(w)
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    wm = WholeMask(batch, L, M, hq, hkv, d, B.BDATTN_BF16, window=window)
    wsf, wsb = wm.workspace(False, dev), wm.workspace(True, dev)
    o, lse = wm.fwd(q, k, v, o_dtype=torch.bfloat16, ws=wsf)
    assert B.bdattn_workspace_status(wsf) == B.BDATTN_OK
    grads = wm.alloc_grads(dev)
    for g_ in grads[:5]:
        g_.fill_(float("nan"))
    dq, dk, dv = wm.bwd(q, k, v, o, lse, do, ws=wsb, grads=grads, overwrite=True)
    assert B.bdattn_workspace_status(wsb) == B.BDATTN_OK
    torch.cuda.synchronize()
    assert not torch.isnan(dq).any() and not torch.isnan(dk).any() and not torch.isnan(dv).any()
    G = hq // hkv
    hq_, hk_, hv_, hdo = host
    p = orc.problem(batch, L, M, hq, hkv, d, bf16=True, window=window)
    rng = np.random.default_rng(seed)
    b = rng.integers(0, batch, n_rows)
    h = rng.integers(0, hq, n_rows)
    i = np.concatenate([rng.integers(0, 2 * L, n_rows - 4), [0, L - 1, L, 2 * L - 1]])
    rdq, ro, rl = orc.dq_rows(p, orc.keys(), orc.keys(), hq_, hk_, hv_, hdo, b, h, i)
    errs = {"O": max_abs(o[b, i, h].float().cpu().numpy(), ro),
            "LSE": max_abs(lse[b, i, h].cpu().numpy(), rl),
            "dQ": rel_l2(dq[b, i, h].cpu().numpy(), rdq)}
    # keys near the end (few rows see them) and corrupted keys, oracle per
    # key; with a window, clean keys anywhere (the window bounds their rows)
    nk = 24
    kb = rng.integers(0, batch, nk)
    kg = rng.integers(0, hkv, nk)
    lo = 0 if window > 0 else L - 3 * M
    kj = np.concatenate([L + rng.integers(0, L, nk // 2), rng.integers(lo, L, nk - nk // 2)])
    rdk, rdv = orc.dkdv_rows(p, orc.share(), orc.keys(), orc.keys(), hq_, hk_, hv_, hdo, kb, kg, kj)
    errs["dK_late"] = rel_l2(dk[kb, kj, kg].cpu().numpy(), rdk)
    errs["dV_late"] = rel_l2(dv[kb, kj, kg].cpu().numpy(), rdv)
    if golden:
        keys, g, gdk, gdv, _ = _golden(name, host, w["b"])
        errs["dK_seq"] = rel_l2(dk[w["b"], keys, g].cpu().numpy(), gdk)
        errs["dV_seq"] = rel_l2(dv[w["b"], keys, g].cpu().numpy(), gdv)
        early = keys < 4 * M  # the first clean keys: the longest sums
        errs["dK_first"] = rel_l2(dk[w["b"], keys[early], g].cpu().numpy(), gdk[early])
        errs["dV_first"] = rel_l2(dv[w["b"], keys[early], g].cpu().numpy(), gdv[early])
    _report(name + ("_window%d" % window if window else ""), errs)
    assert errs["O"] <= TOL_O and errs["LSE"] <= TOL_LSE
    for k_, e in errs.items():
        if k_ not in ("O", "LSE"):
            assert e <= TOL_GRAD, (k_, e)
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
    errs = {"O": max_abs(o.cpu().numpy(), ro), "LSE": max_abs(lse.cpu().numpy(), rl)}
    _report("bdlm_L1K_M16_h4_d64_fp32", errs)
    assert errs["O"] <= TOL_F32
    assert errs["LSE"] <= TOL_F32


def test_config2_bf16_L8K(dev, orc):
    _whole(dev, orc, "bdlm_L8K_M32_b2_h16kv8_d128")


def test_config3_bf16_L64K(dev, orc):
    _whole(dev, orc, "bdlm_L64K_M32_h40kv8_d128", n_rows=64)


def test_config3_window1024(dev, orc):
    """The headline workload under a 1,024-token clean-key sliding window
    (the pages' hybrid models attend through such a window in most layers)."""
    _whole(dev, orc, "bdlm_L64K_M32_h40kv8_d128", n_rows=64, window=1024, golden=False)


def _csbp(dev, orc, name, n_rows=64):
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    w = W.CSBP[name]
    L, M, hq, hkv, d, P, r = (w[x] for x in ("L", "M", "hq", "hkv", "d", "P", "r"))
    t, host, pos, blocks, clean_q, shards = W.csbp_host(w)
    assert B.bdattn_assign_blocks(L // M, P, r).tolist() == blocks  # bit-exact block assignment
    assert orc.assign_blocks(L // M, P, r).tolist() == blocks
    for s in range(P):
        cs = B.bdattn_clean_shard(L, P, s)
        assert [(cs.lo[0], cs.hi[0]), (cs.lo[1], cs.hi[1])] == shards[s] == orc.clean_shard(L, P, s)
    print(f"\n[config] {name} CSBP share L={L} M={M} P={P} r={r} blocks={len(blocks)} clean_q={clean_q} "
          f"hq={hq} hkv={hkv}", flush=True)
    t = {k_: x.to(dev) for k_, x in t.items()}
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, shards)
    wsf, wsb = sh.workspace(False, dev), sh.workspace(True, dev)
    o32, lse, obf = sh.fwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"],
                           ws=wsf)
    assert B.bdattn_workspace_status(wsf) == B.BDATTN_OK
    dq, dkc, dvc, dkx, dvx, _ = sh.bwd(t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"],
                                       t["v_corr"], o32, lse, t["do"], ws=wsb)
    assert B.bdattn_workspace_status(wsb) == B.BDATTN_OK
    torch.cuda.synchronize()
    qh, kh, vh, doh = host
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True)
    owned = orc.share(L, M, clean=clean_q, blocks=blocks)
    rng = np.random.default_rng(w["seed"])
    R = len(pos)
    rows = np.concatenate([rng.integers(0, R, n_rows - 2), [0, R - 1]])
    h = rng.integers(0, hq, n_rows)
    rdq, ro, rl = orc.dq_rows(p, orc.keys(), orc.keys(), qh, kh, vh, doh, np.zeros(n_rows, np.int32), h, pos[rows])
    errs = {"O": max_abs(o32[0, rows, h].cpu().numpy(), ro),
            "LSE": max_abs(lse[0, rows, h].cpu().numpy(), rl)}
    obf_err = max_abs(obf[0, rows, h].float().cpu().numpy(), ro)
    errs["O_bf16"] = obf_err
    errs["dQ"] = rel_l2(dq[0, rows, h].cpu().numpy(), rdq)
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
    errs["dK_late"] = rel_l2(gdk, rdk)
    errs["dV_late"] = rel_l2(gdv, rdv)
    # stored gradients of keys over the whole sequence (doubled positions:
    # clean keys < L index the clean accumulators, corrupted ones the packed rows)
    keys, g, sdk, sdv, _ = _golden(name, host, 0)
    clean = keys < L
    packed = {int(pp): n for n, pp in enumerate(pos[n_clean:])}
    kx2 = np.asarray([packed[int(j)] for j in keys[~clean]])
    mdk = np.concatenate([dkc[0, keys[clean], g].cpu().numpy(), dkx[0, kx2, g].cpu().numpy()])
    mdv = np.concatenate([dvc[0, keys[clean], g].cpu().numpy(), dvx[0, kx2, g].cpu().numpy()])
    ref_k = np.concatenate([sdk[clean], sdk[~clean]])
    ref_v = np.concatenate([sdv[clean], sdv[~clean]])
    errs["dK_seq"] = rel_l2(mdk, ref_k)
    errs["dV_seq"] = rel_l2(mdv, ref_v)
    first = keys[clean] < 4 * M
    errs["dK_first"] = rel_l2(mdk[: clean.sum()][first], sdk[clean][first])
    errs["dV_first"] = rel_l2(mdv[: clean.sum()][first], sdv[clean][first])
    _report(name, errs)
    assert errs["O"] <= TOL_O and errs["LSE"] <= TOL_LSE
    assert obf_err <= TOL_O + np.abs(ro).max() * 2.0 ** -9
    for k_, e in errs.items():
        if k_ not in ("O", "LSE", "O_bf16"):
            assert e <= TOL_GRAD, (k_, e)
    # identities over the share: every key the share sees
    qf = torch.cat([t["q_clean"][0], t["q_corr"][0]]).float().cpu().numpy()
    kf = torch.cat([t["k_clean"][0], t["k_corr"][0]]).float().cpu().numpy()
    vf = torch.cat([t["v_clean"][0], t["v_corr"][0]]).float().cpu().numpy()
    dkf = torch.cat([dkc[0], dkx[0]]).cpu().numpy()
    dvf = torch.cat([dvc[0], dvx[0]]).cpu().numpy()
    _identities(dq[0].cpu().numpy(), dkf, dvf, qf, kf, vf, t["do"][0].float().cpu().numpy(), hq // hkv, hkv)


def test_config4_csbp_L256K(dev, orc):
    _csbp(dev, orc, "csbp_L256K_P8_r0_h32kv8_d128")


def test_config5_csbp_L512K_outliers(dev, orc):
    _csbp(dev, orc, "csbp_L512K_M16_P16_r0_h32kv4_d128")
