"""GPU edge cases of the boundary: a call whose key set is empty, a call
with only the share's own corrupted keys (the local block-diagonal part),
a share made of clean query rows only, and the row term D that the
backward forms.  Each is checked against the oracle on the same rows, a
float64 row sum, or the documented identity of an empty call (O = 0,
LSE = -inf, gradient accumulators left untouched)."""
import numpy as np
import pytest
import torch

from tests.common import TOL_GRAD, TOL_LSE, TOL_O, csbp_inputs, doubled_host, max_abs, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdattn
    bdattn.lib()
    return torch.device("cuda:0")


def _ins(t):
    return t["q_clean"], t["q_corr"], t["k_clean"], t["v_clean"], t["k_corr"], t["v_corr"]


def test_empty_key_set(dev):
    """No clean range and no local keys: every row gets O = 0 and LSE = -inf,
    and the backward adds nothing to any accumulator."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    L, M, hq, hkv, d = 256, 16, 4, 2, 128
    blocks, clean_q = [1, 5, 14], [(32, 96)]
    t = csbp_inputs(400, L, M, hq, hkv, d, blocks, clean_q, device=dev)
    full = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, [[(0, L)]])
    o32, lse_f, _ = full.fwd(*_ins(t))
    empty = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, [[]])
    kv = empty.kv_shards[0]
    ws = empty.workspace(True, dev)
    o = torch.full((1, empty.R, hq, d), 7.0, dtype=torch.float32, device=dev)
    lse = torch.full((1, empty.R, hq), 7.0, dtype=torch.float32, device=dev)
    B.bdattn_fwd(empty.prob, empty.share, kv, *_ins(t), o, B.BDATTN_F32, lse, ws)
    grads = empty.alloc_grads(dev)
    for g in grads[:5]:
        g.fill_(3.0)
    dq, dkc, dvc, dkx, dvx, delta = grads
    B.bdattn_bwd(empty.prob, empty.share, kv, *_ins(t), o32, B.BDATTN_F32, lse_f, t["do"], delta, 0,
                 dq, dkc, dvc, dkx, dvx, ws)
    torch.cuda.synchronize()
    assert (o == 0).all() and torch.isneginf(lse).all()
    for g in grads[:5]:
        assert (g == 3.0).all()
    assert torch.isfinite(delta).all()  # D is still computed for later calls


@pytest.mark.parametrize("L,M,hq,hkv,d,blocks", [(256, 16, 4, 2, 128, [0, 3, 9, 15]), (384, 32, 2, 1, 64, [2, 11])])
def test_local_only_call(dev, orc, L, M, hq, hkv, d, blocks):
    """Only the share's own corrupted keys: the block-diagonal part alone
    ('CSBP 完全拆解', the local attention that runs before any clean shard)."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    t = csbp_inputs(410 + L, L, M, hq, hkv, d, blocks, [], device=dev)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, [], [])
    ws = sh.workspace(True, dev)
    o = torch.empty(1, sh.R, hq, d, dtype=torch.float32, device=dev)
    lse = torch.empty(1, sh.R, hq, dtype=torch.float32, device=dev)
    B.bdattn_fwd(sh.prob, sh.share, sh.kv_local, *_ins(t), o, B.BDATTN_F32, lse, ws)
    grads = sh.alloc_grads(dev)
    dq, dkc, dvc, dkx, dvx, delta = grads
    B.bdattn_bwd(sh.prob, sh.share, sh.kv_local, *_ins(t), o, B.BDATTN_F32, lse, t["do"], delta, 0,
                 dq, dkc, dvc, dkx, dvx, ws)
    torch.cuda.synchronize()
    q, k, v, do, pos = doubled_host(L, hq, hkv, d, t, blocks, [], M)
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True)
    local = orc.keys([], local=True)
    o_ref, lse_ref = orc.fwd(p, local, q, k, v)
    assert max_abs(o.cpu().numpy()[0], o_ref[0, pos]) <= TOL_O
    assert max_abs(lse.cpu().numpy()[0], lse_ref[0, pos]) <= TOL_LSE
    sh_o = orc.share(L, M, blocks=blocks)
    dq_ref, dk_ref, dv_ref = orc.bwd(p, sh_o, local, local, q, k, v, do)
    assert rel_l2(dq.cpu().numpy()[0], dq_ref[0, pos]) <= TOL_GRAD
    assert rel_l2(dkx.cpu().numpy()[0], dk_ref[0, pos]) <= TOL_GRAD
    assert rel_l2(dvx.cpu().numpy()[0], dv_ref[0, pos]) <= TOL_GRAD
    assert (dkc == 0).all() and (dvc == 0).all()  # no clean key in the call


def test_clean_rows_only_share(dev, orc):
    """A share of clean query rows only (two ranges, no blocks) against two
    zigzag clean shards merged by LSE."""
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare
    L, M, hq, hkv, d = 512, 16, 4, 2, 128
    clean_q = [(64, 160), (400, 512)]
    shards = [[(0, 64), (448, 512)], [(64, 448)]]
    t = csbp_inputs(420, L, M, hq, hkv, d, [], clean_q, device=dev)
    sh = CsbpShare(1, L, M, hq, hkv, d, [], clean_q, shards)
    o32, lse, _ = sh.fwd(*_ins(t))
    dq, dkc, dvc, _, _, _ = sh.bwd(*_ins(t), o32, lse, t["do"])
    torch.cuda.synchronize()
    q, k, v, do, pos = doubled_host(L, hq, hkv, d, t, [], clean_q, M)
    p = orc.problem(1, L, M, hq, hkv, d, bf16=True)
    o_ref, lse_ref = orc.fwd(p, orc.keys(), q, k, v)
    assert max_abs(o32.cpu().numpy()[0], o_ref[0, pos]) <= TOL_O
    assert max_abs(lse.cpu().numpy()[0], lse_ref[0, pos]) <= TOL_LSE
    sh_o = orc.share(L, M, clean=clean_q)
    dq_ref, dk_ref, dv_ref = orc.bwd(p, sh_o, orc.keys(), orc.keys(), q, k, v, do)
    assert rel_l2(dq.cpu().numpy()[0], dq_ref[0, pos]) <= TOL_GRAD
    assert rel_l2(dkc.cpu().numpy()[0], dk_ref[0, :L]) <= TOL_GRAD
    assert rel_l2(dvc.cpu().numpy()[0], dv_ref[0, :L]) <= TOL_GRAD


@pytest.mark.parametrize("d,o_f32", [(128, False), (128, True), (64, False)])
def test_delta_rowsum(dev, d, o_f32):
    """D = rowsum(dO * O), formed while the backward packs dO ("CSBP 完全拆解",
    the softmax row term of the chain rule), equals the float64 row sum of
    the same bf16 dO and O values; a later call with delta_ready reads it
    back and gives the same gradients bit for bit."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    from tests.common import doubled_inputs
    batch, L, M, hq, hkv = 2, 200, 8, 4, 2
    q, k, v, do = doubled_inputs(41, batch, L, hq, hkv, d, device=dev)
    wm = WholeMask(batch, L, M, hq, hkv, d)
    o, lse = wm.fwd(q, k, v, o_dtype=torch.float32 if o_f32 else torch.bfloat16)
    grads = wm.alloc_grads(dev)
    ws = wm.workspace(True, dev)
    ins = (q[:, :L], q[:, L:], k[:, :L], v[:, :L], k[:, L:], v[:, L:])
    dq, dkc, dvc, dkx, dvx, delta = grads
    B.bdattn_bwd(wm.prob, wm.share, wm.kv, *ins, o, B.BDATTN_F32 if o_f32 else B.BDATTN_BF16, lse, do, delta, 0,
                 dq, dkc, dvc, dkx, dvx, ws)
    torch.cuda.synchronize()
    want = (do.double() * o.double()).sum(-1)
    got = delta.double()
    assert torch.allclose(got, want, rtol=1e-5, atol=1e-5 * float(want.abs().max()))
    # the same call with delta given: identical gradients
    first = [g.clone() for g in grads[:5]]
    for g in grads[:5]:
        g.zero_()
    o_bad = torch.full_like(o, float("nan"))  # not read when delta is given
    B.bdattn_bwd(wm.prob, wm.share, wm.kv, *ins, o_bad, B.BDATTN_F32 if o_f32 else B.BDATTN_BF16, lse, do, delta,
                 1, dq, dkc, dvc, dkx, dvx, ws)
    torch.cuda.synchronize()
    for a, b in zip(first, grads[:5]):
        assert torch.equal(a, b)


def test_range_flag(dev, orc):
    """Inputs outside the fp16 range: the call clamps them, raises its range
    flag (bdattn_workspace_status -> BDATTN_ERANGE) and keeps the forward
    finite; the next call on the same workspace with in-range inputs
    clears it.  In-range inputs leave it clear and match the oracle."""
    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd.runner import WholeMask
    from tests.common import doubled_inputs, host_bits
    batch, L, M, hq, hkv, d = 1, 256, 16, 4, 2, 128
    q, k, v, do = doubled_inputs(501, batch, L, hq, hkv, d, device=dev)
    wm = WholeMask(batch, L, M, hq, hkv, d)
    wsf, wsb = wm.workspace(False, dev), wm.workspace(True, dev)
    o, lse = wm.fwd(q, k, v, o_dtype=torch.float32, ws=wsf)
    assert B.bdattn_workspace_status(wsf) == B.BDATTN_OK
    wm.bwd(q, k, v, o, lse, do, ws=wsb)
    assert B.bdattn_workspace_status(wsb) == B.BDATTN_OK
    p = orc.problem(batch, L, M, hq, hkv, d, bf16=True)
    ro, rl = orc.fwd(p, orc.keys(), *(host_bits(x) for x in (q, k, v)))
    assert max_abs(o.cpu().numpy(), ro) <= TOL_O and max_abs(lse.cpu().numpy(), rl) <= TOL_LSE
    print("[range] in-range call: flag clear, O and LSE within tolerance", flush=True)
    # V (converted to fp16 by the forward's packing) out of range
    vb = v.clone()
    vb[0, 3, 1, 7] = 1.0e6
    o2, _ = wm.fwd(q, k, vb, o_dtype=torch.float32, ws=wsf)
    assert B.bdattn_workspace_status(wsf) == B.BDATTN_ERANGE
    assert torch.isfinite(o2).all()
    # K (converted by the backward's packing) out of range
    kb = k.clone()
    kb[0, 5, 0, 3] = -7.0e4
    wm.bwd(q, kb, v, o, lse, do, ws=wsb)
    assert B.bdattn_workspace_status(wsb) == B.BDATTN_ERANGE
    # the flag belongs to the last call on the workspace
    wm.fwd(q, k, v, o_dtype=torch.float32, ws=wsf)
    assert B.bdattn_workspace_status(wsf) == B.BDATTN_OK
    wm.bwd(q, k, v, o, lse, do, ws=wsb)
    assert B.bdattn_workspace_status(wsb) == B.BDATTN_OK
