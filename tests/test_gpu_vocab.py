"""GPU parity of the streaming vocabulary loss (libbdvocab) against the fp64
oracle (oracle/vocab.py), through the C ABI.

Bar (the kernel's logits are fp32 from bf16 inputs with fp32 accumulation;
the logit gradient is rounded to bf16 before the gradient GEMM, a relative
error of at most 2^-9 per term):
  lse and per-row loss: max |err| <= 1e-3 (the LSE bar of the attention path);
  loss sum: relative error <= 1e-4;
  dh: relative L2 error <= 1e-2 on every row (the gradient bar);
  dW (head gradient, fp32 accumulation of bf16 products): relative L2
  error <= 1e-2 over the whole [V, d] matrix.
Rows outside the row list keep their contents; ignored targets give loss 0
and dh 0.
"""
import numpy as np
import pytest
import torch

from oracle import vocab as ov
from tests.common import TOL_GRAD, TOL_LSE, max_abs, rel_l2

pytestmark = pytest.mark.gpu

TOL_SUM = 1e-4
SENTINEL = 7.0


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdvocab
    bdvocab.lib()
    return torch.device("cuda:0")


def _host(t):
    return t.detach().float().cpu().numpy()


def _run(dev, seed, T, R, V, d, chunk, row_list, dh_dtype, weighted=True, ignored=(), head_std=None, head_grad=True,
         dw_repeat=1, with_dh=True, tuned=False):
    from block_diffusion_lm_bdlm_amd import bdvocab as BV
    from block_diffusion_lm_bdlm_amd import synth
    print(f"\n[vocab] seed={seed} T={T} R={R} V={V} d={d} chunk={chunk} rows={row_list} dh={dh_dtype}", flush=True)
    if row_list:
        g = torch.Generator().manual_seed(seed)
        rows = torch.sort(torch.randperm(T, generator=g)[:R]).values.to(torch.int32)
    else:
        rows = None
    h, W, y, wt = synth.vocab_inputs(seed, T, d, V, R=R, device=dev, head_std=head_std)
    if weighted:
        g = torch.Generator().manual_seed(seed + 1)
        wt = (0.1 + 1.9 * torch.rand(R, generator=g)).to(dev)
    for i, val in ignored:
        y[i] = val
    vl = BV.VocabLoss(R, V, d, chunk=chunk, dh_dtype=dh_dtype, row_list=row_list, head_grad=head_grad, device=dev)
    out_dt = torch.float32 if dh_dtype == BV.BDVOCAB_F32 else torch.bfloat16
    dh = torch.full((T, d), SENTINEL, dtype=out_dt, device=dev)
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    loss_sum = torch.empty(1, dtype=torch.float32, device=dev)
    rows_dev = None if rows is None else rows.to(dev)
    dw = torch.zeros((V, d), dtype=torch.float32, device=dev) if head_grad else None
    if tuned:  # set-up call: must not touch dh, dw or the loss outputs
        vl.tune(h, W, dh_stride=dh.stride(0) if with_dh else 0)
    for _ in range(dw_repeat):
        loss, _, _, _ = vl(h, W, y, weights=wt, rows=rows_dev, dh=dh if with_dh else None, lse=lse,
                           loss_sum=loss_sum, dw=dw)
    torch.cuda.synchronize()
    idx = np.arange(R) if rows is None else rows.numpy()
    hh, Wh, yh, wh = _host(h), _host(W), y.cpu().numpy(), wt.cpu().numpy()
    lse_ref, loss_ref, dh_ref = ov.vocab_loss_rows(hh, Wh, idx, yh, wh)
    out = dict(lse=_host(lse), loss=_host(loss), sum=float(loss_sum.item()), dh=_host(dh), idx=idx,
               lse_ref=lse_ref, loss_ref=loss_ref, dh_ref=dh_ref, T=T, with_dh=with_dh)
    if head_grad:
        out["dw"] = _host(dw)
        out["dw_ref"] = dw_repeat * ov.vocab_head_grad(hh[idx], Wh, yh, wh)
    return out


def _check(res):
    assert max_abs(res["lse"], res["lse_ref"]) <= TOL_LSE
    assert max_abs(res["loss"], res["loss_ref"]) <= TOL_LSE
    ref_sum = float(res["loss_ref"].sum())
    assert abs(res["sum"] - ref_sum) <= TOL_SUM * max(1.0, abs(ref_sum))
    if "dw" in res:
        assert rel_l2(res["dw"], res["dw_ref"]) <= TOL_GRAD
    if not res["with_dh"]:
        assert np.all(res["dh"] == SENTINEL)
        return
    dh = res["dh"][res["idx"]]
    for r in range(len(res["idx"])):
        if np.any(res["dh_ref"][r]):
            assert rel_l2(dh[r], res["dh_ref"][r]) <= TOL_GRAD, r
        else:
            assert not np.any(dh[r]), r
    untouched = np.setdiff1d(np.arange(res["T"]), res["idx"])
    assert np.all(res["dh"][untouched] == SENTINEL)


# (seed, T, R, V, d, chunk, row_list, dh_dtype): several chunks with a ragged
# last one, vocabularies that are not multiples of the row pitch, of 4, or
# smaller than one workgroup's loads, both dh dtypes, and every storage
# split of the single-read row kernel (1-4 register sub-blocks, 1-4 LDS
# sub-blocks) plus the two-pass kernel above 131,072 logits.
CASES = [
    (1, 300, 300, 5000, 256, 128, False, 0),
    (2, 700, 257, 1001, 64, 64, True, 1),
    (3, 64, 64, 4096, 512, 0, False, 1),
    (4, 1, 1, 7, 8, 0, False, 0),
    (5, 400, 100, 32771, 128, 37, True, 0),
    (6, 96, 96, 70000, 80, 40, False, 0),
    (7, 33, 33, 3, 16, 8, True, 1),
    (8, 48, 48, 140000, 64, 16, False, 0),   # above the single-read capacity: the two-pass kernel
    (9, 64, 40, 131072, 64, 0, True, 1),     # the largest single-read row (register + LDS storage)
]


@pytest.mark.parametrize("tuned", [False, True], ids=["untuned", "tuned"])
@pytest.mark.parametrize("case", CASES, ids=[f"R{c[2]}_V{c[3]}_d{c[4]}_C{c[5]}_{'rows' if c[6] else 'dense'}"
                                             for c in CASES])
def test_vocab_parity(dev, case, tuned):
    """With and without bdvocab_tune first (the GEMMs then run the timed
    algorithms of every shape, the head gradient GEMM included)."""
    seed, T, R, V, d, chunk, row_list, dt = case
    _check(_run(dev, seed, T, R, V, d, chunk, row_list, dt, tuned=tuned))


def test_vocab_ignored_targets_and_unit_weights(dev):
    res = _run(dev, 11, 150, 150, 3000, 128, 64, False, 0, weighted=False, ignored=[(0, -1), (5, 3000), (149, -100)])
    _check(res)
    assert res["loss"][0] == 0 and res["loss"][5] == 0 and res["loss"][149] == 0


def test_vocab_large_logits(dev):
    # logits with std ~30: the lse is far above most terms and the softmax
    # is nearly one-hot
    _check(_run(dev, 12, 128, 128, 20000, 256, 0, False, 0, head_std=30.0 / 16.0))


def test_vocab_head_grad_accumulates_and_alone(dev):
    # two calls add twice the gradient; a call with dW but no dh leaves dh alone
    _check(_run(dev, 14, 300, 150, 2500, 64, 64, True, 0, dw_repeat=2))
    _check(_run(dev, 15, 90, 90, 3001, 128, 32, False, 1, with_dh=False))


def test_vocab_head_grad_full_vocabulary(dev):
    # the benchmark's vocabulary (131,072) with a narrower hidden size so the
    # fp64 oracle of the whole [V, d] gradient stays small; ragged chunks
    _check(_run(dev, 16, 500, 96, 131072, 1024, 40, True, 0))


def test_vocab_zero_rows(dev):
    from block_diffusion_lm_bdlm_amd import bdvocab as BV
    s = torch.full((1,), 5.0, device=dev)
    BV.bdvocab_loss(BV.problem(0, 100, 64), None, 64, None, None, None, None, None, None, s, None, 0, None, None)
    torch.cuda.synchronize()
    assert s.item() == 0.0


def test_vocab_repeat_calls_reuse_workspace(dev):
    # two calls on one workspace: the second sees none of the first's state
    a = _run(dev, 13, 200, 200, 4000, 64, 64, False, 1)
    b = _run(dev, 13, 200, 200, 4000, 64, 64, False, 1)
    _check(a)
    np.testing.assert_array_equal(a["loss"], b["loss"])
    np.testing.assert_array_equal(a["dh"], b["dh"])


def test_vocab_full_size_sampled(dev):
    """The benchmark's workload: 65,536 corrupted positions, the masked ones
    (per-block ratio t ~ U(0, 1)) carry the loss; hidden 5,120, vocabulary
    131,072, default chunk.  Sampled rows against the oracle one by one;
    every row finite and the sum consistent."""
    from block_diffusion_lm_bdlm_amd import bdvocab as BV
    from block_diffusion_lm_bdlm_amd import synth
    L, M, d, V = 65536, 32, 5120, 131072
    rows = synth.masked_rows(77, L, M)
    R = int(rows.numel())
    print(f"\n[vocab full] L={L} R={R} V={V} d={d}", flush=True)
    h, W, y, wt = synth.vocab_inputs(77, L, d, V, R=R, device=dev)
    vl = BV.VocabLoss(R, V, d, row_list=True, device=dev)
    dh = torch.full((L, d), SENTINEL, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    loss_sum = torch.empty(1, dtype=torch.float32, device=dev)
    loss, _, _, _ = vl(h, W, y, weights=wt, rows=rows.to(dev), dh=dh, lse=lse, loss_sum=loss_sum)
    torch.cuda.synchronize()
    assert torch.isfinite(loss).all() and torch.isfinite(lse).all()
    assert abs(loss_sum.item() - loss.double().sum().item()) <= 1e-5 * abs(loss_sum.item())
    pick = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(5).integers(0, R, 6)]))
    Wh = _host(W)
    idx = rows.numpy()[pick]
    lse_ref, loss_ref, dh_ref = ov.vocab_loss_rows(_host(h[rows.to(dev)[pick].long()]), Wh, np.arange(len(pick)),
                                                   y.cpu().numpy()[pick], wt.cpu().numpy()[pick])
    assert max_abs(_host(lse)[pick], lse_ref) <= TOL_LSE
    assert max_abs(_host(loss)[pick], loss_ref) <= TOL_LSE
    got = _host(dh[torch.as_tensor(idx, device=dev).long()])
    for r in range(len(pick)):
        assert rel_l2(got[r], dh_ref[r]) <= TOL_GRAD, r
    # a few positions that carry no loss are untouched
    free = np.setdiff1d(np.arange(0, L, 997), rows.numpy())[:8]
    assert torch.all(dh[torch.as_tensor(free, device=dev).long()] == SENTINEL)


def test_vocab_head_grad_vocabulary_past_transpose_grid(dev):
    """A vocabulary of more than 65535 column tiles of 64 (V > 4,194,240):
    the chunk's gradient transpose for the head GEMM strides its column
    tiles over the capped grid, so the head gradient covers every row of the
    vocabulary."""
    V = 65535 * 64 + 3 * 64 + 5
    _check(_run(dev, 41, 12, 6, V, 8, 4, True, 0, head_grad=True))
