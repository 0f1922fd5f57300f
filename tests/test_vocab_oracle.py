"""Pins for the vocabulary-loss oracle (oracle/vocab.py), each tied to
something other than the oracle's own formula:

 * closed forms: two classes reduce to the logistic loss; a head whose rows
   are all equal gives loss log V and zero gradient; a head column that is
   constant over the vocabulary gets no gradient; one dominant logit gives
   lse = that logit;
 * torch's float64 cross_entropy and autograd on the CPU (a library routine
   with its own logsumexp and backward);
 * central finite differences of the oracle's own loss;
 * the row-list form equals the dense form on the gathered rows;
 * ignored targets (outside [0, V)) carry no loss and no gradient.
"""
import numpy as np
import pytest
import torch

from oracle import vocab as ov


def _rand(seed, R, d, V, scale=1.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((R, d))
    W = rng.standard_normal((V, d)) * scale / np.sqrt(d)
    y = rng.integers(0, V, R)
    w = rng.uniform(0.1, 2.0, R)
    return h, W, y, w


def test_two_classes_is_logistic_loss():
    h, W, y, w = _rand(1, 9, 7, 2, scale=3.0)
    lse, loss, dh = ov.vocab_loss(h, W, y, w)
    for r in range(9):
        a = h[r] @ W[y[r]]
        b = h[r] @ W[1 - y[r]]
        z = b - a
        assert loss[r] == pytest.approx(w[r] * np.log1p(np.exp(z)), rel=1e-12)
        sig = 1.0 / (1.0 + np.exp(-z))
        np.testing.assert_allclose(dh[r], w[r] * sig * (W[1 - y[r]] - W[y[r]]), rtol=1e-11, atol=1e-13)
        assert lse[r] == pytest.approx(np.logaddexp(a, b), rel=1e-12)


def test_equal_head_rows_give_log_vocab():
    rng = np.random.default_rng(2)
    V, d = 37, 11
    u = rng.standard_normal(d)
    W = np.tile(u, (V, 1))
    h = rng.standard_normal((5, d))
    y = rng.integers(0, V, 5)
    lse, loss, dh = ov.vocab_loss(h, W, y)
    np.testing.assert_allclose(loss, np.log(V), rtol=1e-13)
    np.testing.assert_allclose(lse, h @ u + np.log(V), rtol=1e-12, atol=1e-12)
    assert np.abs(dh).max() < 1e-13


def test_constant_head_column_gets_no_gradient():
    h, W, y, w = _rand(3, 6, 10, 50)
    W[:, 4] = 0.7
    _, _, dh = ov.vocab_loss(h, W, y, w)
    assert np.abs(dh[:, 4]).max() < 1e-13
    assert np.abs(dh[:, 3]).max() > 1e-3


def test_dominant_logit_lse_and_no_overflow():
    # one logit 1000 above the rest: lse equals it to double precision, and
    # nothing overflows although exp(1000) would
    V, d = 20, 4
    W = np.zeros((V, d))
    W[7, 0] = 1.0
    h = np.array([[1000.0, 0, 0, 0], [1000.0, 0, 0, 0]])
    lse, loss, dh = ov.vocab_loss(h, W, [7, 3])
    assert lse[0] == 1000.0 and lse[1] == 1000.0
    assert loss[0] == 0.0 and loss[1] == 1000.0
    assert np.all(np.isfinite(dh))
    # the wrong-target row pushes h toward W[3] - W[7]
    np.testing.assert_allclose(dh[1], W[7] - W[3], atol=1e-300)


@pytest.mark.parametrize("R,d,V,scale", [(13, 24, 300, 3.0), (4, 64, 1000, 10.0), (1, 5, 3, 1.0)])
def test_matches_torch_cross_entropy_and_autograd(R, d, V, scale):
    h, W, y, w = _rand(10 + R, R, d, V, scale)
    lse, loss, dh = ov.vocab_loss(h, W, y, w)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tw = torch.tensor(W, dtype=torch.float64)
    logits = torch.nn.functional.linear(th, tw)
    ce = torch.nn.functional.cross_entropy(logits, torch.tensor(y), reduction="none")
    (ce * torch.tensor(w)).sum().backward()
    np.testing.assert_allclose(loss, (ce * torch.tensor(w)).detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, 1).detach().numpy(), rtol=1e-13)


def test_gradient_by_finite_differences():
    h, W, y, w = _rand(4, 3, 6, 17, scale=2.0)
    _, _, dh = ov.vocab_loss(h, W, y, w)
    eps = 1e-6
    for r in range(3):
        for j in range(6):
            hp = h.copy()
            hm = h.copy()
            hp[r, j] += eps
            hm[r, j] -= eps
            num = (ov.vocab_loss(hp, W, y, w)[1].sum() - ov.vocab_loss(hm, W, y, w)[1].sum()) / (2 * eps)
            assert num == pytest.approx(dh[r, j], rel=1e-6, abs=1e-9)


def test_row_list_equals_dense_on_gathered_rows():
    rng = np.random.default_rng(5)
    T, d, V = 40, 8, 30
    h = rng.standard_normal((T, d))
    W = rng.standard_normal((V, d))
    rows = np.array([0, 3, 4, 17, 39])
    y = rng.integers(0, V, len(rows))
    a = ov.vocab_loss_rows(h, W, rows, y)
    b = ov.vocab_loss(h[rows], W, y)
    for x, z in zip(a, b):
        np.testing.assert_array_equal(x, z)


def test_ignored_targets():
    h, W, y, w = _rand(6, 5, 9, 40)
    y = y.copy()
    y[1] = -1
    y[3] = 40
    lse, loss, dh = ov.vocab_loss(h, W, y, w)
    assert loss[1] == 0.0 and loss[3] == 0.0
    assert not dh[1].any() and not dh[3].any()
    lse_ref = np.log(np.exp(h @ W.T).sum(1))
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13)
    keep = [0, 2, 4]
    _, loss_k, dh_k = ov.vocab_loss(h[keep], W, y[keep], w[keep])
    np.testing.assert_array_equal(loss[keep], loss_k)
    np.testing.assert_allclose(dh[keep], dh_k, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- head gradient
@pytest.mark.parametrize("R,d,V,scale", [(13, 24, 300, 3.0), (3, 7, 5, 1.0)])
def test_head_grad_matches_torch_autograd(R, d, V, scale):
    h, W, y, w = _rand(20 + R, R, d, V, scale)
    dW = ov.vocab_head_grad(h, W, y, w)
    th = torch.tensor(h, dtype=torch.float64)
    tw = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(torch.nn.functional.linear(th, tw), torch.tensor(y), reduction="none")
    (ce * torch.tensor(w)).sum().backward()
    np.testing.assert_allclose(dW, tw.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_head_grad_by_finite_differences_and_vocab_sum():
    h, W, y, w = _rand(7, 4, 5, 9, scale=2.0)
    y = y.copy()
    y[2] = -1  # an ignored row contributes nothing
    dW = ov.vocab_head_grad(h, W, y, w)
    eps = 1e-6
    for v in (0, 3, 8):
        for j in (0, 4):
            Wp = W.copy()
            Wm = W.copy()
            Wp[v, j] += eps
            Wm[v, j] -= eps
            num = (ov.vocab_loss(h, Wp, y, w)[1].sum() - ov.vocab_loss(h, Wm, y, w)[1].sum()) / (2 * eps)
            assert num == pytest.approx(dW[v, j], rel=1e-6, abs=1e-9)
    # sum over the vocabulary of g_r is w_r (1 - 1) = 0, so dW sums to zero over v
    assert np.abs(dW.sum(axis=0)).max() < 1e-12
    keep = [0, 1, 3]
    np.testing.assert_allclose(dW, ov.vocab_head_grad(h[keep], W, y[keep], w[keep]), rtol=1e-13, atol=1e-15)
