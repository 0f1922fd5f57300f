"""fp64 CPU oracle of the streaming vocabulary loss.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py``.  The product library never imports
it, and it shares no code with the HIP path.

What is computed (Turbo-dLLM page, "Library" section, tables "Speculative
Decoding Optimizations" and "Block Diffusion Optimizations", row
"Vocabulary loss"): selected rows of the final hidden states go through the
LM head W and a token-level cross-entropy against their target tokens,
together with the gradient with respect to those hidden rows and, where the
head is trained (the block-diffusion row does not call it frozen; the
speculative-decoding row does), with respect to W.  The pages describe how
the work is streamed (token chunks, full-sequence logits never held), not a
formula; the oracle is the plain definition of weighted softmax
cross-entropy, computed here with the full logits of every row at once:

  s_r     = h_r W^T                              (logits, length V)
  lse_r   = log sum_v exp(s_rv)
  loss_r  = w_r (lse_r - s_r[y_r])
  g_r     = w_r (softmax(s_r) - e_{y_r})          (d loss_r / d s_r)
  dh_r    = g_r W                                 (d loss_r / d h_r)
  dW      = sum_r g_r^T h_r                       (d sum_r loss_r / d W)

A row whose target lies outside [0, V) is ignored: loss 0 and gradient 0
(its lse is still reported).
"""
import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _logit_grad(h, w_head, targets, weights):
    """(lse, loss, g) of the rows: g [R, V] is d loss_r / d s_r."""
    h = _f64(h)
    W = _f64(w_head)
    R = h.shape[0]
    V = W.shape[0]
    y = np.asarray(targets, dtype=np.int64).reshape(R)
    w = np.ones(R) if weights is None else _f64(weights).reshape(R)
    s = h @ W.T
    m = s.max(axis=1) if V > 0 else np.zeros(R)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    valid = (y >= 0) & (y < V)
    yc = np.where(valid, y, 0)
    rows = np.arange(R)
    s_y = s[rows, yc]
    loss = np.where(valid, w * (lse - s_y), 0.0)
    g = np.exp(s - lse[:, None])
    g[rows[valid], yc[valid]] -= 1.0
    g *= np.where(valid, w, 0.0)[:, None]
    return lse, loss, g


def vocab_loss(h, w_head, targets, weights=None):
    """Per-row lse, per-row weighted loss and dh for hidden rows ``h``
    [R, d] against the head ``w_head`` [V, d].  ``weights`` defaults to 1.
    Returns (lse [R], loss [R], dh [R, d]) in float64."""
    lse, loss, g = _logit_grad(h, w_head, targets, weights)
    return lse, loss, g @ _f64(w_head)


def vocab_head_grad(h, w_head, targets, weights=None):
    """dW [V, d] = sum_r g_r^T h_r, the gradient of the summed loss with
    respect to the head (float64)."""
    _, _, g = _logit_grad(h, w_head, targets, weights)
    return g.T @ _f64(h)


def vocab_loss_rows(h_all, w_head, rows, targets, weights=None):
    """The same loss over the rows ``rows`` of ``h_all`` [T, d] (the rows
    that carry the loss).  Returns (lse [R], loss [R], dh_rows [R, d]),
    row r of each belonging to position rows[r] of the sequence."""
    idx = np.asarray(rows, dtype=np.int64)
    return vocab_loss(_f64(h_all)[idx], w_head, targets, weights)
