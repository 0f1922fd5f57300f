"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module only draws random numbers; it holds none of the attention
arithmetic.  Both sides of every parity check receive the same tensor (the
HIP path a device copy, the oracle a host copy), so they see identical bits.

Recipe:
  * seed = SEED_BASE + workload index; each tensor has its own stream id
    (``TID``), so adding a tensor never changes the others.
  * draws are N(0, 1) float32 from torch's generator on the requested device,
    multiplied by ``std``, then rounded to nearest-even into ``dtype``.
  * ``outlier_frac`` > 0 scales a Bernoulli(outlier_frac) subset of rows by
    ``outlier_scale``; a row is one (token, head) vector of length d_h, and
    the subset is drawn from its own stream.
  * vocabulary-loss rows: every block of M corrupted positions draws a mask
    ratio t ~ U(0, 1) and masks each position with probability t; the
    masked positions are the rows that carry the loss, in increasing order,
    each with a target token uniform in [0, V) and weight 1 / (rows kept).
    Hidden rows are N(0, 1), the head N(0, head_std^2).
"""
import torch

SEED_BASE = 0x5EED0000
TID = {"q": 1, "k": 2, "v": 3, "do": 4, "q_corr": 5, "k_corr": 6, "v_corr": 7,
       "q_clean": 8, "h": 9, "w_head": 10, "targets": 11, "mask_t": 12, "mask_u": 13}
_OUTLIER_STREAM = 64


def _generator(device, seed, tid):
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed((int(seed) * 1_000_003 + int(tid)) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal(shape, seed, tensor, device="cpu", dtype=torch.bfloat16, std=1.0,
           outlier_frac=0.0, outlier_scale=8.0):
    """Seeded N(0, std^2) tensor of ``shape`` rounded to ``dtype``."""
    tid = TID[tensor] if isinstance(tensor, str) else int(tensor)
    g = _generator(device, seed, tid)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if outlier_frac > 0.0:
        g2 = _generator(device, seed, tid + _OUTLIER_STREAM)
        sel = torch.rand(tuple(shape[:-1]), generator=g2, device=device) < outlier_frac
        x[sel] *= outlier_scale
    return x.to(dtype)


def integers(shape, seed, tensor, high, device="cpu"):
    """Seeded integers uniform in [0, high) as int32."""
    g = _generator(device, seed, TID[tensor])
    return torch.randint(0, int(high), tuple(shape), generator=g, device=device, dtype=torch.int64).to(torch.int32)


def masked_rows(seed, L, M, device="cpu"):
    """Positions in [0, L) masked by a per-block ratio t ~ U(0, 1), as
    sorted int32 on ``device`` (drawn on the CPU, so the set does not
    depend on the device)."""
    nb = L // M
    t = torch.rand((nb, 1), generator=_generator("cpu", seed, TID["mask_t"]), dtype=torch.float64)
    u = torch.rand((nb, M), generator=_generator("cpu", seed, TID["mask_u"]), dtype=torch.float64)
    rows = torch.nonzero((u < t).reshape(-1)).reshape(-1).to(torch.int32)
    return rows.to(device)


def vocab_inputs(seed, T, d, V, R=None, device="cpu", head_std=None, rows=None):
    """Hidden rows h [T, d], head W [V, d] (bf16), targets [R] (int32) and
    weights [R] (fp32, all 1/R) for R loss rows (R defaults to T, or to
    len(rows) when a row list is given)."""
    if R is None:
        R = T if rows is None else int(rows.numel())
    std = head_std if head_std is not None else 3.0 / float(d) ** 0.5
    h = normal((T, d), seed, "h", device=device)
    w = normal((V, d), seed, "w_head", device=device, std=std)
    y = integers((R,), seed, "targets", V, device=device)
    wt = torch.full((R,), 1.0 / max(R, 1), dtype=torch.float32, device=device)
    return h, w, y, wt
