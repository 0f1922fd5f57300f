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
"""
import torch

SEED_BASE = 0x5EED0000
TID = {"q": 1, "k": 2, "v": 3, "do": 4, "q_corr": 5, "k_corr": 6, "v_corr": 7,
       "q_clean": 8}
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
