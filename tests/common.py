"""Helpers shared by the parity tests: input generation, host copies for the
oracle, error metrics and the tolerances of the parity bar.

Tolerances (stated per test):
  fp32 inputs: max |err| <= 1e-4 on O and LSE.
  bf16 inputs: max |err| <= 2e-2 on O, <= 1e-3 on LSE, relative L2 <= 1e-2 on
  dQ, dK, dV.
"""
import numpy as np
import torch

from block_diffusion_lm_bdlm_amd import synth

TOL_F32 = 1e-4
TOL_O = 2e-2
TOL_LSE = 1e-3
TOL_GRAD = 1e-2


def host_bits(t):
    """Host copy the oracle reads: uint16 bf16 bit patterns, or float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.float().numpy()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.abs(np.where(both_inf, 0.0, a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0


def doubled_inputs(seed, batch, L, hq, hkv, d, dtype=torch.bfloat16, std=1.0, device="cuda",
                   outlier_frac=0.0):
    """q, dO [batch, 2L, hq, d]; k, v [batch, 2L, hkv, d] (clean copy first)."""
    n2 = 2 * L
    q = synth.normal((batch, n2, hq, d), seed, "q", device, dtype, std, outlier_frac)
    k = synth.normal((batch, n2, hkv, d), seed, "k", device, dtype, std, outlier_frac)
    v = synth.normal((batch, n2, hkv, d), seed, "v", device, dtype, std, outlier_frac)
    do = synth.normal((batch, n2, hq, d), seed, "do", device, dtype, 1.0)
    return q, k, v, do
