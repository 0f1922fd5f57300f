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


def csbp_inputs(seed, L, M, hq, hkv, d, blocks, clean_q, device="cuda", outlier_frac=0.0, std=1.0):
    """One rank's tensors: share clean query rows (packed), packed corrupted
    q/k/v of `blocks`, clean k/v [1, L, hkv, d], dO over the share rows."""
    n_clean = sum(hi - lo for lo, hi in clean_q)
    nx = len(blocks) * M
    R = n_clean + nx
    f = dict(device=device, dtype=torch.bfloat16, std=std, outlier_frac=outlier_frac)
    return {
        "q_clean": synth.normal((1, max(n_clean, 1), hq, d), seed, "q_clean", **f)[:, :n_clean],
        "q_corr": synth.normal((1, nx, hq, d), seed, "q_corr", **f),
        "k_corr": synth.normal((1, nx, hkv, d), seed, "k_corr", **f),
        "v_corr": synth.normal((1, nx, hkv, d), seed, "v_corr", **f),
        "k_clean": synth.normal((1, L, hkv, d), seed, "k", **f),
        "v_clean": synth.normal((1, L, hkv, d), seed, "v", **f),
        "do": synth.normal((1, R, hq, d), seed, "do", device, torch.bfloat16, 1.0),
    }


def share_positions(L, M, blocks, clean_q):
    """Doubled-input position of every share row, in share row order."""
    pos = [np.arange(lo, hi) for lo, hi in clean_q]
    blocks = np.asarray(blocks, dtype=np.int64)
    pos.append((L + blocks[:, None] * M + np.arange(M)[None, :]).reshape(-1))
    return np.concatenate(pos).astype(np.int64)


def doubled_host(L, hq, hkv, d, t, blocks, clean_q, M):
    """Scatter a rank's tensors into the oracle's doubled layout (host,
    uint16 bf16 bits).  Rows the rank does not hold stay zero; the oracle
    reads only share rows and the keys they see."""
    pos = share_positions(L, M, blocks, clean_q)
    n_clean = sum(hi - lo for lo, hi in clean_q)
    q = np.zeros((1, 2 * L, hq, d), dtype=np.uint16)
    do = np.zeros((1, 2 * L, hq, d), dtype=np.uint16)
    k = np.zeros((1, 2 * L, hkv, d), dtype=np.uint16)
    v = np.zeros((1, 2 * L, hkv, d), dtype=np.uint16)
    if n_clean:
        q[0, pos[:n_clean]] = host_bits(t["q_clean"])[0]
    q[0, pos[n_clean:]] = host_bits(t["q_corr"])[0]
    do[0, pos] = host_bits(t["do"])[0]
    k[0, :L] = host_bits(t["k_clean"])[0]
    v[0, :L] = host_bits(t["v_clean"])[0]
    k[0, pos[n_clean:]] = host_bits(t["k_corr"])[0]
    v[0, pos[n_clean:]] = host_bits(t["v_corr"])[0]
    return q, k, v, do, pos
