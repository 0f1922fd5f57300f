"""The five benchmark workloads, their seeded inputs on the host, and the key
rows whose gradients are stored under tests/golden/ (fullsize_keys_*.npz).

Inputs are drawn on the CPU (synth.normal, torch's CPU generator) so that
the GPU tests and the script that writes the stored oracle values see the
same bits; the GPU tests copy them to the device.

Stored keys: one batch entry and one KV head per workload, clean keys
spread over [0, L) -- the first keys, which every later row sees and whose
gradients are the longest sums, keys around L/4, L/2 and 3L/4, and the last
keys -- plus corrupted keys of the share's own blocks.
"""
import numpy as np

from block_diffusion_lm_bdlm_amd import synth
from tests.common import csbp_inputs, doubled_host, doubled_inputs, host_bits

SEED0 = synth.SEED_BASE

WHOLE = {
    "bdlm_L8K_M32_b2_h16kv8_d128": dict(batch=2, L=8192, M=32, hq=16, hkv=8, d=128, std=128 ** -0.5,
                                        seed=SEED0 + 1, b=1, g=5),
    "bdlm_L64K_M32_h40kv8_d128": dict(batch=1, L=65536, M=32, hq=40, hkv=8, d=128, std=1.0, seed=SEED0 + 2,
                                      b=0, g=3),
}
CSBP = {
    "csbp_L256K_P8_r0_h32kv8_d128": dict(L=262144, M=32, hq=32, hkv=8, d=128, P=8, r=0, clean_queries=False,
                                         seed=SEED0 + 3, outlier_frac=0.0, g=2),
    "csbp_L512K_M16_P16_r0_h32kv4_d128": dict(L=524288, M=16, hq=32, hkv=4, d=128, P=16, r=0,
                                              clean_queries=True, seed=SEED0 + 4, outlier_frac=0.01, g=1),
}


def clean_keys(L, M):
    """Clean key rows (token positions) whose gradients are stored."""
    ks = [0, 1, M - 1, M, 3 * M + 5, L // 8 + 7, L // 4, L // 2 - 1, L // 2, 3 * L // 4 + 3, L - 2 * M - 1, L - 1]
    return sorted(set(ks))


def assign(L, M, P, r):
    """Dual-end block share and zigzag clean shards, by the chunk formula
    (pinned against the library's and the oracle's in test_abi_cpu.py)."""
    B = L // M
    c = B // (2 * P)
    chunks = np.arange(B).reshape(2 * P, c)
    blocks = np.concatenate([chunks[r], chunks[2 * P - 1 - r]]).tolist()
    w = L // (2 * P)
    shards = [[(s * w, (s + 1) * w), ((2 * P - 1 - s) * w, (2 * P - s) * w)] for s in range(P)]
    return blocks, shards


def whole_host(w):
    """Host tensors (CPU torch) of a whole-mask workload and their oracle copies."""
    q, k, v, do = doubled_inputs(w["seed"], w["batch"], w["L"], w["hq"], w["hkv"], w["d"], std=w["std"],
                                 device="cpu")
    return (q, k, v, do), tuple(host_bits(x) for x in (q, k, v, do))


def csbp_host(w):
    """Host tensors of a CSBP share workload, the oracle's doubled copies and
    the share's row positions."""
    blocks, shards = assign(w["L"], w["M"], w["P"], w["r"])
    clean_q = shards[w["r"]] if w["clean_queries"] else []
    t = csbp_inputs(w["seed"], w["L"], w["M"], w["hq"], w["hkv"], w["d"], blocks, clean_q, device="cpu",
                    outlier_frac=w["outlier_frac"])
    qh, kh, vh, doh, pos = doubled_host(w["L"], w["hq"], w["hkv"], w["d"], t, blocks, clean_q, w["M"])
    return t, (qh, kh, vh, doh), pos, blocks, clean_q, shards


def csbp_keys(w, blocks):
    """Stored keys of a share: clean keys over [0, L) and corrupted keys of
    the share's first, middle and last owned blocks (doubled positions)."""
    L, M = w["L"], w["M"]
    corr = [L + blocks[0] * M, L + blocks[len(blocks) // 2] * M + M // 2, L + blocks[-1] * M + M - 1]
    return clean_keys(L, M) + corr
