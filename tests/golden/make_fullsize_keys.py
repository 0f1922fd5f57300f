"""Writes tests/golden/fullsize_keys_<workload>.npz: the oracle's dK and dV of
selected key rows of the full-size workloads (tests/workloads.py), for the
GPU parity tests.

Calls only the oracle (oracle/rowstats.py, the batched fp64 route pinned
against the C oracle by tests/test_rowstats_oracle.py) on inputs from the
seeded generator; nothing here runs or reads the HIP path.

Each file holds: keys (doubled positions), b, g, dk, dv (float64 [keys, d]),
and fingerprints of the inputs it was computed from (the bf16 bits of K at
the keys, and of Q and dO at a few rows), which the GPU test compares with
the inputs it generates before comparing gradients.

usage: python tests/golden/make_fullsize_keys.py [workload ...]   (default: all)
The 512K share takes about half an hour on 8 cores.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import oracle as orc  # noqa: E402
from oracle import rowstats as RS  # noqa: E402
from tests import workloads as W  # noqa: E402

FP_ROWS = 8


def out_path(name):
    return os.path.join(HERE, f"fullsize_keys_{name}.npz")


def fingerprint_rows(n2):
    return np.linspace(0, n2 - 1, FP_ROWS).astype(np.int64)


def _save(name, meta, keys, b, g, dk, dv, host):
    qh, kh, _, doh = host
    fr = fingerprint_rows(qh.shape[1])
    np.savez(out_path(name), keys=np.asarray(keys, np.int64), b=b, g=g, dk=dk, dv=dv,
             fp_k=kh[b, keys, g], fp_q=qh[b, fr], fp_do=doh[b, fr], fp_rows=fr,
             meta=json.dumps(meta, sort_keys=True))


def make_whole(name):
    w = W.WHOLE[name]
    _, host = W.whole_host(w)
    qh, kh, vh, doh = host
    p = orc.problem(w["batch"], w["L"], w["M"], w["hq"], w["hkv"], w["d"], bf16=True)
    L = w["L"]
    keys = W.clean_keys(L, w["M"]) + [L, L + L // 2 + 5, 2 * L - 1]
    rows = np.arange(2 * L)
    lse, D = RS.row_stats(p, qh, kh, vh, doh, w["b"], w["g"], rows)
    dk, dv = RS.dkdv_keys(p, qh, kh, vh, doh, w["b"], w["g"], keys, rows, lse, D)
    _save(name, dict(w, kind="whole"), keys, w["b"], w["g"], dk, dv, host)


def make_csbp(name):
    w = W.CSBP[name]
    _, host, pos, blocks, _, _ = W.csbp_host(w)
    qh, kh, vh, doh = host
    p = orc.problem(1, w["L"], w["M"], w["hq"], w["hkv"], w["d"], bf16=True)
    keys = W.csbp_keys(w, blocks)
    lse, D = RS.row_stats(p, qh, kh, vh, doh, 0, w["g"], pos)
    dk, dv = RS.dkdv_keys(p, qh, kh, vh, doh, 0, w["g"], keys, pos, lse, D)
    _save(name, dict(w, kind="csbp"), keys, 0, w["g"], dk, dv, host)


def main(names):
    for name in names:
        t = time.time()
        (make_whole if name in W.WHOLE else make_csbp)(name)
        print(f"{name}: {time.time() - t:.0f} s -> {out_path(name)}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(W.WHOLE) + list(W.CSBP))
