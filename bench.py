"""Benchmark: BDLM attention forward + backward on one MI355X.

Default workload (the headline metric's configuration): whole BDLM mask at
L = 65536 clean tokens (131072 positions), block size M = 32, batch 1,
40 query heads / 8 KV heads, d_h = 128, bf16 inputs ~ N(0, 1), synthetic.
One step = forward (bf16 O, fp32 LSE), backward (dQ, dK, dV; the gradient
kernels write their outputs, so nothing needs zeroing) — the whole hot
path, nothing skipped.

Useful FLOPs count visible (query, key) pairs only: 4 d per pair forward and
10 d per pair backward, pairs per head = L (L + M) for the block-causal
clean copy.  Printed as one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    # name: (batch, L, M, hq, hkv, d[, clean-key window in tokens])
    "bdlm_L64K_M32_h40kv8_d128": (1, 65536, 32, 40, 8, 128),
    "bdlm_L8K_M32_b2_h16kv8_d128": (2, 8192, 32, 16, 8, 128),
    "bdlm_L64K_M32_h40kv8_d128_window1024": (1, 65536, 32, 40, 8, 128, 1024),
}


def whole_workload(work):
    """(batch, L, M, hq, hkv, d, window) of a WORKLOADS entry (window 0: none)."""
    return tuple(work[:6]) + ((work[6] if len(work) > 6 else 0),)
DEFAULT = "bdlm_L64K_M32_h40kv8_d128"
# One GPU's CSBP share: name -> (seed index, L, M, hq, hkv, P, clean-shard
# query rows, outlier fraction); rank 0, d = 128.
CSBP_WORKLOADS = {
    "csbp_L256K_P8_r0_h32kv8_d128": (3, 262144, 32, 32, 8, 8, False, 0.0),
    "csbp_L512K_M16_P16_r0_h32kv4_d128": (4, 524288, 16, 32, 4, 16, True, 0.01),
}
VOCAB_WORKLOADS = {
    # name: (L corrupted positions, block size M, hidden d, vocabulary V)
    "vocab_L64K_M32_d5120_V131072": (65536, 32, 5120, 131072),
}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def sources_sha(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, scaled by the copy-kernel calibration; None when absent,
    when the counters were taken on another workload, or when the kernel's
    sources changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("workload") != workload:
        return None
    if not all(os.path.exists(os.path.join(ROOT, r)) for r in rec["sources"]):
        return None
    if sources_sha(rec["sources"]) != rec["sha256"]:
        return None
    return int(rec["bytes_per_launch"])


def calibrate_copy(nbytes):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}), flush=True)


def visible_pairs(L, M, window=0, token_causal=False):
    """Visible (query, key) pairs per head of the whole mask.  Without a
    window, L (L + M) for the block-causal clean copy.  With a clean-key
    window W, per token position t (block b = t // M, offset i = t % M):
    the clean row sees (b + 1) M - max(0, t - W + 1) keys (min(t + 1, W)
    token-causal) and the corrupted row M + max(0, min(b M, W - 1 - i))."""
    if window <= 0 and not token_causal:
        return L * (L + M)
    t = np.arange(L, dtype=np.int64)
    b, i = t // M, t % M
    if window <= 0:
        return int((t + 1).sum() + ((b + 1) * M).sum())
    if token_causal:
        clean = np.minimum(t + 1, window)
    else:
        clean = (b + 1) * M - np.maximum(0, t - window + 1)
    corr = M + np.maximum(0, np.minimum(b * M, window - 1 - i))
    return int(clean.sum() + corr.sum())


def tile_counts(L, M, qt=128, kt=64, window=0):
    """(visited, total) (query tile, key tile) pairs per head of the whole
    block-causal mask at the forward kernel's granularity (128 query rows,
    64 keys), from the mask geometry: a clean query tile sees the clean
    keys up to the end of its last row's block; a corrupted query tile sees
    the clean keys before its last row's block and the corrupted keys of
    its own blocks.  With a clean-key window W, the tile's first row sees
    clean keys from its position - W + 1 on (exact for W > M, where the
    rows of a tile together see one unbroken key range).  Key tiles of the
    clean and corrupted key spaces start at 0 and at L."""
    a = np.arange(0, L, qt, dtype=np.int64)
    last = np.minimum(a + qt, L) - 1
    lo = np.maximum(0, a - window + 1) // kt * kt if window > 0 else np.zeros_like(a)
    clean_end = (last // M + 1) * M
    visited = ((clean_end + kt - 1) // kt - lo // kt).sum()
    corr_clean = (last // M) * M
    own_lo, own_hi = (a // M) * M, (last // M + 1) * M
    visited += np.where(corr_clean > lo, (corr_clean + kt - 1) // kt - lo // kt, 0).sum()
    visited += ((own_hi + kt - 1) // kt - own_lo // kt).sum()
    nkt = 2 * ((L + kt - 1) // kt)
    return int(visited), int(2 * len(a) * nkt)


def _sclk_file():
    """The pp_dpm_sclk sysfs file of cuda:0's card (matched by PCI address),
    or None.  Called before the timed region."""
    import glob

    import torch
    try:
        pr = torch.cuda.get_device_properties(0)
        want = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}."
    except Exception:  # measurement aid only
        return None
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            if os.path.basename(os.path.realpath(os.path.dirname(f))).lower().startswith(want):
                return f
        except OSError:
            continue
    return None


def gpu_clock_sample(delay_s, path, out):
    """After `delay_s`, read the current sclk level (the line marked '*') from
    the card's sysfs file: a plain file read, no process is started.  Runs in
    a thread while the timed steps execute; stores "(NNNNMhz)" text or None."""
    time.sleep(delay_s)
    try:
        with open(path) as f:
            cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
        out.append(f"sclk {cur[0]} (pp_dpm_sclk)" if cur else None)
    except Exception:  # measurement aid only
        out.append(None)


def frac_at_clock(tflops, clock_line):
    """Useful TFLOP/s over the bf16 peak scaled from 2.4 GHz to the sampled
    clock (the first "NNNNMhz" in the sysfs line), or None."""
    import re
    m = re.search(r"(\d+)\s*Mhz", clock_line or "", re.I)
    if not m:
        return None
    return round(tflops / (PEAK_BF16_TFLOPS * int(m.group(1)) / 2400.0), 4)


def kernel_flops(name, pairs, hq, batch, d):
    """Algorithmic FLOPs one launch of each kernel performs on visible pairs:
    forward 4d (QK^T, PV); dK/dV kernel 8d (QK^T, dO V^T, P^T dO, dS^T Q);
    dQ kernel 2d useful (dS K; its QK^T and dO V^T recompute is not counted)."""
    per = {"fwd_bf16": 4 * d, "dkdv": 8 * d, "dq": 2 * d}.get(name)
    return None if per is None else per * pairs * hq * batch


def cpu_baseline(work, q, k, v, do, nrows, seed=0):
    """Oracle (fp64 CPU) on a bounded sample of the same workload: forward
    and dQ of `nrows` seeded (row, head) pairs of KV group 0."""
    import torch

    from oracle import oracle as orc
    batch, L, M, hq, hkv, d, window = whole_workload(work)
    G = hq // hkv
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, 2 * L, size=nrows)
    heads = rng.integers(0, G, size=nrows)
    bsel = np.zeros(nrows, dtype=np.int32)

    def host_full(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    hk, hv = host_full(k), host_full(v)
    hq_ = np.zeros((batch, 2 * L, hq, d), dtype=np.uint16)
    hdo = np.zeros((batch, 2 * L, hq, d), dtype=np.uint16)
    idx = torch.as_tensor(pos, device=q.device)
    hq_[0, pos, :G] = host_full(q[0, idx, :G])
    hdo[0, pos, :G] = host_full(do[0, idx, :G])
    p = orc.problem(batch, L, M, hq, hkv, d, bf16=True, window=window)
    t0 = time.perf_counter()
    orc.dq_rows(p, orc.keys(), orc.keys(), hq_, hk, hv, hdo, bsel, heads, pos)
    dt = time.perf_counter() - t0
    # visible keys of each sampled row (block-causal clean copy; clean keys
    # from t - W + 1 on under a window W; a corrupted row adds its own block)
    t = np.where(pos < L, pos, pos - L)
    blk = t // M
    lo = np.maximum(0, t - window + 1) if window > 0 else np.zeros_like(t)
    clean_hi = np.where(pos < L, (blk + 1) * M, blk * M)
    nvis = np.maximum(0, clean_hi - lo) + np.where(pos < L, 0, M)
    flops = float(nvis.sum()) * 8 * d  # forward 4d + dQ part of the backward 4d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"fp64 forward + dQ of {nrows} seeded (row, head) pairs of KV group 0; "
                      f"useful FLOPs 8*d per visible pair; {dt:.1f} s"}


def share_pairs(L, M, blocks, clean_q):
    """Visible (query, key) pairs per head of a share over every key."""
    blocks = np.asarray(blocks, dtype=np.int64)
    n = int(((blocks + 1) * M).sum() * M)  # corrupted block b: M rows x (b+1)M keys
    for lo, hi in clean_q:
        t = np.arange(lo, hi, dtype=np.int64)
        n += int(((t // M + 1) * M).sum())
    return n


def csbp_setup(name, dev):
    """Inputs, buffers and one-step closure of a CSBP share workload: the
    local call, P zigzag shard calls each followed by an LSE merge, then the
    backward over the local keys and every shard (accumulators zeroed first,
    as the first call of a step needs).  Returns a dict with the step, the
    useful FLOPs per step and the merge's algorithmic bytes per step."""
    import torch

    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd import synth
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare

    idx, L, M, hq, hkv, P, clean_queries, outl = CSBP_WORKLOADS[name]
    d = 128
    blocks = B.bdattn_assign_blocks(L // M, P, 0).tolist()
    cs = B.bdattn_clean_shard(L, P, 0)
    clean_q = [(cs.lo[0], cs.hi[0]), (cs.lo[1], cs.hi[1])] if clean_queries else []
    shards = []
    for s_ in range(P):
        kk = B.bdattn_clean_shard(L, P, s_)
        shards.append([(kk.lo[0], kk.hi[0]), (kk.lo[1], kk.hi[1])])
    seed = synth.SEED_BASE + idx
    n_clean = sum(hi - lo for lo, hi in clean_q)
    nx = len(blocks) * M
    f = dict(device=dev, outlier_frac=outl)
    qc = synth.normal((1, max(n_clean, 1), hq, d), seed, "q_clean", **f)[:, :n_clean]
    qx = synth.normal((1, nx, hq, d), seed, "q_corr", **f)
    kx = synth.normal((1, nx, hkv, d), seed, "k_corr", **f)
    vx = synth.normal((1, nx, hkv, d), seed, "v_corr", **f)
    kc = synth.normal((1, L, hkv, d), seed, "k", **f)
    vc = synth.normal((1, L, hkv, d), seed, "v", **f)
    sh = CsbpShare(1, L, M, hq, hkv, d, blocks, clean_q, shards)
    do = synth.normal((1, sh.R, hq, d), seed, "do", dev)
    wf, wb = sh.workspace(False, dev), sh.workspace(True, dev)
    grads = sh.alloc_grads(dev)

    def step(mid=None):
        o32, lse, _ = sh.fwd(qc, qx, kc, vc, kx, vx, ws=wf)
        if mid is not None:
            mid.record()
        for g_ in grads[:5]:
            g_.zero_()
        sh.bwd(qc, qx, kc, vc, kx, vx, o32, lse, do, ws=wb, grads=grads)

    # merge: per merged row, read two (O, LSE) partials and write one in fp32,
    # plus the bf16 O of the last merge: P merges of R * hq rows per step
    mrows = sh.R * hq
    return {"step": step, "flops": 14 * d * share_pairs(L, M, blocks, clean_q) * hq, "L": L, "M": M, "P": P,
            "hq": hq, "hkv": hkv, "d": d, "R": sh.R, "blocks": len(blocks), "clean_q": clean_q,
            "merge_bytes": P * mrows * 3 * (4 * d + 4) + mrows * 2 * d,
            "merge_rows_per_launch": mrows}


def report_all(reps=3):
    """Times every benchmark workload (stderr table, one JSON line per
    workload on stdout).  Not the headline line: that is the default run."""
    import torch

    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd import synth
    from block_diffusion_lm_bdlm_amd.runner import CsbpShare, WholeMask

    dev = torch.device("cuda:0")

    def timed(fn):
        """Average ms per call and each kernel's average ms per call, over
        enough calls to fill about 150 ms of GPU time (at least `reps`, at
        most 50): a few steps of a small workload are too short a window
        for a stable clock."""
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        est_ms = (time.perf_counter() - t0) * 1e3
        n = max(reps, min(50, math.ceil(150.0 / max(est_ms, 1e-3))))
        B.bdattn_profile_read()
        B.bdattn_profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        B.bdattn_profile_enable(False)
        prof = B.bdattn_profile_read()
        return e0.elapsed_time(e1) / n, {k: t / n for k, (_, t) in prof.items()}

    rows = []
    whole = [("fp32_L1K_M16_h4_d64_fwd", 0, (1, 1024, 16, 4, 4, 64), torch.float32, 1.0, False, 0),
             ("bf16_L8K_M32_b2_h16kv8", 1, (2, 8192, 32, 16, 8, 128), torch.bfloat16, 128 ** -0.5, True, 0),
             ("bf16_L64K_M32_h40kv8", 2, (1, 65536, 32, 40, 8, 128), torch.bfloat16, 1.0, True, 0),
             # the 64K workload under a 1,024-token clean-key sliding window
             ("bf16_L64K_M32_h40kv8_window1024", 2, (1, 65536, 32, 40, 8, 128), torch.bfloat16, 1.0, True,
              1024)]
    for name, idx, (batch, L, M, hq, hkv, d), dt, std, bwd, window in whole:
        seed = synth.SEED_BASE + idx
        n2 = 2 * L
        q = synth.normal((batch, n2, hq, d), seed, "q", dev, dt, std)
        k = synth.normal((batch, n2, hkv, d), seed, "k", dev, dt, std)
        v = synth.normal((batch, n2, hkv, d), seed, "v", dev, dt, std)
        do = synth.normal((batch, n2, hq, d), seed, "do", dev, torch.bfloat16)
        wm = WholeMask(batch, L, M, hq, hkv, d, B.BDATTN_F32 if dt == torch.float32 else B.BDATTN_BF16,
                       window=window)
        wf, wb = wm.workspace(False, dev), wm.workspace(True, dev)
        grads = wm.alloc_grads(dev)
        o_code = B.BDATTN_F32 if dt == torch.float32 else B.BDATTN_BF16
        o = torch.empty(batch, n2, hq, d, dtype=dt, device=dev)
        lse = torch.empty(batch, n2, hq, dtype=torch.float32, device=dev)

        def step():
            # the library calls themselves, as in the headline step (the
            # runner's bwd also joins the clean and corrupted dK/dV: a copy
            # the hot path does not make)
            B.bdattn_fwd(wm.prob, wm.share, wm.kv, q[:, :L], q[:, L:], k[:, :L], v[:, :L], k[:, L:], v[:, L:],
                         o, o_code, lse, wf)
            if bwd:
                dq, dkc, dvc, dkx, dvx, delta = grads
                B.bdattn_bwd(wm.prob, wm.share, wm.kv, q[:, :L], q[:, L:], k[:, :L], v[:, :L], k[:, L:], v[:, L:],
                             o, o_code, lse, do, delta, B.BDATTN_BWD_OVERWRITE, dq, dkc, dvc, dkx, dvx, wb)

        ms, kern = timed(step)
        pairs = visible_pairs(L, M, window) * hq * batch
        flops = (14 if bwd else 4) * d * pairs
        rows.append((name, ms, flops, batch * L, kern))
        del q, k, v, do, wm, wf, wb, grads, o, lse
        torch.cuda.empty_cache()
    merge_bytes = {}
    for name in CSBP_WORKLOADS:
        cs_ = csbp_setup(name, dev)
        ms, kern = timed(cs_["step"])
        merge_bytes[name] = cs_["merge_bytes"]
        rows.append((name, ms, cs_["flops"], cs_["L"] // cs_["P"], kern))
        del cs_
        torch.cuda.empty_cache()
    print(f"{'workload':36s} {'ms':>9s} {'useful TF/s':>12s} {'% of 2.5PF':>10s} {'tokens/s':>12s}",
          file=sys.stderr)
    for name, ms, flops, toks, kern in rows:
        tf = flops / (ms * 1e-3) / 1e12
        print(f"{name:36s} {ms:9.2f} {tf:12.1f} {100 * tf / PEAK_BF16_TFLOPS:10.2f} {toks / (ms * 1e-3):12.0f}",
              file=sys.stderr)
        print("    kernels (ms per step): " + ", ".join(f"{n} {t:.3f}" for n, t in sorted(kern.items(), key=lambda x: -x[1])),
              file=sys.stderr)
        line = {"workload": name, "ms": round(ms, 3), "useful_tflops": round(tf, 2),
                "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "tokens_per_s": round(toks / (ms * 1e-3), 1),
                "kernels_ms": {n: round(t, 4) for n, t in kern.items()}}
        if name in merge_bytes and kern.get("merge"):
            gbs = merge_bytes[name] / (kern["merge"] * 1e-3) / 1e9
            line["merge_roofline"] = {"bound": "hbm", "algorithmic_bytes": merge_bytes[name],
                                      "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / PEAK_HBM_GBS, 4)}
            print(f"    merge: {merge_bytes[name] / 1e9:.2f} GB per step, {gbs:.0f} GB/s", file=sys.stderr)
        print(json.dumps(line), flush=True)


def vocab_cpu_baseline(h, W, rows, y, wt, nrows, seed=0):
    """Oracle (fp64 CPU) on a bounded sample of the vocabulary-loss workload:
    loss, lse and dh of `nrows` seeded loss rows against the full head."""
    from threadpoolctl import threadpool_info

    from oracle import vocab as ov
    rng = np.random.default_rng(seed)
    pick = np.sort(rng.choice(rows.numel(), size=min(nrows, rows.numel()), replace=False))
    hs = h[rows.to(h.device)[pick].long()].float().cpu().numpy()
    Wh = W.float().cpu().numpy()
    t0 = time.perf_counter()
    ov.vocab_loss(hs, Wh, y.cpu().numpy()[pick], wt.cpu().numpy()[pick])
    dt = time.perf_counter() - t0
    cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {"value": round(len(pick) / dt, 3), "unit": "loss rows/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 lse, loss and dh of {len(pick)} seeded loss rows against the full "
                      f"{W.shape[0]} x {W.shape[1]} head (numpy BLAS); {dt:.1f} s"}


def bench_vocab(args):
    """Streaming vocabulary loss: the masked positions of L corrupted
    positions (per-block ratio t ~ U(0, 1)) go through the head in chunks of
    8192 rows; one step = loss, lse, loss sum and dh of every loss row
    (frozen head; useful FLOPs 4 R V d: logits GEMM + gradient GEMM).  The
    line also times the step with the head trained (dW cleared and
    accumulated; 6 R V d) under "with_head_grad"."""
    import torch

    from block_diffusion_lm_bdlm_amd import bdvocab as BV
    from block_diffusion_lm_bdlm_amd import synth

    L, M, d, V = VOCAB_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    seed = synth.SEED_BASE + 3
    print(f"[bench] generating inputs for {args.workload}", file=sys.stderr, flush=True)
    rows = synth.masked_rows(seed, L, M)
    R = int(rows.numel())
    h, W, y, wt = synth.vocab_inputs(seed, L, d, V, R=R, device=dev)
    rows_d = rows.to(dev)
    vl = BV.VocabLoss(R, V, d, row_list=True, device=dev)
    dh = torch.zeros((L, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    loss = torch.empty(R, dtype=torch.float32, device=dev)
    loss_sum = torch.empty(1, dtype=torch.float32, device=dev)

    def step():
        vl(h, W, y, weights=wt, rows=rows_d, dh=dh, lse=lse, loss=loss, loss_sum=loss_sum)

    print("[bench] tuning the GEMMs (set-up, outside the timed steps)", file=sys.stderr, flush=True)
    vl.tune(h, W, dh_stride=dh.stride(0))
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    BV.bdvocab_profile_read()
    BV.bdvocab_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    BV.bdvocab_profile_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    prof = BV.bdvocab_profile_read()
    print(f"[bench] {args.steps} steps, {ms:.2f} ms/step; kernels: "
          + ", ".join(f"{n} {c}x {t / c:.3f} ms" for n, (c, t) in sorted(prof.items(), key=lambda x: -x[1][1])),
          file=sys.stderr, flush=True)
    useful = 4.0 * R * V * d
    tflops = useful / (ms * 1e-3) / 1e12
    chunk = min(8192, R)
    n_chunks = (R + chunk - 1) // chunk
    gemm_flops = 2.0 * chunk * V * d  # per launch of a full chunk (the ragged last one is smaller)
    dom_name, (dom_cnt, dom_ms) = max(((k_, v_) for k_, v_ in prof.items() if k_.endswith("gemm")),
                                      key=lambda kv_: kv_[1][1])
    dom_flops = 2.0 * R * V * d * args.steps / dom_cnt  # average work per launch
    dom_avg = dom_ms / dom_cnt
    ach = dom_flops / (dom_avg * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom_name, args.workload),
            "avg_ms": round(dom_avg, 3), "library": "hipBLASLt"}
    rc, rms = prof["rows"]
    rows_bytes = 6.0 * R * V * args.steps / rc  # fp32 logits read once + bf16 gradient written, per launch
    rach = rows_bytes / (rms / rc * 1e-3) / 1e9
    roof_rows = {"bound": "hbm", "kernel": "rows", "achieved": round(rach, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(rach / PEAK_HBM_GBS, 4), "traffic": measured_traffic("vocab_rows", args.workload),
                 "avg_ms": round(rms / rc, 3)}
    # the same step with the head trained: dW cleared, then accumulated per chunk
    dw = torch.zeros((V, d), dtype=torch.float32, device=dev)
    del vl
    torch.cuda.empty_cache()
    vl_dw = BV.VocabLoss(R, V, d, row_list=True, head_grad=True, device=dev)
    vl_dw.tune(h, W, dh_stride=dh.stride(0))

    def step_dw():
        dw.zero_()
        vl_dw(h, W, y, weights=wt, rows=rows_d, dh=dh, lse=lse, loss=loss, loss_sum=loss_sum, dw=dw)

    for _ in range(args.warmup):
        step_dw()
    torch.cuda.synchronize()
    BV.bdvocab_profile_enable(True)
    e0.record()
    for _ in range(args.steps):
        step_dw()
    e1.record()
    torch.cuda.synchronize()
    BV.bdvocab_profile_enable(False)
    ms_dw = e0.elapsed_time(e1) / args.steps
    prof_dw = BV.bdvocab_profile_read()
    print(f"[bench] with head gradient: {ms_dw:.2f} ms/step; kernels: "
          + ", ".join(f"{n} {c}x {t / c:.3f} ms" for n, (c, t) in sorted(prof_dw.items(), key=lambda x: -x[1][1])),
          file=sys.stderr, flush=True)
    with_dw = {"ms_per_step": round(ms_dw, 3), "loss_rows_per_s": round(R / (ms_dw * 1e-3), 1),
               "useful_tflops": round(6.0 * R * V * d / (ms_dw * 1e-3) / 1e12, 2),
               "kernels": {n: {"launches": c, "avg_ms": round(t / c, 4)} for n, (c, t) in prof_dw.items()}}
    del dw, vl_dw
    cpu = None
    if args.cpu_rows > 0:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        cpu = vocab_cpu_baseline(h, W, rows, y, wt, min(args.cpu_rows, 4096))
    out = {
        "metric": "vocabulary loss rows/s through the frozen head, loss + dh (1 GPU)",
        "value": round(R / (ms * 1e-3), 1),
        "unit": "loss rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) hidden rows, N(0, 9/d) head, uniform targets, seeded",
        "config": {"workload": args.workload, "L": L, "M": M, "loss_rows": R, "hidden": d, "vocab": V,
                   "chunk": chunk, "chunks": n_chunks, "parallelism": "single GPU"},
        "useful_tflops": round(tflops, 2),
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_flop_per_full_chunk": gemm_flops,
        "logits_bytes_per_chunk": chunk * ((V + 63) // 64 * 64) * 4,
        "kernels": {n: {"launches": c, "avg_ms": round(t / c, 4)} for n, (c, t) in prof.items()},
        "roofline": roof,
        "roofline_rows": roof_rows,
        "with_head_grad": with_dw,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_csbp(args):
    """One GPU's CSBP share: P shard calls merged by LSE and the sharded
    backward, timed per step; the dominant kernel's MFMA roofline and the
    LSE merge's HBM roofline (algorithmic bytes per launch over its average
    launch time)."""
    import torch

    from block_diffusion_lm_bdlm_amd import bdattn as B

    dev = torch.device("cuda:0")
    print(f"[bench] generating inputs for {args.workload}", file=sys.stderr, flush=True)
    cs = csbp_setup(args.workload, dev)
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        cs["step"]()
    torch.cuda.synchronize()
    B.bdattn_profile_read()
    B.bdattn_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        marks[i][0].record()
        cs["step"](marks[i][1])
        marks[i][2].record()
    e1.record()
    torch.cuda.synchronize()
    B.bdattn_profile_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    prof = B.bdattn_profile_read()
    print(f"[bench] {args.steps} steps, {ms:.2f} ms/step; kernels: "
          + ", ".join(f"{n} {c}x {t / c:.3f} ms" for n, (c, t) in sorted(prof.items(), key=lambda x: -x[1][1])),
          file=sys.stderr, flush=True)
    tflops = cs["flops"] / (ms * 1e-3) / 1e12
    dom_name, (dom_cnt, dom_ms) = max(prof.items(), key=lambda kv_: kv_[1][1])
    dom_avg = dom_ms / dom_cnt
    # the share's useful FLOPs of the dominant kernel per step, spread over its launches
    per_pair = {"fwd_bf16": 4, "dkdv": 8, "dq": 2}.get(dom_name)
    roof = None
    if per_pair is not None:
        ach = per_pair / 14.0 * cs["flops"] / dom_cnt * args.steps / (dom_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "avg_ms": round(dom_avg, 3)}
    merge = None
    if "merge" in prof:
        mc, mt = prof["merge"]
        per_launch = cs["merge_bytes"] / cs["P"]  # the last merge also writes bf16 O: averaged in
        gbs = per_launch / (mt / mc * 1e-3) / 1e9
        merge = {"bound": "hbm", "kernel": "merge", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": int(per_launch),
                 "rows_per_launch": cs["merge_rows_per_launch"], "avg_ms": round(mt / mc, 4)}
    step_ms = [m[0].elapsed_time(m[2]) for m in marks]
    out = {
        "metric": "useful attention TFLOP/s fwd+bwd of one GPU's CSBP share (1 GPU); % of bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic N(0,1) bf16 inputs, seeded",
        "config": {"workload": args.workload, "L": cs["L"], "M": cs["M"], "P": cs["P"], "rank": 0,
                   "blocks": cs["blocks"], "share_rows": cs["R"], "clean_query_ranges": cs["clean_q"],
                   "hq": cs["hq"], "hkv": cs["hkv"], "d": cs["d"], "parallelism": "single GPU"},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(cs["L"] / cs["P"] / (ms * 1e-3), 1),
        "step_ms": {"median": round(float(np.median(step_ms)), 3), "min": round(min(step_ms), 3),
                    "max": round(max(step_ms), 3)},
        "fwd_ms_median": round(float(np.median([m[0].elapsed_time(m[1]) for m in marks])), 3),
        "bwd_ms_median": round(float(np.median([m[1].elapsed_time(m[2]) for m in marks])), 3),
        "kernels": {n: {"launches": c, "avg_ms": round(t / c, 4)} for n, (c, t) in prof.items()},
        "roofline": roof,
        "merge_roofline": merge,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT,
                    choices=sorted(WORKLOADS) + sorted(CSBP_WORKLOADS) + sorted(VOCAB_WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=8192, help="oracle sample size (0: skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--report-all", action="store_true",
                    help="time every benchmark workload (table on stderr) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.report_all:
        report_all()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the hot path; runs on more than one GPU are not "
              "part of this build (see DESIGN.md, 'How the path would shard').", file=sys.stderr)
        sys.exit(2)

    if args.workload in VOCAB_WORKLOADS:
        bench_vocab(args)
        return
    if args.workload in CSBP_WORKLOADS:
        bench_csbp(args)
        return

    import torch

    from block_diffusion_lm_bdlm_amd import bdattn as B
    from block_diffusion_lm_bdlm_amd import synth
    from block_diffusion_lm_bdlm_amd.runner import WholeMask

    dev = torch.device("cuda:0")
    work = WORKLOADS[args.workload]
    batch, L, M, hq, hkv, d, window = whole_workload(work)
    seed = synth.SEED_BASE + 2
    n2 = 2 * L
    print(f"[bench] generating inputs for {args.workload}", file=sys.stderr, flush=True)
    q = synth.normal((batch, n2, hq, d), seed, "q", dev)
    k = synth.normal((batch, n2, hkv, d), seed, "k", dev)
    v = synth.normal((batch, n2, hkv, d), seed, "v", dev)
    do = synth.normal((batch, n2, hq, d), seed, "do", dev)
    wm = WholeMask(batch, L, M, hq, hkv, d, window=window)
    ws_f = wm.workspace(False, dev)
    ws_b = wm.workspace(True, dev)
    grads = wm.alloc_grads(dev)
    o = torch.empty(batch, n2, hq, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(batch, n2, hq, dtype=torch.float32, device=dev)
    L_ = L

    def step(mid=None):
        B.bdattn_fwd(wm.prob, wm.share, wm.kv, q[:, :L_], q[:, L_:], k[:, :L_], v[:, :L_], k[:, L_:],
                     v[:, L_:], o, B.BDATTN_BF16, lse, ws_f)
        if mid is not None:
            mid.record()
        dq, dkc, dvc, dkx, dvx, delta = grads
        B.bdattn_bwd(wm.prob, wm.share, wm.kv, q[:, :L_], q[:, L_:], k[:, :L_], v[:, :L_], k[:, L_:],
                     v[:, L_:], o, B.BDATTN_BF16, lse, do, delta, B.BDATTN_BWD_OVERWRITE, dq, dkc, dvc, dkx, dvx, ws_b)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    B.bdattn_plan_order(wm.prob, wm.share, wm.kv)  # the host plan of the whole-mask call
    plan_ms = (time.perf_counter() - t0) * 1e3
    B.bdattn_profile_read()  # drop anything recorded so far
    B.bdattn_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    clock = []
    import threading
    sclk = _sclk_file()
    clk = threading.Thread(target=gpu_clock_sample, args=(0.25, sclk, clock), daemon=True) if sclk else None
    torch.cuda.synchronize()
    if clk:
        clk.start()
    e0.record()
    for i in range(args.steps):
        marks[i][0].record()
        step(marks[i][1])
        marks[i][2].record()
    e1.record()
    torch.cuda.synchronize()
    if clk:
        clk.join(timeout=30)
    B.bdattn_profile_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    prof = B.bdattn_profile_read()
    step_ms = [m[0].elapsed_time(m[2]) for m in marks]
    fwd_ms = [m[0].elapsed_time(m[1]) for m in marks]
    bwd_ms = [m[1].elapsed_time(m[2]) for m in marks]
    print(f"[bench] {args.steps} steps, {ms:.2f} ms/step; kernels: "
          + ", ".join(f"{n} {c}x {t / c:.3f} ms" for n, (c, t) in sorted(prof.items(), key=lambda x: -x[1][1])),
          file=sys.stderr, flush=True)

    pairs = visible_pairs(L, M, window)
    tiles = tile_counts(L, M, window=window)
    useful = 14.0 * d * pairs * hq * batch
    tflops = useful / (ms * 1e-3) / 1e12
    # dominant kernel by time
    dom = max(prof.items(), key=lambda kv_: kv_[1][1])
    dom_name, (dom_cnt, dom_ms) = dom
    dom_avg = dom_ms / dom_cnt
    dflops = kernel_flops(dom_name, pairs, hq, batch, d)
    roof = None
    if dflops is not None:
        ach = dflops / (dom_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom_name, args.workload), "avg_ms": round(dom_avg, 3)}
    cpu = None
    if args.cpu_rows > 0:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(work, q, k, v, do, args.cpu_rows)
    kernels = {n: {"launches": c, "avg_ms": round(t / c, 4)} for n, (c, t) in prof.items()}
    out = {
        "metric": ("useful attention TFLOP/s fwd+bwd at 64K (1 GPU); % of bf16 MFMA peak" if args.workload == DEFAULT
                   else f"useful attention TFLOP/s fwd+bwd, {args.workload} (1 GPU); % of bf16 MFMA peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16 inputs, seeded",
        "config": {"workload": args.workload, "batch": batch, "L": L, "positions": n2, "M": M, "hq": hq,
                   "hkv": hkv, "d": d, "clean_mask": "block-causal", "window": window, "parallelism": "single GPU"},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(batch * L / (ms * 1e-3), 1),
        "positions_per_s": round(batch * n2 / (ms * 1e-3), 1),
        "useful_tflop_per_step": round(useful / 1e12, 3),
        # the stricter count: 12*d per pair (forward 4d, backward 8d without
        # the recomputed Q K^T)
        "useful_tflops_12d": round(12.0 / 14.0 * tflops, 2),
        # per-step events: forward = forward call, backward = backward call
        "step_ms": {"median": round(float(np.median(step_ms)), 3), "min": round(min(step_ms), 3),
                    "max": round(max(step_ms), 3)},
        "fwd_ms_median": round(float(np.median(fwd_ms)), 3),
        "bwd_ms_median": round(float(np.median(bwd_ms)), 3),
        "plan_ms": round(plan_ms, 3),
        "tiles_per_head": {"visited": tiles[0], "total": tiles[1], "skipped_frac": round(1 - tiles[0] / tiles[1], 4),
                           "granularity": "128 query rows x 64 keys"},
        "gpu_clock": clock[0] if clock else None,
        # the 2.5 PF figure assumes 2.4 GHz; the same peak scaled to the sampled clock
        "frac_of_peak_at_clock": frac_at_clock(tflops, clock[0] if clock else None),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
