"""Batched fp64 route of the oracle for gradients of single key rows at full
size.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and by the committed script
``tests/golden/make_fullsize_keys.py`` that writes stored expected values;
the product library never imports it.

It computes the same definitions as ``bdoracle.c`` (the visible set of a
row, its softmax over that whole set, and the per-pair backward terms for
the loss sum(O * dO)), with torch float64 CPU matrix products in place of
the per-pair loops, so that the rows seeing an early clean key -- up to
every row of a 512K-token share -- finish in minutes:

* Visible set of a query at doubled position i ("CSBP 完全拆解", section
  "传统上下文并行为什么会传错东西", key/value set [K_b; K^clean_<b]; clean
  copy causal over itself, read block-causal or token-causal; optional
  clean-key window on token distance):
    clean query i < L:      clean keys [lo, hi), hi = (i // M + 1) M
                            (block-causal) or i + 1 (token-causal)
    corrupted query i >= L: clean keys [lo, b M) with b = (i - L) // M,
                            plus the corrupted keys of block b
  with lo = max(0, t - W + 1) for a window W (t the row's token position),
  else 0.  ``tests/test_rowstats_oracle.py`` checks this against the C
  predicate pair by pair.
* Row statistics over the full visible set: s = scale q . k,
  LSE = log sum exp s, O = sum softmax(s) v, D = dO . O.
* Gradient of one key j over a set of rows (a share), for the G query
  heads of its KV head: P = exp(s - LSE), dP = dO . v_j, dS = P (dP - D),
  dV_j = sum P dO, dK_j = scale sum dS q  ("CSBP 完全拆解", section
  "CSBP：BP 管损坏块，CP 管干净上下文": clean keys collect contributions
  from every later block).

Rows are batched only where their visible sets are identical (the rows of
one block, in the block-causal mask without a window), so each batch is one
plain softmax over one key set.
"""
import numpy as np
import torch


def _f64(a):
    """Host array (uint16 bf16 bits or float32) -> float64 torch tensor."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32)).double()
    return torch.from_numpy(a.astype(np.float32)).double()


def key_ranges(p, i):
    """Visible keys of doubled row i as (clean lo, clean hi, corrupted lo,
    corrupted hi), half-open, in doubled positions."""
    L, M, W = int(p.L), int(p.M), int(p.window)
    i = int(i)
    if i < L:
        t = i
        hi = i + 1 if p.token_causal else (i // M + 1) * M
        clo = chi = 0
    else:
        t = i - L
        b = t // M
        hi = b * M
        clo, chi = L + b * M, L + (b + 1) * M
    lo = max(0, t - W + 1) if W > 0 else 0
    if hi < lo:
        hi = lo
    return lo, hi, clo, chi


def _groups(p, rows):
    """Rows grouped by identical visible key ranges: {ranges: [rows]}."""
    out = {}
    for i in rows:
        out.setdefault(key_ranges(p, i), []).append(int(i))
    return out


def row_stats(p, q, k, v, dO, b, g, rows):
    """LSE and D of doubled rows `rows` (batch b) for every query head of KV
    head g, over each row's full visible set: arrays [len(rows), G]."""
    G = p.hq // p.hkv
    heads = slice(g * G, (g + 1) * G)
    rows = np.asarray(rows, dtype=np.int64)
    lse = np.full((rows.size, G), -np.inf)
    D = np.zeros((rows.size, G))
    where = {int(r): n for n, r in enumerate(rows)}
    K = _f64(k[b, :, g])
    V = _f64(v[b, :, g])
    for (lo, hi, clo, chi), rs in _groups(p, rows).items():
        if hi <= lo and chi <= clo:
            continue
        # the visible set is two contiguous ranges; their K and V rows back to back
        Kk = torch.cat([K[lo:hi], K[clo:chi]])                 # [n, d]
        Vk = torch.cat([V[lo:hi], V[clo:chi]])
        Q = _f64(q[b, rs][:, heads]).reshape(-1, p.d)          # [rows * G, d]
        s = p.scale * (Q @ Kk.T)                               # [rows * G, n]
        m = s.max(dim=1, keepdim=True).values
        e = torch.exp(s - m)
        den = e.sum(dim=1, keepdim=True)
        l = (m + torch.log(den)).reshape(len(rs), G)
        O = (e @ Vk) / den                                     # softmax(s) V
        dOr = _f64(dO[b, rs][:, heads]).reshape(-1, p.d)
        d_ = (dOr * O).sum(dim=1).reshape(len(rs), G)
        for n, r in enumerate(rs):
            lse[where[r]] = l[n].numpy()
            D[where[r]] = d_[n].numpy()
    return lse, D


def rows_seeing(p, j, rows):
    """The rows among `rows` (doubled positions) whose visible set holds key j."""
    rows = np.asarray(rows, dtype=np.int64)
    sel = []
    for i in rows:
        lo, hi, clo, chi = key_ranges(p, i)
        if lo <= j < hi or clo <= j < chi:
            sel.append(i)
    return np.asarray(sel, dtype=np.int64)


def dkdv_keys(p, q, k, v, dO, b, g, keys, rows, lse, D):
    """dK, dV [len(keys), d] of keys `keys` of KV head g (batch b) over the
    query rows `rows` (the share; doubled positions) with their statistics
    lse, D [len(rows), G] from row_stats."""
    G = p.hq // p.hkv
    heads = slice(g * G, (g + 1) * G)
    rows = np.asarray(rows, dtype=np.int64)
    where = {int(r): n for n, r in enumerate(rows)}
    dk = np.zeros((len(keys), p.d))
    dv = np.zeros((len(keys), p.d))
    for n, j in enumerate(keys):
        rs = rows_seeing(p, int(j), rows)
        if rs.size == 0:
            continue
        at = np.asarray([where[int(r)] for r in rs])
        kj = _f64(k[b, int(j), g])
        vj = _f64(v[b, int(j), g])
        Q = _f64(q[b, rs][:, heads])                           # [r, G, d]
        dOr = _f64(dO[b, rs][:, heads])
        s = p.scale * (Q @ kj)                                 # [r, G]
        P = torch.exp(s - torch.from_numpy(lse[at]))
        dP = dOr @ vj
        dS = P * (dP - torch.from_numpy(D[at]))
        dv[n] = (P[..., None] * dOr).sum(dim=(0, 1)).numpy()
        dk[n] = (p.scale * (dS[..., None] * Q).sum(dim=(0, 1))).numpy()
    return dk, dv
