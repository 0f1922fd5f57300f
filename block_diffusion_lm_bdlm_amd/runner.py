"""Device-memory plumbing around the C ABI for the two call patterns.

* whole mask: one bdattn_fwd / bdattn_bwd launch over the doubled input
  ``[batch, 2L, heads, d]`` (clean copy first), the single structured-mask
  call per layer of the Turbo-dLLM page ("Block Diffusion Optimizations").
* CSBP share: one rank's blocks B_r (and optionally its clean shard of query
  rows) attended first against their own corrupted keys, then against the
  clean key shards one at a time, each partial merged by log-sum-exp
  ("CSBP 完全拆解", section "在线 softmax 合并", steps 2-4 of the schedule);
  the backward reuses the final O and LSE for every call (step 5, local part).

Only allocation and argument marshalling live here; all arithmetic runs in
libbdattn's kernels.
"""
from dataclasses import dataclass, field

import torch

from . import bdattn as B


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def dtype_code(t):
    return B.BDATTN_F32 if t.dtype == torch.float32 else B.BDATTN_BF16


# ------------------------------------------------------------------ whole mask
@dataclass
class WholeMask:
    batch: int
    L: int
    M: int
    hq: int
    hkv: int
    d: int
    dtype: int = B.BDATTN_BF16
    clean_mask: int = B.BDATTN_CLEAN_BLOCK_CAUSAL
    scale: float = 0.0
    window: int = 0  # clean-key sliding window in tokens; 0 = none

    def __post_init__(self):
        self.prob = B.problem(self.batch, self.L, self.M, self.hq, self.hkv, self.d, self.dtype,
                              self.clean_mask, self.scale, self.window)
        self.share = B.share(range(self.L // self.M), [(0, self.L)])
        self.kv = B.kv([(0, self.L)], True)

    def workspace(self, bwd, device):
        return _ws(B.bdattn_workspace_bytes(self.prob, self.share, self.kv, bwd), device)

    def fwd(self, q, k, v, o_dtype=None, ws=None, stream=None):
        """q [batch, 2L, hq, d], k/v [batch, 2L, hkv, d] -> O [batch, 2L, hq, d], LSE [batch, 2L, hq]."""
        L = self.L
        if o_dtype is None:
            o_dtype = torch.float32 if self.dtype == B.BDATTN_F32 else torch.bfloat16
        o = torch.empty(q.shape, dtype=o_dtype, device=q.device)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.workspace(False, q.device)
        B.bdattn_fwd(self.prob, self.share, self.kv, q[:, :L], q[:, L:], k[:, :L], v[:, :L], k[:, L:], v[:, L:],
                     o, dtype_code(o), lse, ws, stream)
        return o, lse

    def bwd(self, q, k, v, o, lse, do, ws=None, stream=None, grads=None, overwrite=False):
        """-> dq [batch, 2L, hq, d] fp32, dk, dv [batch, 2L, hkv, d] fp32.
        overwrite: the kernels write the gradients instead of adding to
        them (``grads`` then need no zeroing)."""
        L, dev = self.L, q.device
        if grads is None:
            grads = self.alloc_grads(dev)
        dq, dkc, dvc, dkx, dvx, delta = grads
        if ws is None:
            ws = self.workspace(True, dev)
        flags = B.BDATTN_BWD_OVERWRITE if overwrite else 0
        B.bdattn_bwd(self.prob, self.share, self.kv, q[:, :L], q[:, L:], k[:, :L], v[:, :L], k[:, L:], v[:, L:],
                     o, dtype_code(o), lse, do, delta, flags, dq, dkc, dvc, dkx, dvx, ws, stream)
        return dq, torch.cat([dkc, dkx], 1), torch.cat([dvc, dvx], 1)

    def alloc_grads(self, dev):
        n2 = 2 * self.L
        f = torch.float32
        dq = torch.zeros(self.batch, n2, self.hq, self.d, dtype=f, device=dev)
        kv_shape = (self.batch, self.L, self.hkv, self.d)
        dkc, dvc, dkx, dvx = (torch.zeros(kv_shape, dtype=f, device=dev) for _ in range(4))
        delta = torch.empty(self.batch, n2, self.hq, dtype=f, device=dev)
        return dq, dkc, dvc, dkx, dvx, delta


# ------------------------------------------------------------------ CSBP share
@dataclass
class CsbpShare:
    """One rank's share: blocks (sorted), optional clean query ranges, and
    the clean key shards streamed one at a time."""
    batch: int
    L: int
    M: int
    hq: int
    hkv: int
    d: int
    blocks: list
    clean_q: list = field(default_factory=list)
    shards: list = field(default_factory=list)  # list of lists of (lo, hi) clean key ranges
    scale: float = 0.0
    window: int = 0  # clean-key sliding window in tokens; 0 = none

    def __post_init__(self):
        self.prob = B.problem(self.batch, self.L, self.M, self.hq, self.hkv, self.d, B.BDATTN_BF16,
                              B.BDATTN_CLEAN_BLOCK_CAUSAL, self.scale, self.window)
        self.share = B.share(self.blocks, self.clean_q)
        self.kv_local = B.kv([], True)
        self.kv_shards = [B.kv(s, False) for s in self.shards]
        self.n_clean = sum(hi - lo for lo, hi in self.clean_q)
        self.R = self.n_clean + len(self.blocks) * self.M

    def workspace(self, bwd, device):
        n = max(B.bdattn_workspace_bytes(self.prob, self.share, k, bwd) for k in [self.kv_local] + self.kv_shards)
        return _ws(n, device)

    def fwd(self, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, ws=None, stream=None):
        """q_clean [b, n_clean, hq, d] (share clean rows), q_corr/k_corr/v_corr packed corrupted rows,
        k_clean/v_clean [b, L, hkv, d].  -> (O fp32 merged, LSE, O bf16)."""
        dev = k_clean.device
        rows = (self.batch, self.R, self.hq)
        o_acc = torch.empty(*rows, self.d, dtype=torch.float32, device=dev)
        lse_acc = torch.empty(rows, dtype=torch.float32, device=dev)
        o_part = torch.empty_like(o_acc)
        lse_part = torch.empty_like(lse_acc)
        o_bf16 = torch.empty(*rows, self.d, dtype=torch.bfloat16, device=dev)
        if ws is None:
            ws = self.workspace(False, dev)
        B.bdattn_fwd(self.prob, self.share, self.kv_local, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr,
                     o_acc, B.BDATTN_F32, lse_acc, ws, stream)
        nrows = self.batch * self.R * self.hq
        for i, kvs in enumerate(self.kv_shards):
            B.bdattn_fwd(self.prob, self.share, kvs, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr,
                         o_part, B.BDATTN_F32, lse_part, ws, stream)
            last = i == len(self.kv_shards) - 1
            B.bdattn_shard_merge(nrows, self.d, o_acc, lse_acc, o_part, lse_part, o_bf16 if last else None, stream)
        if not self.kv_shards:
            o_bf16.copy_(o_acc)
        return o_acc, lse_acc, o_bf16

    def alloc_grads(self, dev):
        f = torch.float32
        dq = torch.zeros(self.batch, self.R, self.hq, self.d, dtype=f, device=dev)
        dkc = torch.zeros(self.batch, self.L, self.hkv, self.d, dtype=f, device=dev)
        dvc = torch.zeros_like(dkc)
        nx = len(self.blocks) * self.M
        dkx = torch.zeros(self.batch, nx, self.hkv, self.d, dtype=f, device=dev)
        dvx = torch.zeros_like(dkx)
        delta = torch.empty(self.batch, self.R, self.hq, dtype=f, device=dev)
        return dq, dkc, dvc, dkx, dvx, delta

    def bwd(self, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, o, lse, do, ws=None, stream=None,
            grads=None):
        dev = k_clean.device
        if grads is None:
            grads = self.alloc_grads(dev)
        dq, dkc, dvc, dkx, dvx, delta = grads
        if ws is None:
            ws = self.workspace(True, dev)
        od = dtype_code(o)
        B.bdattn_bwd(self.prob, self.share, self.kv_local, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr,
                     o, od, lse, do, delta, 0, dq, dkc, dvc, dkx, dvx, ws, stream)
        for kvs in self.kv_shards:
            B.bdattn_bwd(self.prob, self.share, kvs, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr,
                         o, od, lse, do, delta, 1, dq, dkc, dvc, dkx, dvx, ws, stream)
        return grads
