"""ctypes binding of libbdattn (include/bdattn.h): same names, argument
marshalling only.  Every step of the computation runs in the library's HIP
kernels; PyTorch only provides device memory and streams.

Importing this module never builds anything; ``lib()`` raises if the shared
library is missing, so the product path fails loudly instead of falling back.
"""
import ctypes as C
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbdattn.so")

BDATTN_OK, BDATTN_EINVAL, BDATTN_ENOTSUP, BDATTN_EHIP, BDATTN_EWORKSPACE = 0, -1, -2, -3, -4
BDATTN_ERANGE, BDATTN_ESCRATCH = -5, -6
BDATTN_STATIC_SCRATCH_BYTES = 256 << 20
BDATTN_BF16, BDATTN_F32 = 0, 1
BDATTN_CLEAN_BLOCK_CAUSAL, BDATTN_CLEAN_TOKEN_CAUSAL = 0, 1
BDATTN_BWD_DELTA_READY, BDATTN_BWD_OVERWRITE = 1, 2
BDATTN_MAX_RUNS = 8


class Problem(C.Structure):
    _fields_ = [("batch", C.c_int32), ("L", C.c_int32), ("M", C.c_int32), ("hq", C.c_int32),
                ("hkv", C.c_int32), ("d", C.c_int32), ("dtype", C.c_int32),
                ("clean_mask", C.c_int32), ("scale", C.c_float), ("window", C.c_int32)]


class Share(C.Structure):
    _fields_ = [("blocks", C.POINTER(C.c_int32)), ("n_blocks", C.c_int32), ("n_clean", C.c_int32),
                ("clean_lo", C.c_int32 * 2), ("clean_hi", C.c_int32 * 2)]


class KV(C.Structure):
    _fields_ = [("n", C.c_int32), ("lo", C.c_int32 * 2), ("hi", C.c_int32 * 2),
                ("include_local", C.c_int32)]


class Tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("batch_stride", C.c_int64), ("row_stride", C.c_int64),
                ("head_stride", C.c_int64)]


class BdattnError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {bdattn_status_string(status)} ({status})")
        self.status = status


_lib = None
EXPORTS = ("bdattn_assign_blocks", "bdattn_clean_shard", "bdattn_plan_order", "bdattn_plan_order_keys",
           "bdattn_workspace_bytes", "bdattn_fwd", "bdattn_fwd_static", "bdattn_shard_merge", "bdattn_bwd",
           "bdattn_workspace_status", "bdattn_status_string", "bdattn_profile_enable",
           "bdattn_profile_read")


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libbdattn.so not built ({LIB_PATH}); run __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    P, vp, i32, i64 = C.POINTER, C.c_void_p, C.c_int32, C.c_int64
    L.bdattn_assign_blocks.argtypes = [i32, i32, i32, P(C.c_int32)]
    L.bdattn_clean_shard.argtypes = [i32, i32, i32, P(KV)]
    L.bdattn_plan_order.argtypes = [P(Problem), P(Share), P(KV), P(C.c_int32), i64, P(C.c_int64)]
    L.bdattn_plan_order_keys.argtypes = [P(Problem), P(Share), P(KV), P(C.c_int32), i64, P(C.c_int64)]
    L.bdattn_workspace_status.argtypes = [vp, vp]
    L.bdattn_workspace_bytes.argtypes = [P(Problem), P(Share), P(KV), C.c_int]
    L.bdattn_workspace_bytes.restype = C.c_size_t
    L.bdattn_fwd.argtypes = [P(Problem), P(Share), P(KV)] + [Tensor] * 7 + [i32, vp, vp, C.c_size_t, vp]
    L.bdattn_fwd_static.argtypes = [P(Problem), P(Share), P(KV)] + [Tensor] * 7 + [i32, vp, vp]
    L.bdattn_shard_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp]
    L.bdattn_bwd.argtypes = ([P(Problem), P(Share), P(KV)] + [Tensor] * 7 + [i32, vp, Tensor, vp, i32]
                             + [vp] * 5 + [vp, C.c_size_t, vp])
    L.bdattn_status_string.argtypes = [C.c_int]
    L.bdattn_status_string.restype = C.c_char_p
    L.bdattn_profile_enable.argtypes = [C.c_int]
    L.bdattn_profile_read.argtypes = [P(C.c_char_p), P(C.c_int64), P(C.c_double), i32, P(C.c_int32)]
    for name in EXPORTS:
        getattr(L, name).restype = getattr(L, name).restype if name in (
            "bdattn_workspace_bytes", "bdattn_status_string") else C.c_int
    _lib = L
    return L


def _check(status, what):
    if status != BDATTN_OK:
        raise BdattnError(status, what)
    return status


# ------------------------------------------------------------------ builders
def problem(batch, L, M, hq, hkv, d, dtype=BDATTN_BF16, clean_mask=BDATTN_CLEAN_BLOCK_CAUSAL, scale=0.0,
            window=0):
    return Problem(batch, L, M, hq, hkv, d, dtype, clean_mask, scale, window)


def share(blocks=(), clean=()):
    """Share of sorted corrupted ``blocks`` and <= 2 clean token ranges."""
    arr = np.ascontiguousarray(np.asarray(list(blocks) if not isinstance(blocks, np.ndarray) else blocks,
                                          dtype=np.int32))
    s = Share()
    s._arr = arr  # keep the host block list alive with the struct
    s.blocks = arr.ctypes.data_as(C.POINTER(C.c_int32)) if arr.size else None
    s.n_blocks = int(arr.size)
    s.n_clean = len(clean)
    for r, (lo, hi) in enumerate(clean):
        s.clean_lo[r], s.clean_hi[r] = int(lo), int(hi)
    return s


def kv(ranges=(), include_local=False):
    k = KV()
    k.n = len(ranges)
    for r, (lo, hi) in enumerate(ranges):
        k.lo[r], k.hi[r] = int(lo), int(hi)
    k.include_local = int(bool(include_local))
    return k


def tensor(t):
    """bdattn_tensor of a [batch, rows, heads, d] torch view (None -> null)."""
    if t is None:
        return Tensor(None, 0, 0, 0)
    assert t.dim() == 4 and t.stride(3) == 1, "need [batch, rows, heads, d] with d contiguous"
    return Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ------------------------------------------------------------------ entry points
def bdattn_status_string(status):
    return lib().bdattn_status_string(int(status)).decode()


def bdattn_assign_blocks(B, P, r):
    out = np.zeros(max(B // max(P, 1), 1), dtype=np.int32)
    _check(lib().bdattn_assign_blocks(B, P, r, out.ctypes.data_as(C.POINTER(C.c_int32))), "bdattn_assign_blocks")
    return out[: B // P]


def bdattn_clean_shard(L, P, s):
    out = KV()
    _check(lib().bdattn_clean_shard(L, P, s, C.byref(out)), "bdattn_clean_shard")
    return out


def _order(fn, name, prob, sh, kvs):
    n = C.c_int64(0)
    _check(fn(C.byref(prob), C.byref(sh), C.byref(kvs), None, 0, C.byref(n)), name)
    items = np.zeros(4 * n.value, dtype=np.int32)
    _check(fn(C.byref(prob), C.byref(sh), C.byref(kvs), items.ctypes.data_as(C.POINTER(C.c_int32)), items.size,
              C.byref(n)), name)
    return items.reshape(-1, 4)


def bdattn_plan_order(prob, sh, kvs):
    """Query-major order: rows (batch, query head, tile, tile or -1)."""
    return _order(lib().bdattn_plan_order, "bdattn_plan_order", prob, sh, kvs)


def bdattn_plan_order_keys(prob, sh, kvs):
    """Key-major order: rows (batch, KV head, key tile, key tile or -1)."""
    return _order(lib().bdattn_plan_order_keys, "bdattn_plan_order_keys", prob, sh, kvs)


def bdattn_workspace_status(workspace, stream=None):
    """BDATTN_OK or BDATTN_ERANGE for the last call that used ``workspace``
    (synchronises the stream); raises on other errors."""
    st = lib().bdattn_workspace_status(_p(workspace), _stream(stream))
    if st not in (BDATTN_OK, BDATTN_ERANGE):
        _check(st, "bdattn_workspace_status")
    return st


def bdattn_workspace_bytes(prob, sh, kvs, bwd):
    return int(lib().bdattn_workspace_bytes(C.byref(prob), C.byref(sh), C.byref(kvs), int(bool(bwd))))


def bdattn_fwd(prob, sh, kvs, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse,
               workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return _check(lib().bdattn_fwd(C.byref(prob), C.byref(sh), C.byref(kvs), tensor(q_clean), tensor(q_corr),
                                   tensor(k_clean), tensor(v_clean), tensor(k_corr), tensor(v_corr),
                                   tensor(o), o_dtype, _p(lse), _p(workspace), ws_bytes, _stream(stream)),
                  "bdattn_fwd")


def bdattn_fwd_static(prob, sh, kvs, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse,
                      stream=None):
    """bdattn_fwd with the library's static device scratch (no workspace)."""
    return _check(lib().bdattn_fwd_static(C.byref(prob), C.byref(sh), C.byref(kvs), tensor(q_clean),
                                          tensor(q_corr), tensor(k_clean), tensor(v_clean), tensor(k_corr),
                                          tensor(v_corr), tensor(o), o_dtype, _p(lse), _stream(stream)),
                  "bdattn_fwd_static")


def bdattn_shard_merge(rows, d, o_acc, lse_acc, o_part, lse_part, o_final_bf16=None, stream=None):
    return _check(lib().bdattn_shard_merge(int(rows), int(d), _p(o_acc), _p(lse_acc), _p(o_part), _p(lse_part),
                                           _p(o_final_bf16), _stream(stream)), "bdattn_shard_merge")


def bdattn_bwd(prob, sh, kvs, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, o_final, o_dtype, lse_final,
               d_o, delta, flags, dq_acc, dk_clean_acc, dv_clean_acc, dk_corr_acc, dv_corr_acc,
               workspace, stream=None):
    """flags: BDATTN_BWD_DELTA_READY and/or BDATTN_BWD_OVERWRITE (a bool is
    read as the delta-ready flag alone)."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return _check(lib().bdattn_bwd(C.byref(prob), C.byref(sh), C.byref(kvs), tensor(q_clean), tensor(q_corr),
                                   tensor(k_clean), tensor(v_clean), tensor(k_corr), tensor(v_corr),
                                   tensor(o_final), o_dtype, _p(lse_final), tensor(d_o), _p(delta),
                                   int(flags), _p(dq_acc), _p(dk_clean_acc), _p(dv_clean_acc),
                                   _p(dk_corr_acc), _p(dv_corr_acc), _p(workspace), ws_bytes,
                                   _stream(stream)), "bdattn_bwd")


def bdattn_profile_enable(enable=True):
    return _check(lib().bdattn_profile_enable(int(bool(enable))), "bdattn_profile_enable")


def bdattn_profile_read():
    cap = 16
    names = (C.c_char_p * cap)()
    counts = (C.c_int64 * cap)()
    ms = (C.c_double * cap)()
    n = C.c_int32(0)
    _check(lib().bdattn_profile_read(names, counts, ms, cap, C.byref(n)), "bdattn_profile_read")
    return {names[i].decode(): (int(counts[i]), float(ms[i])) for i in range(n.value)}
