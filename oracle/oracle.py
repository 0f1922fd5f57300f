"""ctypes wrapper around the fp64 CPU oracle (``bdoracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py``.  The product library never imports
it.

Layout: the doubled input, clean copy at positions [0, L), corrupted copy at
[L, 2L).  ``q``/``dO`` are ``[batch, 2L, hq, d]``, ``k``/``v`` are
``[batch, 2L, hkv, d]``; numpy float32 or uint16 (bf16 bit patterns).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


class Problem(C.Structure):
    _fields_ = [("batch", C.c_int32), ("L", C.c_int32), ("M", C.c_int32),
                ("hq", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32),
                ("token_causal", C.c_int32), ("in_dtype", C.c_int32),
                ("scale", C.c_double), ("window", C.c_int32)]


class Keys(C.Structure):
    _fields_ = [("n_ranges", C.c_int32), ("local", C.c_int32),
                ("lo", C.c_int64 * 2), ("hi", C.c_int64 * 2)]


class Share(C.Structure):
    _fields_ = [("all", C.c_int32), ("n_clean", C.c_int32),
                ("clean_lo", C.c_int64 * 2), ("clean_hi", C.c_int64 * 2),
                ("owned", C.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        P = C.POINTER
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.orc_visible.argtypes = [P(Problem), i64, i64]
        L.orc_visible.restype = C.c_int
        L.orc_num_threads.restype = C.c_int
        L.orc_fwd_rows.argtypes = [P(Problem), P(Keys), vp, vp, vp, i64, vp, vp, vp, vp, vp]
        L.orc_fwd.argtypes = [P(Problem), P(Keys), vp, vp, vp, vp, vp]
        L.orc_dq_rows.argtypes = [P(Problem), P(Keys), P(Keys), vp, vp, vp, vp, i64,
                                  vp, vp, vp, vp, vp, vp]
        L.orc_dkdv_rows.argtypes = [P(Problem), P(Share), P(Keys), P(Keys), vp, vp, vp, vp,
                                    i64, vp, vp, vp, vp, vp]
        L.orc_bwd.argtypes = [P(Problem), P(Share), P(Keys), P(Keys), vp, vp, vp, vp,
                              vp, vp, vp]
        L.orc_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp]
        L.orc_assign_blocks.argtypes = [i32, i32, i32, vp]
        L.orc_assign_blocks.restype = C.c_int
        L.orc_clean_shard.argtypes = [i64, i32, i32, vp, vp]
        L.orc_clean_shard.restype = C.c_int
        _lib = L
    return _lib


def num_threads():
    return lib().orc_num_threads()


def problem(batch, L, M, hq, hkv, d, token_causal=False, bf16=False, scale=None, window=0):
    return Problem(batch, L, M, hq, hkv, d, int(bool(token_causal)), int(bool(bf16)),
                   float(scale) if scale is not None else 1.0 / np.sqrt(d), int(window))


def keys(ranges=None, local=True):
    """Key set of one call: ``ranges`` None → every clean key, else a list of
    at most two half-open clean token ranges; ``local`` adds corrupted keys."""
    k = Keys()
    k.local = int(bool(local))
    if ranges is None:
        k.n_ranges = -1
    else:
        assert len(ranges) <= 2
        k.n_ranges = len(ranges)
        for r, (lo, hi) in enumerate(ranges):
            k.lo[r], k.hi[r] = lo, hi
    return k


def share(L=None, M=None, clean=None, blocks=None):
    """Query rows of a share: ``clean`` list of <= 2 token ranges, ``blocks``
    iterable of owned corrupted blocks.  ``share()`` is every row."""
    s = Share()
    s._owned = None
    if clean is None and blocks is None:
        s.all = 1
        return s
    s.all = 0
    clean = clean or []
    assert len(clean) <= 2
    s.n_clean = len(clean)
    for r, (lo, hi) in enumerate(clean):
        s.clean_lo[r], s.clean_hi[r] = lo, hi
    owned = np.zeros(L // M, dtype=np.uint8)
    if blocks is not None:
        owned[np.asarray(list(blocks), dtype=np.int64)] = 1
    s._owned = owned
    s.owned = owned.ctypes.data
    return s


def _dtype_flag(p, *arrays):
    for a in arrays:
        if p.in_dtype == 1:
            assert a.dtype == np.uint16, a.dtype
        else:
            assert a.dtype == np.float32, a.dtype
        assert a.flags.c_contiguous


def _ptr(a):
    return a.ctypes.data if a is not None else None


def visible(p, i, j):
    return lib().orc_visible(C.byref(p), int(i), int(j))


def fwd(p, ks, q, k, v):
    _dtype_flag(p, q, k, v)
    n2 = 2 * p.L
    o = np.zeros((p.batch, n2, p.hq, p.d))
    lse = np.zeros((p.batch, n2, p.hq))
    lib().orc_fwd(C.byref(p), C.byref(ks), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse))
    return o, lse


def _rows(b, h, i):
    b = np.ascontiguousarray(b, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.int32)
    i = np.ascontiguousarray(i, dtype=np.int64)
    assert b.shape == h.shape == i.shape and b.ndim == 1
    return b, h, i


def fwd_rows(p, ks, q, k, v, b, h, i):
    _dtype_flag(p, q, k, v)
    b, h, i = _rows(b, h, i)
    n = b.shape[0]
    o = np.zeros((n, p.d))
    lse = np.zeros(n)
    lib().orc_fwd_rows(C.byref(p), C.byref(ks), _ptr(q), _ptr(k), _ptr(v), n,
                       _ptr(b), _ptr(h), _ptr(i), _ptr(o), _ptr(lse))
    return o, lse


def dq_rows(p, kn, kg, q, k, v, dO, b, h, i):
    _dtype_flag(p, q, k, v, dO)
    b, h, i = _rows(b, h, i)
    n = b.shape[0]
    dq = np.zeros((n, p.d))
    o = np.zeros((n, p.d))
    lse = np.zeros(n)
    lib().orc_dq_rows(C.byref(p), C.byref(kn), C.byref(kg), _ptr(q), _ptr(k), _ptr(v),
                      _ptr(dO), n, _ptr(b), _ptr(h), _ptr(i), _ptr(dq), _ptr(o), _ptr(lse))
    return dq, o, lse


def dkdv_rows(p, sh, kn, kg, q, k, v, dO, b, g, j):
    _dtype_flag(p, q, k, v, dO)
    b, g, j = _rows(b, g, j)
    n = b.shape[0]
    dk = np.zeros((n, p.d))
    dv = np.zeros((n, p.d))
    lib().orc_dkdv_rows(C.byref(p), C.byref(sh), C.byref(kn), C.byref(kg), _ptr(q), _ptr(k),
                        _ptr(v), _ptr(dO), n, _ptr(b), _ptr(g), _ptr(j), _ptr(dk), _ptr(dv))
    return dk, dv


def bwd(p, sh, kn, kg, q, k, v, dO):
    _dtype_flag(p, q, k, v, dO)
    n2 = 2 * p.L
    dq = np.zeros((p.batch, n2, p.hq, p.d))
    dk = np.zeros((p.batch, n2, p.hkv, p.d))
    dv = np.zeros((p.batch, n2, p.hkv, p.d))
    lib().orc_bwd(C.byref(p), C.byref(sh), C.byref(kn), C.byref(kg), _ptr(q), _ptr(k),
                  _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def merge(o1, z1, o2, z2):
    o1, o2 = (np.ascontiguousarray(x, dtype=np.float64) for x in (o1, o2))
    z1, z2 = (np.ascontiguousarray(x, dtype=np.float64) for x in (z1, z2))
    d = o1.shape[-1]
    n = z1.size
    assert o1.size == n * d and o2.shape == o1.shape and z2.shape == z1.shape
    o = np.zeros_like(o1)
    z = np.zeros_like(z1)
    lib().orc_merge(n, d, _ptr(o1), _ptr(z1), _ptr(o2), _ptr(z2), _ptr(o), _ptr(z))
    return o, z


def assign_blocks(B, P, r):
    out = np.zeros(max(B // max(P, 1), 1), dtype=np.int32)
    n = lib().orc_assign_blocks(B, P, r, _ptr(out))
    if n < 0:
        raise ValueError("invalid (B, P, r)")
    return out[:n]


def clean_shard(L, P, s):
    lo = np.zeros(2, dtype=np.int64)
    hi = np.zeros(2, dtype=np.int64)
    n = lib().orc_clean_shard(L, P, s, _ptr(lo), _ptr(hi))
    if n < 0:
        raise ValueError("invalid (L, P, s)")
    return [(int(lo[r]), int(hi[r])) for r in range(n)]
