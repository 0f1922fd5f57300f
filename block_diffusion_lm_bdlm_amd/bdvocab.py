"""ctypes binding of libbdvocab (include/bdvocab.h): same names, argument
marshalling only.  Every step of the vocabulary loss runs in the library
(hand-written HIP kernels plus hipBLASLt GEMMs); PyTorch only provides
device memory and streams.

Importing this module never builds anything; ``lib()`` raises if the shared
library is missing, so the product path fails loudly instead of falling back.
"""
import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbdvocab.so")

BDVOCAB_OK, BDVOCAB_EINVAL, BDVOCAB_ENOTSUP, BDVOCAB_EHIP, BDVOCAB_EWORKSPACE, BDVOCAB_EBLAS = 0, -1, -2, -3, -4, -5
BDVOCAB_BF16, BDVOCAB_F32 = 0, 1
BDVOCAB_WS_ROW_LIST, BDVOCAB_WS_HEAD_GRAD = 1, 2

EXPORTS = ("bdvocab_workspace_bytes", "bdvocab_loss", "bdvocab_tune", "bdvocab_status_string",
           "bdvocab_profile_enable", "bdvocab_profile_read")


class Problem(C.Structure):
    _fields_ = [("n_rows", C.c_int64), ("vocab", C.c_int32), ("hidden", C.c_int32), ("chunk", C.c_int32),
                ("dh_dtype", C.c_int32)]


class BdvocabError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {bdvocab_status_string(status)} ({status})")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libbdvocab.so not built ({LIB_PATH}); run __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32, P = C.c_void_p, C.c_int64, C.c_int32, C.POINTER
    L.bdvocab_workspace_bytes.argtypes = [P(Problem), C.c_int]
    L.bdvocab_workspace_bytes.restype = C.c_size_t
    L.bdvocab_loss.argtypes = [P(Problem), vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, C.c_size_t, vp]
    L.bdvocab_loss.restype = C.c_int
    L.bdvocab_tune.argtypes = [P(Problem), C.c_int, vp, i64, vp, i64, vp, C.c_size_t, vp]
    L.bdvocab_tune.restype = C.c_int
    L.bdvocab_status_string.argtypes = [C.c_int]
    L.bdvocab_status_string.restype = C.c_char_p
    L.bdvocab_profile_enable.argtypes = [C.c_int]
    L.bdvocab_profile_enable.restype = C.c_int
    L.bdvocab_profile_read.argtypes = [P(C.c_char_p), P(C.c_int64), P(C.c_double), i32, P(C.c_int32)]
    L.bdvocab_profile_read.restype = C.c_int
    _lib = L
    return L


def _check(status, what):
    if status != BDVOCAB_OK:
        raise BdvocabError(status, what)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def problem(n_rows, vocab, hidden, chunk=0, dh_dtype=BDVOCAB_BF16):
    return Problem(int(n_rows), int(vocab), int(hidden), int(chunk), int(dh_dtype))


def bdvocab_status_string(status):
    return lib().bdvocab_status_string(int(status)).decode()


def bdvocab_workspace_bytes(prob, row_list, head_grad=False):
    flags = (BDVOCAB_WS_ROW_LIST if row_list else 0) | (BDVOCAB_WS_HEAD_GRAD if head_grad else 0)
    return int(lib().bdvocab_workspace_bytes(C.byref(prob), flags))


def bdvocab_loss(prob, h, h_stride, w_head, rows, targets, weights, lse, loss, loss_sum, dh, dh_stride, dw,
                 workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bdvocab_loss(C.byref(prob), _p(h), int(h_stride), _p(w_head), _p(rows), _p(targets), _p(weights),
                              _p(lse), _p(loss), _p(loss_sum), _p(dh), int(dh_stride), _p(dw), _p(workspace),
                              ws_bytes, _stream(stream)), "bdvocab_loss")


def bdvocab_tune(prob, flags, h, h_stride, w_head, dh_stride, workspace, stream=None):
    """Times the GEMM candidates for the shapes of matching bdvocab_loss calls
    (set-up call: synchronises the stream)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bdvocab_tune(C.byref(prob), int(flags), _p(h), int(h_stride), _p(w_head), int(dh_stride),
                              _p(workspace), ws_bytes, _stream(stream)), "bdvocab_tune")


def bdvocab_profile_enable(enable=True):
    _check(lib().bdvocab_profile_enable(1 if enable else 0), "bdvocab_profile_enable")


def bdvocab_profile_read():
    """{kind name: (launches, total ms)} of the launches recorded since the
    last read."""
    cap = 8
    names = (C.c_char_p * cap)()
    counts = (C.c_int64 * cap)()
    ms = (C.c_double * cap)()
    n = C.c_int32(0)
    _check(lib().bdvocab_profile_read(names, counts, ms, cap, C.byref(n)), "bdvocab_profile_read")
    return {names[i].decode(): (int(counts[i]), float(ms[i])) for i in range(n.value)}


class VocabLoss:
    """Owns the workspace for repeated calls of one problem shape."""

    def __init__(self, n_rows, vocab, hidden, chunk=0, dh_dtype=BDVOCAB_BF16, row_list=False, head_grad=False,
                 device="cuda"):
        import torch
        self.prob = problem(n_rows, vocab, hidden, chunk, dh_dtype)
        nbytes = bdvocab_workspace_bytes(self.prob, row_list, head_grad)
        self.head_grad = head_grad
        if nbytes == 0:
            raise BdvocabError(BDVOCAB_EINVAL, "bdvocab_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.row_list = row_list

    def tune(self, h, w_head, dh_stride=0, stream=None):
        """Times the GEMM candidates for this workspace's calls (dh_stride: the
        calls' dh row stride, 0 when they pass no dh)."""
        flags = (BDVOCAB_WS_ROW_LIST if self.row_list else 0) | (BDVOCAB_WS_HEAD_GRAD if self.head_grad else 0)
        bdvocab_tune(self.prob, flags, h, h.stride(0), w_head, dh_stride, self.workspace, stream)

    def __call__(self, h, w_head, targets, weights=None, rows=None, dh=None, lse=None, loss=None, loss_sum=None,
                 dw=None, stream=None):
        """Fills ``loss`` (allocated when None), ``lse``, ``loss_sum`` and
        ``dh`` (rows written in place), adds the head gradient to ``dw``
        (fp32 [V, d]) when given, and returns (loss, lse, loss_sum, dh)."""
        import torch
        R = self.prob.n_rows
        if (rows is not None) != self.row_list:
            raise ValueError("row list presence differs from the workspace's")
        if dw is not None and not self.head_grad:
            raise ValueError("dw needs a workspace made with head_grad=True")
        if loss is None:
            loss = torch.empty(R, dtype=torch.float32, device=h.device)
        bdvocab_loss(self.prob, h, h.stride(0), w_head, rows, targets, weights, lse, loss, loss_sum, dh,
                     0 if dh is None else dh.stride(0), dw, self.workspace, stream)
        return loss, lse, loss_sum, dh
