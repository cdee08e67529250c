"""ctypes binding of libkdchunk.so (argument marshalling only).

Every step of the loss runs in the HIP library; this module converts torch
tensors (or raw integer device addresses) to pointers, passes the current HIP
stream, and turns non-zero status codes into exceptions.  There is no
fallback: if the library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDCHUNK_LIB names another build of the same library (e.g. the host
# sanitizer build the ABI tests run under); default: the in-tree build
LIB_PATH = os.environ.get("KDCHUNK_LIB") or os.path.join(_HERE, "libkdchunk.so")

KD_OK, KD_ERR_NULL, KD_ERR_SHAPE, KD_ERR_DTYPE, KD_ERR_ALIGN, KD_ERR_WORKSPACE, KD_ERR_DEVICE, \
    KD_ERR_LAUNCH = range(8)
KD_F32, KD_BF16 = 0, 1

# names declared by include/kd_chunked.h and include/kd_profile.h
EXPORTS = ("kd_chunked_workspace_size", "kd_status_string", "kd_chunked_fwd", "kd_chunked_bwd",
           "kd_chunked_fwd_bwd_workspace_size", "kd_chunked_fwd_bwd", "kd_teacher_topk_workspace_size",
           "kd_teacher_topk", "kd_chunked_validate", "kd_profile_enable", "kd_profile_read",
           "kd_chunked_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20  # KD_NOALLOC_SCRATCH_BYTES of include/kd_chunked.h
KD_K_COUNT = 15


class KDError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kd_status_string(status)} (status {status})")
        self.status = status


class KDProblem(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("d", ctypes.c_int32), ("v", ctypes.c_int32),
                ("k", ctypes.c_int32), ("chunk", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("t_dtype", ctypes.c_int32), ("tau", ctypes.c_float), ("dw_chunks", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkdchunk.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m chunked_kl_loss_row_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER(KDProblem)
        L.kd_chunked_workspace_size.argtypes = [P]
        L.kd_chunked_workspace_size.restype = ctypes.c_size_t
        L.kd_status_string.argtypes = [ctypes.c_int]
        L.kd_status_string.restype = ctypes.c_char_p
        L.kd_chunked_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.kd_chunked_fwd.restype = ctypes.c_int
        L.kd_chunked_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.kd_chunked_fwd_noalloc.restype = ctypes.c_int
        L.kd_chunked_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.kd_chunked_bwd.restype = ctypes.c_int
        L.kd_chunked_fwd_bwd_workspace_size.argtypes = [P]
        L.kd_chunked_fwd_bwd_workspace_size.restype = ctypes.c_size_t
        L.kd_chunked_fwd_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.kd_chunked_fwd_bwd.restype = ctypes.c_int
        L.kd_teacher_topk_workspace_size.argtypes = [P]
        L.kd_teacher_topk_workspace_size.restype = ctypes.c_size_t
        L.kd_teacher_topk.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.kd_teacher_topk.restype = ctypes.c_int
        L.kd_chunked_validate.argtypes = [P, vp, vp, vp, vp]
        L.kd_chunked_validate.restype = ctypes.c_int
        L.kd_profile_enable.argtypes = [ctypes.c_int]
        L.kd_profile_enable.restype = ctypes.c_int
        L.kd_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                      ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.kd_profile_read.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass workspace_bytes explicitly with a raw workspace address")
    return x.numel() * x.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def problem(n: int, d: int, v: int, k: int, chunk: int, x_dtype: int = KD_BF16,
            t_dtype: Optional[int] = None, tau: float = 1.0, dw_chunks: int = 1) -> KDProblem:
    return KDProblem(int(n), int(d), int(v), int(k), int(chunk), int(x_dtype),
                     int(x_dtype if t_dtype is None else t_dtype), float(tau), int(dw_chunks))


def kd_status_string(status: int) -> str:
    return lib().kd_status_string(int(status)).decode()


def kd_chunked_workspace_size(prob: KDProblem) -> int:
    return int(lib().kd_chunked_workspace_size(ctypes.byref(prob)))


def kd_chunked_fwd(prob: KDProblem, H, W, t_ids, t_logits, mask, loss, lse, row_loss=None, zg=None,
                   workspace=None, workspace_bytes: Optional[int] = None, stream=None,
                   check: bool = True) -> int:
    """Enqueue the forward (see include/kd_chunked.h).  Returns the status;
    raises KDError on a non-zero status when ``check`` is true."""
    wsb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    st = lib().kd_chunked_fwd(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(t_ids), _ptr(t_logits),
                              _ptr(mask), _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(zg),
                              _ptr(workspace), wsb, _stream(stream))
    if check and st != KD_OK:
        raise KDError(st, "kd_chunked_fwd")
    return st


def kd_chunked_fwd_noalloc(prob: KDProblem, H, W, t_ids, t_logits, mask, loss, lse, row_loss=None, zg=None,
                           stream=None, check: bool = True) -> int:
    """Enqueue the forward with the library's own device scratch instead of a
    workspace (see include/kd_chunked.h); allocates nothing."""
    st = lib().kd_chunked_fwd_noalloc(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(t_ids), _ptr(t_logits),
                                      _ptr(mask), _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(zg),
                                      _stream(stream))
    if check and st != KD_OK:
        raise KDError(st, "kd_chunked_fwd_noalloc")
    return st


def kd_chunked_bwd(prob: KDProblem, H, W, t_ids, t_logits, mask, lse, grad_loss, dH, dW,
                   workspace=None, workspace_bytes: Optional[int] = None, stream=None,
                   check: bool = True) -> int:
    """Enqueue the backward (see include/kd_chunked.h)."""
    wsb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    st = lib().kd_chunked_bwd(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(t_ids), _ptr(t_logits),
                              _ptr(mask), _ptr(lse), _ptr(grad_loss), _ptr(dH), _ptr(dW),
                              _ptr(workspace), wsb, _stream(stream))
    if check and st != KD_OK:
        raise KDError(st, "kd_chunked_bwd")
    return st


def kd_chunked_validate(prob: KDProblem, t_ids, mask, out, stream=None, check: bool = True) -> int:
    """Enqueue the teacher-record check (see include/kd_chunked.h); ``out``
    is an int64 [4] device buffer."""
    st = lib().kd_chunked_validate(ctypes.byref(prob), _ptr(t_ids), _ptr(mask), _ptr(out), _stream(stream))
    if check and st != KD_OK:
        raise KDError(st, "kd_chunked_validate")
    return st


def kd_chunked_fwd_bwd_workspace_size(prob: KDProblem) -> int:
    return int(lib().kd_chunked_fwd_bwd_workspace_size(ctypes.byref(prob)))


def kd_chunked_fwd_bwd(prob: KDProblem, H, W, t_ids, t_logits, mask, grad_loss, loss, lse, dH, dW,
                       workspace=None, workspace_bytes: Optional[int] = None, stream=None,
                       check: bool = True) -> int:
    """Enqueue forward + backward in one call (see include/kd_chunked.h)."""
    wsb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    st = lib().kd_chunked_fwd_bwd(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(t_ids), _ptr(t_logits),
                                  _ptr(mask), _ptr(grad_loss), _ptr(loss), _ptr(lse), _ptr(dH), _ptr(dW),
                                  _ptr(workspace), wsb, _stream(stream))
    if check and st != KD_OK:
        raise KDError(st, "kd_chunked_fwd_bwd")
    return st


def kd_teacher_topk_workspace_size(prob: KDProblem) -> int:
    return int(lib().kd_teacher_topk_workspace_size(ctypes.byref(prob)))


def kd_teacher_topk(prob: KDProblem, H, W, ids, logits, overflow_rows=None, workspace=None,
                    workspace_bytes: Optional[int] = None, stream=None, check: bool = True) -> int:
    """Enqueue the teacher top-K producer (see include/kd_topk.h)."""
    wsb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    st = lib().kd_teacher_topk(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(ids), _ptr(logits), _ptr(overflow_rows),
                               _ptr(workspace), wsb, _stream(stream))
    if check and st != KD_OK:
        raise KDError(st, "kd_teacher_topk")
    return st


def kd_profile_enable(on: bool) -> int:
    """Record HIP events around every kernel the library enqueues (see
    include/kd_profile.h); clears the accumulated totals."""
    return int(lib().kd_profile_enable(1 if on else 0))


def kd_profile_read(kind: int):
    """(name, total_ms, launches) of kernel kind ``kind`` since the last enable."""
    name = ctypes.c_char_p()
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    st = lib().kd_profile_read(int(kind), ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n))
    if st != KD_OK:
        raise KDError(st, "kd_profile_read")
    return name.value.decode(), ms.value, n.value


def kd_profile_all() -> dict:
    """{name: (total_ms, launches)} for every kernel kind."""
    out = {}
    for k in range(KD_K_COUNT):
        name, ms, n = kd_profile_read(k)
        out[name] = (ms, n)
    return out
