"""Python binding of the MI355X Q8_0 decode matvec library (libq8gemv.so).

Argument marshalling only: tensors become device pointers, torch streams
become hipStream_t handles, and every computation happens in the HIP
kernels behind the C ABI declared in include/q8gemv.h.  There is no other
implementation: if the library is missing, importing this package raises.

The names follow the C ABI:
    gemv(x, w, y=None, stream=None)            -> q8_0_gemv
    gemm_smallm(X, w, Y=None, stream=None)     -> q8_0_gemm_smallm
    Chain(ops, fuse=True) .run(mode, stream)   -> q8_0_chain_create / q8_0_decode_chain
    stream_wait(stream, timeout_ms)            -> q8_0_stream_wait
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libq8gemv.so")

Q8_OK = 0
Q8_ERR_INVALID_ARG = -1
Q8_ERR_SHAPE = -2
Q8_ERR_ALIGN = -3
Q8_ERR_ALIAS = -4
Q8_ERR_NO_DEVICE = -5
Q8_ERR_HIP = -6
Q8_ERR_TIMEOUT = -7
Q8_ERR_UNSUPPORTED = -8

Q8_CHAIN_FUSE = 0
Q8_CHAIN_PER_OP = 1
MODE_GRAPH = 0
MODE_EAGER = 1
MODE_SYNC_EACH = 2

BLOCK_QUANTS = 32
BLOCK_BYTES = 34

EXPORTS = ("q8_0_gemv", "q8_0_gemm_smallm", "q8_0_chain_create", "q8_0_decode_chain",
           "q8_0_chain_launches", "q8_0_chain_destroy", "q8_0_stream_wait",
           "q8_0_status_string", "q8_0_last_error")


class Q8Error(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        super().__init__("%s (%d): %s" % (_status_string(code), code, detail))


class Q8Op(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("p", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIBRARY):
        raise ImportError("libq8gemv.so is not built; run __graft_entry__.build() "
                          "or python q8_block_quantized_gemv_amd/build.py")
    lib = ctypes.CDLL(LIBRARY)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q8_0_gemv.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.q8_0_gemm_smallm.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.q8_0_chain_create.argtypes = [ctypes.POINTER(Q8Op), i64, ctypes.c_uint32,
                                      ctypes.POINTER(vp)]
    lib.q8_0_decode_chain.argtypes = [vp, ctypes.c_int, vp]
    lib.q8_0_chain_launches.argtypes = [vp]
    lib.q8_0_chain_destroy.argtypes = [vp]
    lib.q8_0_stream_wait.argtypes = [vp, i64]
    lib.q8_0_status_string.argtypes = [ctypes.c_int]
    lib.q8_0_status_string.restype = ctypes.c_char_p
    lib.q8_0_last_error.argtypes = []
    lib.q8_0_last_error.restype = ctypes.c_char_p
    for name in ("q8_0_gemv", "q8_0_gemm_smallm", "q8_0_chain_create", "q8_0_decode_chain",
                 "q8_0_chain_launches", "q8_0_chain_destroy", "q8_0_stream_wait"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _status_string(code: int) -> str:
    return lib.q8_0_status_string(code).decode()


def last_error() -> str:
    return lib.q8_0_last_error().decode()


def check(rc: int) -> int:
    if rc < 0:
        raise Q8Error(rc, last_error())
    return rc


# ------------------------------------------------------------------ raw calls
def gemv_raw(x: int, w: int, y: int, n: int, p: int, stream: int = 0) -> int:
    """Call q8_0_gemv with raw device addresses; returns the status code."""
    return lib.q8_0_gemv(x, w, y, n, p, stream)


def gemm_smallm_raw(X: int, w: int, Y: int, m: int, n: int, p: int, stream: int = 0) -> int:
    return lib.q8_0_gemm_smallm(X, w, Y, m, n, p, stream)


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def _stream_handle(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t, dtype, what):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % what)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (what, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)


def weight_shape(w) -> Tuple[int, int]:
    """(p, n) of a Q8_0 weight tensor shaped (p, n/32*34), uint8."""
    if w.dim() != 2 or w.shape[1] % BLOCK_BYTES:
        raise ValueError("w must be uint8 of shape (p, n/32*34)")
    return int(w.shape[0]), int(w.shape[1]) // BLOCK_BYTES * BLOCK_QUANTS


def gemv(x, w, y=None, stream=None):
    """y = W x.  x float32 (n,), w uint8 (p, n/32*34); returns y float32 (p,)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(w, torch.uint8, "w")
    p, n = weight_shape(w)
    if x.numel() != n:
        raise ValueError("x has %d elements, w has %d columns" % (x.numel(), n))
    if y is None:
        y = torch.empty(p, dtype=torch.float32, device=x.device)
    _need(y, torch.float32, "y")
    if y.numel() != p:
        raise ValueError("y has %d elements, w has %d rows" % (y.numel(), p))
    check(lib.q8_0_gemv(x.data_ptr(), w.data_ptr(), y.data_ptr(), n, p, _stream_handle(stream)))
    return y


def gemm_smallm(X, w, Y=None, stream=None):
    """Y = X W^T for X float32 (m, n), m in 1..16; returns Y float32 (m, p)."""
    torch = _torch()
    _need(X, torch.float32, "X")
    _need(w, torch.uint8, "w")
    p, n = weight_shape(w)
    if X.dim() != 2 or X.shape[1] != n:
        raise ValueError("X must be (m, %d)" % n)
    m = int(X.shape[0])
    if Y is None:
        Y = torch.empty((m, p), dtype=torch.float32, device=X.device)
    _need(Y, torch.float32, "Y")
    if tuple(Y.shape) != (m, p):
        raise ValueError("Y must be (%d, %d)" % (m, p))
    check(lib.q8_0_gemm_smallm(X.data_ptr(), w.data_ptr(), Y.data_ptr(), m, n, p,
                               _stream_handle(stream)))
    return Y


def stream_wait(stream=None, timeout_ms: int = -1) -> int:
    return check(lib.q8_0_stream_wait(_stream_handle(stream), int(timeout_ms)))


class Chain:
    """A decode step's matvec chain, recorded once and replayed per token.

    ops: sequence of (x, w, y) tensors.  The tensors must stay alive and in
    place for the chain's lifetime (their addresses are recorded); the chain
    keeps references to them.
    """

    def __init__(self, ops: Sequence, fuse: bool = True):
        torch = _torch()
        arr = (Q8Op * len(ops))()
        self._keep = []
        for i, (x, w, y) in enumerate(ops):
            _need(x, torch.float32, "ops[%d].x" % i)
            _need(w, torch.uint8, "ops[%d].w" % i)
            _need(y, torch.float32, "ops[%d].y" % i)
            p, n = weight_shape(w)
            if x.numel() != n or y.numel() != p:
                raise ValueError("ops[%d]: shapes of x, w, y disagree" % i)
            arr[i] = Q8Op(x.data_ptr(), w.data_ptr(), y.data_ptr(), n, p)
            self._keep.append((x, w, y))
        h = ctypes.c_void_p()
        check(lib.q8_0_chain_create(arr, len(ops), Q8_CHAIN_FUSE if fuse else Q8_CHAIN_PER_OP,
                                    ctypes.byref(h)))
        self._h = h
        self.n_ops = len(ops)

    @property
    def launches(self) -> int:
        return check(lib.q8_0_chain_launches(self._h))

    def run(self, mode: int = MODE_GRAPH, stream=None) -> None:
        if self._h is None:
            raise RuntimeError("chain is closed")
        check(lib.q8_0_decode_chain(self._h, mode, _stream_handle(stream)))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib.q8_0_chain_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
