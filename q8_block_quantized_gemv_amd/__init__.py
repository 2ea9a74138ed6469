"""Python binding of the MI355X Q8_0 decode matvec library (libq8gemv.so).

Argument marshalling only: tensors become device pointers, torch streams
become hipStream_t handles, and every computation happens in the HIP
kernels behind the C ABI declared in include/q8gemv.h.  There is no other
implementation: if the library is missing, importing this package raises.

The names follow the C ABI:
    gemv(x, w, y=None, stream=None)            -> q8_0_gemv
    gemv(x, w, shape=(c, waves, stages))       -> q8_0_gemv_shaped
    gemm_smallm(X, w, Y=None, stream=None)     -> q8_0_gemm_smallm (+ _workspace)
    gemm_smallm(X, w, kernel=SMALLM_MFMA)      -> q8_0_gemm_smallm_kernel
    gemv_q8q8(x, w, y=None), quantize(x)       -> q8_0_gemv_q8q8, q8_0_quantize
    Chain(ops, fuse=True, split_k=False) .run  -> q8_0_chain_create / q8_0_decode_chain
    stream_wait(stream, timeout_ms)            -> q8_0_stream_wait
    rms_norm, rope, append_kv, attention_decode, add_inplace,
    silu_hadamard, argmax                      -> the q8_0_* calls of include/q8step.h

Calls whose kernels need scratch memory take a caller-owned device
workspace (workspace=, a uint8 tensor); when none is given the binding
allocates one of the size the library's query returns, on the call's
stream, through torch's allocator -- the library itself allocates nothing.
    Step(cfg, weights) .reset/.run             -> q8_0_step_create / _reset / _run
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
Q8_CHAIN_SPLIT_K = 2
Q8_CHAIN_XQ = 4
MODE_GRAPH = 0
MODE_EAGER = 1
MODE_SYNC_EACH = 2

SMALLM_AUTO = 0
SMALLM_VALU = 1
SMALLM_MFMA = 2
SMALLM_VROW = 3
SMALLM_VROW1 = 4
SMALLM_KS = 5

BLOCK_QUANTS = 32
BLOCK_BYTES = 34

EXPORTS = ("q8_0_gemv", "q8_0_gemv_shaped", "q8_0_gemm_smallm", "q8_0_gemm_smallm_kernel",
           "q8_0_gemm_smallm_workspace", "q8_0_attention_workspace", "q8_0_argmax_workspace",
           "q8_0_gemm_smallm_noalloc", "q8_0_gemm_smallm_choice", "q8_0_gemv_plan", "q8_0_chain_plan",
           "q8_0_chain_create", "q8_0_decode_chain",
           "q8_0_chain_launches", "q8_0_chain_destroy", "q8_0_stream_wait",
           "q8_0_status_string", "q8_0_last_error", "q8_0_gemv_q8q8", "q8_0_quantize",
           "q8_0_rms_norm", "q8_0_rope", "q8_0_append_kv", "q8_0_attention_decode",
           "q8_0_add_inplace", "q8_0_silu_hadamard", "q8_0_argmax",
           "q8_0_step_create", "q8_0_step_reset", "q8_0_step_run", "q8_0_step_launches",
           "q8_0_step_buffers", "q8_0_step_destroy")

NO_INDEX = 0xFFFFFFFF   # argmax of a row of NaN
MAX_SEQ = 65536


class Q8Error(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        super().__init__("%s (%d): %s" % (_status_string(code), code, detail))


class Q8Op(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("p", ctypes.c_int64)]


class Q8LaunchPlan(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("tile_rows", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("first_op", ctypes.c_int64), ("n_ops", ctypes.c_int64),
                ("workgroups", ctypes.c_int64), ("first_tile", ctypes.c_int64)]


LAUNCH_ROWS, LAUNCH_SUPERROWS, LAUNCH_FUSED, LAUNCH_FUSED_MIXED = 0, 1, 2, 3
TAIL_BIT = 0x80000000


class Q8LayerW(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown",
                 "attn_norm", "ffn_norm", "q_norm", "k_norm")]


class Q8Model(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int64) for k in
                ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab",
                 "max_seq")] + [
               ("eps", ctypes.c_float), ("theta", ctypes.c_float),
               ("embed", ctypes.c_void_p), ("out_norm", ctypes.c_void_p),
               ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(Q8LayerW))]


class Q8StepBufs(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("token", "pos", "x", "logits", "k_cache", "v_cache")]


def _load():
    if not os.path.exists(LIBRARY):
        raise ImportError("libq8gemv.so is not built; run __graft_entry__.build() "
                          "or python q8_block_quantized_gemv_amd/build.py")
    # PyTorch's ROCm wheel carries a HIP runtime of its own; the library uses
    # the system's.  Both work in one process when torch's runtime has
    # started before the library is loaded (or when the library's runtime
    # starts first), but not when the library is loaded, torch's runtime
    # starts, and then the library's: the library then sees no device.  So
    # torch's runtime is started here, before the library is loaded.
    try:
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
    except ImportError:
        pass
    lib = ctypes.CDLL(LIBRARY)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q8_0_gemv.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.q8_0_gemv_shaped.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    sz = ctypes.c_size_t
    lib.q8_0_gemm_smallm.argtypes = [vp, vp, vp, i64, i64, i64, vp, sz, vp]
    lib.q8_0_gemm_smallm_kernel.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, vp, sz, vp]
    lib.q8_0_gemm_smallm_workspace.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(sz)]
    lib.q8_0_gemm_smallm_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.q8_0_gemm_smallm_choice.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_int)]
    ip = ctypes.POINTER(ctypes.c_int)
    lib.q8_0_gemv_plan.argtypes = [i64, i64, i64, ip, ip, ip, ip, ctypes.POINTER(i64)]
    lib.q8_0_chain_plan.argtypes = [ctypes.POINTER(Q8Op), i64, ctypes.c_uint32, i64,
                                    ctypes.POINTER(Q8LaunchPlan), i64, ctypes.POINTER(i64),
                                    ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_uint32), i64,
                                    ctypes.POINTER(i64)]
    lib.q8_0_attention_workspace.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
    lib.q8_0_argmax_workspace.argtypes = [i64, ctypes.POINTER(sz)]
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
    lib.q8_0_gemv_q8q8.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.q8_0_quantize.argtypes = [vp, vp, i64, vp]
    f32, u32, i32 = ctypes.c_float, ctypes.c_uint32, ctypes.c_int
    lib.q8_0_rms_norm.argtypes = [vp, vp, vp, i64, i64, f32, vp]
    lib.q8_0_rope.argtypes = [vp, i64, i64, i64, f32, vp]
    lib.q8_0_append_kv.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.q8_0_attention_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, sz, vp]
    lib.q8_0_add_inplace.argtypes = [vp, vp, i64, vp]
    lib.q8_0_silu_hadamard.argtypes = [vp, vp, vp, i64, vp]
    lib.q8_0_argmax.argtypes = [vp, i64, vp, vp, sz, vp]
    lib.q8_0_step_create.argtypes = [ctypes.POINTER(Q8Model), ctypes.POINTER(vp)]
    lib.q8_0_step_reset.argtypes = [vp, i64, u32, vp]
    lib.q8_0_step_run.argtypes = [vp, i32, vp]
    lib.q8_0_step_launches.argtypes = [vp]
    lib.q8_0_step_buffers.argtypes = [vp, ctypes.POINTER(Q8StepBufs)]
    lib.q8_0_step_destroy.argtypes = [vp]
    for name in EXPORTS:
        if name not in ("q8_0_status_string", "q8_0_last_error"):
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


def gemm_smallm_raw(X: int, w: int, Y: int, m: int, n: int, p: int, ws: int = 0, ws_bytes: int = 0,
                    stream: int = 0) -> int:
    return lib.q8_0_gemm_smallm(X, w, Y, m, n, p, ws, ws_bytes, stream)


def _size_query(fn, *args) -> int:
    out = ctypes.c_size_t(0)
    check(fn(*args, ctypes.byref(out)))
    return int(out.value)


def gemm_smallm_workspace(m: int, n: int, p: int, kernel: int = SMALLM_AUTO) -> int:
    """Workspace bytes q8_0_gemm_smallm needs on the current device."""
    return _size_query(lib.q8_0_gemm_smallm_workspace, int(m), int(n), int(p), int(kernel))


def gemm_smallm_choice(m: int, n: int, p: int) -> int:
    """The kernel (SMALLM_*) q8_0_gemm_smallm runs for (m, n, p), m = 2..16."""
    out = ctypes.c_int(0)
    check(lib.q8_0_gemm_smallm_choice(int(m), int(n), int(p), ctypes.byref(out)))
    return int(out.value)


def attention_workspace(seq: int, head_dim: int, n_heads: int) -> int:
    return _size_query(lib.q8_0_attention_workspace, int(seq), int(head_dim), int(n_heads))


def argmax_workspace(n: int) -> int:
    return _size_query(lib.q8_0_argmax_workspace, int(n))


def gemv_plan(n: int, p: int, cus: int = 256):
    """(lanes_per_row, waves, stages, tile_rows, workgroups) of q8_0_gemv for
    (n, p) on a GPU of `cus` compute units (host only)."""
    c, w, st, tr, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    check(lib.q8_0_gemv_plan(int(n), int(p), int(cus), ctypes.byref(c), ctypes.byref(w), ctypes.byref(st),
                             ctypes.byref(tr), ctypes.byref(g)))
    return c.value, w.value, st.value, tr.value, g.value


def chain_plan(ops, flags: int = 0, cus: int = 256):
    """The launches q8_0_chain_create would record for ops, a sequence of
    (x, w, y, n, p) with raw device addresses (compared, never read): a list
    of dicts, and for fused launches each workgroup's (op, tile) items as two
    lists.  Host only."""
    arr = (Q8Op * len(ops))(*[Q8Op(int(x), int(w), int(y), int(n), int(p)) for x, w, y, n, p in ops])
    nl, nt = ctypes.c_int64(), ctypes.c_int64()
    check(lib.q8_0_chain_plan(arr, len(ops), flags, cus, None, 0, ctypes.byref(nl), None, None, 0,
                              ctypes.byref(nt)))
    L = (Q8LaunchPlan * max(1, nl.value))()
    top = (ctypes.c_int64 * max(1, nt.value))()
    tid = (ctypes.c_uint32 * max(1, nt.value))()
    check(lib.q8_0_chain_plan(arr, len(ops), flags, cus, L, nl.value, ctypes.byref(nl), top, tid, nt.value,
                              ctypes.byref(nt)))
    launches = [{f: getattr(L[k], f) for f, _ in Q8LaunchPlan._fields_} for k in range(nl.value)]
    return launches, list(top[:nt.value]), list(tid[:nt.value])


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


def gemv(x, w, y=None, stream=None, shape=None):
    """y = W x.  x float32 (n,), w uint8 (p, n/32*34); returns y float32 (p,).

    shape=(lanes_per_row, waves, stages) launches on that explicit shape
    (q8_0_gemv_shaped, n a multiple of 256): the same bits, another launch."""
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
    if shape is None:
        check(lib.q8_0_gemv(x.data_ptr(), w.data_ptr(), y.data_ptr(), n, p, _stream_handle(stream)))
    else:
        c, waves, stages = shape
        check(lib.q8_0_gemv_shaped(x.data_ptr(), w.data_ptr(), y.data_ptr(), n, p, int(c), int(waves),
                                   int(stages), _stream_handle(stream)))
    return y


def gemv_q8q8(x, w, y=None, stream=None):
    """y = W x with x quantized to Q8_0 and integer block dots (q8_0_gemv_q8q8)."""
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
    check(lib.q8_0_gemv_q8q8(x.data_ptr(), w.data_ptr(), y.data_ptr(), n, p, _stream_handle(stream)))
    return y


def quantize(x, xq=None, stream=None):
    """x float32 (n,) -> Q8_0 bytes uint8 (n/32*34,) (q8_0_quantize)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    n = x.numel()
    if xq is None:
        xq = torch.empty(n // BLOCK_QUANTS * BLOCK_BYTES, dtype=torch.uint8, device=x.device)
    _need(xq, torch.uint8, "xq")
    if xq.numel() != n // BLOCK_QUANTS * BLOCK_BYTES:
        raise ValueError("xq must hold n/32 blocks of 34 bytes")
    check(lib.q8_0_quantize(x.data_ptr(), xq.data_ptr(), n, _stream_handle(stream)))
    return xq


def _workspace(nbytes: int, device, stream, given):
    """The caller's workspace (a uint8 device tensor), or one of nbytes
    allocated on the call's stream (so torch's allocator reuses it only after
    the work queued there)."""
    torch = _torch()
    if given is not None:
        _need(given, torch.uint8, "workspace")
        return given
    if nbytes == 0:
        return None
    if isinstance(stream, torch.cuda.Stream):
        with torch.cuda.stream(stream):
            return torch.empty(nbytes, dtype=torch.uint8, device=device)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_args(ws):
    return (0, 0) if ws is None else (ws.data_ptr(), ws.numel())


def gemm_smallm(X, w, Y=None, stream=None, kernel=None, workspace=None):
    """Y = X W^T for X float32 (m, n), m in 1..16; returns Y float32 (m, p).

    kernel=SMALLM_* runs a named kernel (q8_0_gemm_smallm_kernel);
    workspace: a uint8 device tensor of at least gemm_smallm_workspace bytes."""
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
    k = SMALLM_AUTO if kernel is None else int(kernel)
    ws = _workspace(gemm_smallm_workspace(m, n, p, k) if workspace is None else 0, X.device, stream,
                    workspace)
    wp, wn = _ws_args(ws)
    if kernel is None:
        check(lib.q8_0_gemm_smallm(X.data_ptr(), w.data_ptr(), Y.data_ptr(), m, n, p, wp, wn,
                                   _stream_handle(stream)))
    else:
        check(lib.q8_0_gemm_smallm_kernel(X.data_ptr(), w.data_ptr(), Y.data_ptr(), m, n, p, k, wp, wn,
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

    def __init__(self, ops: Sequence, fuse: bool = True, split_k: bool = False, xq: bool = False):
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
        flags = ((Q8_CHAIN_FUSE if fuse else Q8_CHAIN_PER_OP) | (Q8_CHAIN_SPLIT_K if split_k else 0) |
                 (Q8_CHAIN_XQ if xq else 0))
        check(lib.q8_0_chain_create(arr, len(ops), flags, ctypes.byref(h)))
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


# ------------------------------------------------------------------ the rest of a decode step
def _f32(t, what, numel=None):
    torch = _torch()
    _need(t, torch.float32, what)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (what, t.numel(), numel))


def rms_norm(x, w, out=None, eps: float = 1e-6, stream=None):
    """Each row of x (rows, dim) times (mean(x^2) + eps)^(-1/2) times w (dim,).
    out may be x (in place)."""
    torch = _torch()
    dim = int(w.numel())
    _f32(w, "w")
    _f32(x, "x")
    if x.numel() % dim:
        raise ValueError("x is not a whole number of rows of %d" % dim)
    if out is None:
        out = torch.empty_like(x)
    _f32(out, "out", x.numel())
    check(lib.q8_0_rms_norm(x.data_ptr(), w.data_ptr(), out.data_ptr(), dim, x.numel() // dim,
                            float(eps), _stream_handle(stream)))
    return out


def rope(x, head_dim: int, pos: int, theta: float, stream=None):
    """Rotary embedding of every head of x (heads, head_dim), in place."""
    _f32(x, "x")
    if x.numel() % head_dim:
        raise ValueError("x is not a whole number of heads of %d" % head_dim)
    check(lib.q8_0_rope(x.data_ptr(), head_dim, x.numel() // head_dim, int(pos), float(theta),
                        _stream_handle(stream)))
    return x


def append_kv(k, v, kc, vc, pos: int, stream=None):
    """Row pos of the caches kc, vc (rows, width) becomes k, v (width,)."""
    width = int(k.numel())
    _f32(k, "k")
    _f32(v, "v", width)
    _f32(kc, "kc")
    _f32(vc, "vc", kc.numel())
    if kc.numel() < (int(pos) + 1) * width:
        raise ValueError("the caches hold fewer than pos + 1 rows")
    check(lib.q8_0_append_kv(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), width,
                             int(pos), _stream_handle(stream)))


def attention_decode(q, kc, vc, seq: int, head_dim: int, kv_group: int, out=None, stream=None,
                     workspace=None):
    """Decode attention of q (n_heads, head_dim) over the first seq rows of
    the caches kc, vc (rows, kv_width); returns out (n_heads, head_dim)."""
    torch = _torch()
    _f32(q, "q")
    _f32(kc, "kc")
    _f32(vc, "vc", kc.numel())
    if q.numel() % head_dim:
        raise ValueError("q is not a whole number of heads")
    n_heads = q.numel() // head_dim
    if kc.dim() != 2:
        raise ValueError("kc must be (rows, kv_width)")
    kv_width = int(kc.shape[1])
    if kc.shape[0] < seq:
        raise ValueError("the caches hold fewer than seq rows")
    if out is None:
        out = torch.empty((n_heads, head_dim), dtype=torch.float32, device=q.device)
    _f32(out, "out", n_heads * head_dim)
    ws = _workspace(attention_workspace(seq, head_dim, n_heads) if workspace is None else 0, q.device, stream,
                    workspace)
    wp, wn = _ws_args(ws)
    check(lib.q8_0_attention_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), out.data_ptr(),
                                    int(seq), kv_width, head_dim, n_heads, int(kv_group), wp, wn,
                                    _stream_handle(stream)))
    return out


def add_inplace(x, y, stream=None):
    _f32(x, "x")
    _f32(y, "y", x.numel())
    check(lib.q8_0_add_inplace(x.data_ptr(), y.data_ptr(), x.numel(), _stream_handle(stream)))
    return x


def silu_hadamard(gate, up, out=None, stream=None):
    torch = _torch()
    _f32(gate, "gate")
    _f32(up, "up", gate.numel())
    if out is None:
        out = torch.empty_like(gate)
    _f32(out, "out", gate.numel())
    check(lib.q8_0_silu_hadamard(gate.data_ptr(), up.data_ptr(), out.data_ptr(), gate.numel(),
                                 _stream_handle(stream)))
    return out


def argmax(x, out=None, stream=None, workspace=None):
    """Index of the largest value of x (ties to the lowest index, NaN never
    wins) into out, a one-element int32 device tensor holding the uint32
    index (NO_INDEX, read as -1, when every value is NaN)."""
    torch = _torch()
    _f32(x, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=x.device)
    _need(out, torch.int32, "out")
    ws = _workspace(argmax_workspace(x.numel()) if workspace is None else 0, x.device, stream, workspace)
    wp, wn = _ws_args(ws)
    check(lib.q8_0_argmax(x.data_ptr(), x.numel(), out.data_ptr(), wp, wn, _stream_handle(stream)))
    return out


class _DeviceView:
    """A borrowed device buffer, shown to torch through __cuda_array_interface__."""

    def __init__(self, ptr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr,
                                         "data": (int(ptr), False), "version": 2,
                                         "strides": None}


LAYER_KEYS = ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown",
              "attn_norm", "ffn_norm", "q_norm", "k_norm")
CONFIG_KEYS = ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab",
               "max_seq", "eps", "theta")


class Step:
    """A whole decode step of a Qwen3-style model, recorded once into a
    hipGraph and replayed per token (q8_0_step_*).

    cfg: dict with CONFIG_KEYS.  weights: dict with "embed" (vocab, hidden)
    float32, "out_norm" (hidden,) float32, "lm_head" uint8 Q8_0 (vocab rows
    of hidden) and "layers", a list of n_layers dicts with LAYER_KEYS (the
    seven Q8_0 projections, uint8 (p, n/32*34), and the four float32 norm
    weights).  The step keeps references to every tensor: their addresses
    are recorded.
    """

    def __init__(self, cfg: dict, weights: dict):
        torch = _torch()
        c = {k: cfg[k] for k in CONFIG_KEYS}
        hid, inter, hd = int(c["hidden"]), int(c["inter"]), int(c["head_dim"])
        qw, kvw = int(c["n_heads"]) * hd, int(c["n_kv_heads"]) * hd
        vocab = int(c["vocab"])
        layers = weights["layers"]
        if len(layers) != int(c["n_layers"]):
            raise ValueError("weights hold %d layers, cfg says %d" % (len(layers), c["n_layers"]))
        shapes = {"wq": (qw, hid), "wk": (kvw, hid), "wv": (kvw, hid), "wo": (hid, qw),
                  "wgate": (inter, hid), "wup": (inter, hid), "wdown": (hid, inter)}
        lens = {"attn_norm": hid, "ffn_norm": hid, "q_norm": hd, "k_norm": hd}
        arr = (Q8LayerW * len(layers))()
        self._keep = []
        for i, L in enumerate(layers):
            ptrs = []
            for k in LAYER_KEYS:
                t = L[k]
                if k in shapes:
                    _need(t, torch.uint8, "layers[%d].%s" % (i, k))
                    if weight_shape(t) != shapes[k]:
                        raise ValueError("layers[%d].%s is %s, expected %s"
                                         % (i, k, weight_shape(t), shapes[k]))
                else:
                    _f32(t, "layers[%d].%s" % (i, k), lens[k])
                ptrs.append(t.data_ptr())
                self._keep.append(t)
            arr[i] = Q8LayerW(*ptrs)
        _f32(weights["embed"], "embed", vocab * hid)
        _f32(weights["out_norm"], "out_norm", hid)
        _need(weights["lm_head"], torch.uint8, "lm_head")
        if weight_shape(weights["lm_head"]) != (vocab, hid):
            raise ValueError("lm_head must be vocab rows of hidden columns")
        for k in ("embed", "out_norm", "lm_head"):
            self._keep.append(weights[k])
        self._layers = arr
        model = Q8Model(c["n_layers"], hid, c["n_heads"], c["n_kv_heads"], hd, inter, vocab,
                        c["max_seq"], float(c["eps"]), float(c["theta"]),
                        weights["embed"].data_ptr(), weights["out_norm"].data_ptr(),
                        weights["lm_head"].data_ptr(), arr)
        h = ctypes.c_void_p()
        check(lib.q8_0_step_create(ctypes.byref(model), ctypes.byref(h)))
        self._h = h
        self.cfg = c
        b = Q8StepBufs()
        check(lib.q8_0_step_buffers(self._h, ctypes.byref(b)))
        self._views = {
            "token": (b.token, (1,), "<i4"), "pos": (b.pos, (1,), "<i4"),
            "x": (b.x, (hid,), "<f4"), "logits": (b.logits, (vocab,), "<f4"),
            "k_cache": (b.k_cache, (int(c["n_layers"]), int(c["max_seq"]), kvw), "<f4"),
            "v_cache": (b.v_cache, (int(c["n_layers"]), int(c["max_seq"]), kvw), "<f4")}

    def _handle(self):
        if self._h is None:
            raise RuntimeError("step is closed")
        return self._h

    @property
    def launches(self) -> int:
        return check(lib.q8_0_step_launches(self._handle()))

    def reset(self, pos: int, token: int, stream=None) -> None:
        check(lib.q8_0_step_reset(self._handle(), int(pos), int(token) & 0xFFFFFFFF,
                                  _stream_handle(stream)))

    def run(self, mode: int = MODE_GRAPH, stream=None) -> None:
        check(lib.q8_0_step_run(self._handle(), int(mode), _stream_handle(stream)))

    def buffer(self, name: str):
        """A device tensor viewing one of the step's buffers (token, pos, x,
        logits, k_cache, v_cache); valid while the step is open."""
        torch = _torch()
        self._handle()
        ptr, shape, ts = self._views[name]
        return torch.as_tensor(_DeviceView(ptr, shape, ts), device="cuda")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib.q8_0_step_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
