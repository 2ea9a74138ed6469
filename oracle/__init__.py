"""CPU oracle for the Q8_0 decode matvec -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``q8_block_quantized_gemv_amd``) never does.

The arithmetic lives in ``q8_0_oracle.c`` (plain serial C, float64
accumulation); this module only compiles it with gcc and marshals numpy
arrays through ctypes.  See the C file's header for what is computed and
which passages of the pages it follows (page "IV.4: One command buffer per
token": section "Eight kernels", the q8_matvec kernel; section "The
correctness ladder", the exact-float reference of rung one).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Iterable, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q8_0_oracle.c")
LIBRARY = os.path.join(_HERE, "libq8_0_oracle.so")

BLOCK_QUANTS = 32
BLOCK_BYTES = 34


def compile_oracle(src: str, out: str, werror: bool = True) -> str:
    """gcc, no FMA contraction, no fast-math (warnings are errors by default)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall"] + (["-Werror"] if werror else []) + [
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_oracle(SOURCE, LIBRARY)
    return LIBRARY


def row_bytes(n: int) -> int:
    return (n // BLOCK_QUANTS) * BLOCK_BYTES


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_w(w) -> np.ndarray:
    w = np.ascontiguousarray(np.asarray(w))
    if w.dtype != np.uint8:
        w = w.view(np.uint8)
    return w.reshape(-1)


class Oracle:
    """ctypes view of one compiled copy of the oracle."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        lib.q8o_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.q8o_f16_to_double.restype = ctypes.c_double
        p = ctypes.c_void_p
        lib.q8o_gemv.argtypes = [p, p, ctypes.c_int64, ctypes.c_int64, p, p, p]
        lib.q8o_gemv.restype = ctypes.c_int
        lib.q8o_gemm.argtypes = [p, p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, p, p, p]
        lib.q8o_gemm.restype = ctypes.c_int
        lib.q8o_f32_to_f16.argtypes = [ctypes.c_float]
        lib.q8o_f32_to_f16.restype = ctypes.c_uint16
        lib.q8o_quantize_x.argtypes = [p, ctypes.c_int64, p]
        lib.q8o_quantize_x.restype = ctypes.c_int
        lib.q8o_gemv_q8q8.argtypes = [p, p, ctypes.c_int64, ctypes.c_int64, p, p, p]
        lib.q8o_gemv_q8q8.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def f16_to_double(self, bits: int) -> float:
        """Decode one binary16 bit pattern with the oracle's own decoder."""
        return self.lib.q8o_f16_to_double(int(bits) & 0xFFFF)

    def gemv(self, w, x, n: int, p: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(y float32[p], y64 float64[p], mag float64[p]) for W (p x n) and x."""
        w = _as_w(w)
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        if n <= 0 or n % BLOCK_QUANTS:
            raise ValueError("n must be a positive multiple of 32")
        if w.size < p * row_bytes(n) or x.size < n:
            raise ValueError("buffer too small for the stated shape")
        y = np.empty(p, np.float32)
        y64 = np.empty(p, np.float64)
        mag = np.empty(p, np.float64)
        rc = self.lib.q8o_gemv(_ptr(w), _ptr(x), n, p, _ptr(y), _ptr(y64), _ptr(mag))
        if rc != 0:
            raise ValueError("oracle rejected the shape")
        return y, y64, mag

    def gemv_rows(self, w, x, n: int, rows: Iterable[int]):
        """The same as gemv() for the listed rows of W only."""
        w = _as_w(w)
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        rows = np.asarray(list(rows), dtype=np.int64)
        rb = row_bytes(n)
        y = np.empty(rows.size, np.float32)
        y64 = np.empty(rows.size, np.float64)
        mag = np.empty(rows.size, np.float64)
        base = _ptr(w)
        for i, r in enumerate(rows):
            if r < 0 or (r + 1) * rb > w.size:
                raise IndexError("row %d out of range" % r)
            self.lib.q8o_gemv(base + int(r) * rb, _ptr(x), n, 1,
                              _ptr(y[i:]), _ptr(y64[i:]), _ptr(mag[i:]))
        return y, y64, mag

    def gemm(self, w, X, m: int, n: int, p: int):
        """Y[i] = gemv(W, X[i]) for i < m; returns (Y, Y64, MAG), each m x p."""
        w = _as_w(w)
        X = np.ascontiguousarray(X, dtype=np.float32).reshape(-1)
        if w.size < p * row_bytes(n) or X.size < m * n:
            raise ValueError("buffer too small for the stated shape")
        Y = np.empty((m, p), np.float32)
        Y64 = np.empty((m, p), np.float64)
        MAG = np.empty((m, p), np.float64)
        rc = self.lib.q8o_gemm(_ptr(w), _ptr(X), m, n, p, _ptr(Y), _ptr(Y64), _ptr(MAG))
        if rc != 0:
            raise ValueError("oracle rejected the shape")
        return Y, Y64, MAG


    def f32_to_f16(self, v: float) -> int:
        """binary16 bits of a float32 value, nearest with ties to even."""
        return int(self.lib.q8o_f32_to_f16(float(np.float32(v))))

    def quantize_x(self, x) -> np.ndarray:
        """x (n floats) as n/32 Q8_0 blocks: uint8[n/32*34] (the reading of
        the pages' activation quantization, see the C source)."""
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        out = np.empty(row_bytes(x.size), np.uint8)
        if self.lib.q8o_quantize_x(_ptr(x), x.size, _ptr(out)) != 0:
            raise ValueError("n must be a positive multiple of 32")
        return out

    def gemv_q8q8(self, w, x, n: int, p: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """The integer matvec (x quantized to Q8_0): (y, y64, mag) as gemv()."""
        w = _as_w(w)
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        if n <= 0 or n % BLOCK_QUANTS:
            raise ValueError("n must be a positive multiple of 32")
        if w.size < p * row_bytes(n) or x.size < n:
            raise ValueError("buffer too small for the stated shape")
        y = np.empty(p, np.float32)
        y64 = np.empty(p, np.float64)
        mag = np.empty(p, np.float64)
        if self.lib.q8o_gemv_q8q8(_ptr(w), _ptr(x), n, p, _ptr(y), _ptr(y64), _ptr(mag)) != 0:
            raise ValueError("oracle rejected the shape")
        return y, y64, mag


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build(force=True)
        _default = Oracle(LIBRARY)
    return _default


def f16_to_double(bits: int) -> float:
    return default().f16_to_double(bits)


def gemv(w, x, n: int, p: int):
    return default().gemv(w, x, n, p)


def gemv_rows(w, x, n: int, rows: Iterable[int]):
    return default().gemv_rows(w, x, n, rows)


def gemv_threaded(w, x, n: int, p: int, threads: Optional[int] = None):
    """gemv() with contiguous row ranges on a pool of host threads (the C
    call releases the GIL).  Every row is the same serial oracle on the same
    bytes, so the results equal gemv()'s exactly."""
    from concurrent.futures import ThreadPoolExecutor
    o = default()
    w = _as_w(w)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if w.size < p * row_bytes(n) or x.size < n:
        raise ValueError("buffer too small for the stated shape")
    threads = max(1, min(threads or min(16, os.cpu_count() or 1), p))
    y = np.empty(p, np.float32)
    y64 = np.empty(p, np.float64)
    mag = np.empty(p, np.float64)
    rb = row_bytes(n)
    cuts = [p * k // threads for k in range(threads + 1)]

    def part(k):
        a, b = cuts[k], cuts[k + 1]
        if b > a and o.lib.q8o_gemv(_ptr(w) + a * rb, _ptr(x), n, b - a, _ptr(y[a:]), _ptr(y64[a:]),
                                    _ptr(mag[a:])) != 0:
            raise ValueError("oracle rejected the shape")

    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(part, range(threads)))
    return y, y64, mag


def gemm(w, X, m: int, n: int, p: int):
    return default().gemm(w, X, m, n, p)


def f32_to_f16(v: float) -> int:
    return default().f32_to_f16(v)


def quantize_x(x):
    return default().quantize_x(x)


def gemv_q8q8(w, x, n: int, p: int):
    return default().gemv_q8q8(w, x, n, p)
