"""Checks that pin the CPU oracle to facts that do not come from the oracle.

Every check takes an ``oracle.Oracle`` so that the same checks can run on the
real oracle (where all must pass) and on copies with a planted mistake (where
at least one must fail).  Expected values come from: the pages (the scale
bytes of the test fabricator), hand-worked closed forms, exact integer or
rational arithmetic, numpy's own binary16 decoding, and a dense float64
dequantize-then-matmul written independently of the oracle's loop nest.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, _, v = line.partition(" ")
            vals[k] = v.strip()
    return vals


def dense_reference(w: np.ndarray, x: np.ndarray, n: int, p: int):
    """Dequantize the whole matrix with numpy (binary16 through numpy's own
    cast), then a float64 dense matvec; returns (y64, mag)."""
    nb = n // 32
    blk = w.reshape(p * nb, 34)
    d = blk[:, 0:2].copy().view("<f2").astype(np.float64).reshape(p, nb)
    q = blk[:, 2:].copy().view(np.int8).astype(np.float64).reshape(p, nb, 32)
    dense = (d[:, :, None] * q).reshape(p, n)
    xd = x.astype(np.float64)
    y = dense @ xd
    mag = np.abs(dense) @ np.abs(xd)
    return y, mag


# ---------------------------------------------------------------- decoding
def pin_f16_exhaustive(o):
    """All 65536 binary16 patterns against numpy's float16 -> float64 cast."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([o.f16_to_double(int(b)) for b in bits], dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "NaN set differs"
    ok = nan_ref | (got == ref)
    assert ok.all(), "first mismatch at bits 0x%04x" % int(np.argmin(ok))
    # signed zero is preserved too
    assert math.copysign(1.0, o.f16_to_double(0x8000)) == -1.0


def pin_page_scale_bytes(o):
    g = _read_golden("page_scale_bytes.txt")
    b0, b1 = [int(t, 16) for t in g["bytes"].split()]
    assert (b0 | (b1 << 8)) == int(g["bits"], 16)
    assert o.f16_to_double(b0 | (b1 << 8)) == float(g["value"])
    # and through the matvec: one block of quant 1 at column 0, x = 1
    w = np.zeros(34, np.uint8)
    w[0], w[1], w[2] = b0, b1, 1
    x = np.zeros(32, np.float32)
    x[0] = 1.0
    y, y64, _ = o.gemv(w, x, 32, 1)
    assert y64[0] == float(g["value"]) and y[0] == np.float32(g["value"])


def pin_hand_worked_row(o):
    g = _read_golden("hand_worked_row.txt")
    n, p = int(g["n"]), int(g["p"])
    blk0 = np.zeros(34, np.uint8)
    blk0[0:2] = [0x00, 0x3C]
    blk0[2:] = (np.arange(32) - 16).astype(np.int8).view(np.uint8)
    blk1 = np.zeros(34, np.uint8)
    blk1[0:2] = [0x00, 0xB8]
    blk1[2:] = 2
    w = np.concatenate([blk0, blk1])
    x = np.concatenate([np.ones(32), np.arange(32)]).astype(np.float32)
    y, y64, mag = o.gemv(w, x, n, p)
    assert y64[0] == float(g["y"]) and y[0] == np.float32(g["y"])
    assert mag[0] == float(g["mag"])


def pin_quant_byte_range(o):
    """Every quant byte value 0..255 read as two's-complement int8, at every
    position of a block (one-hot quants, x = column index + 1)."""
    n = 64
    x = (np.arange(n) + 1).astype(np.float32)
    for byte in range(256):
        q = byte - 256 if byte >= 128 else byte
        for col in (0, 17, 31, 32, 50, 63):
            w = np.zeros(2 * 34, np.uint8)
            b, j = divmod(col, 32)
            w[34 * b:34 * b + 2] = [0x00, 0x3C]          # scale 1.0
            w[34 * b + 2 + j] = byte
            _, y64, _ = o.gemv(w, x, n, 1)
            assert y64[0] == q * (col + 1), (byte, col, y64[0])


# ---------------------------------------------------------------- matvec
def pin_brute_force(o):
    """Oracle vs dense float64 dequantize-then-matmul on tiny shapes."""
    shapes = [(32, 1), (32, 5), (64, 3), (96, 50), (256, 17), (128, 64), (896, 7)]
    for k, (n, p) in enumerate(shapes):
        rng = np.random.default_rng(1000 + k)
        w = synth.q8_weights(n, p, rng)
        x = synth.activations(n, rng)
        y, y64, mag = o.gemv(w, x, n, p)
        ry, rmag = dense_reference(w, x, n, p)
        assert np.all(np.abs(y64 - ry) <= 1e-12 * rmag + 1e-300), (n, p)
        assert np.allclose(mag, rmag, rtol=1e-12, atol=0), (n, p)
        assert np.array_equal(y, y64.astype(np.float32)), (n, p)


def pin_page_shape(o):
    """The page's rung-one matvec test: 50 x 96, weights from its generator
    with seed 7, x with seed 42.  Its exact-float reference sums
    scale * quant * x in float32 per row; the page holds its GPU kernel to
    5e-4 absolute against that, so the oracle must sit inside that bar too."""
    p, n = 50, 96
    w = synth.page_q8_bytes(p, n, 7)
    x = synth.page_x(n, 42)
    y, y64, _ = o.gemv(w, x, n, p)
    blk = w.reshape(-1, 34)
    d = blk[:, 0:2].copy().view("<f2").astype(np.float32)[:, 0]
    q = blk[:, 2:].copy().view(np.int8).astype(np.float32)
    ref = np.zeros(p, np.float32)
    for r in range(p):
        s = np.float32(0.0)
        for b in range(n // 32):
            for j in range(32):
                s = np.float32(s + np.float32(np.float32(d[r * 3 + b] * q[r * 3 + b, j]) * x[32 * b + j]))
        ref[r] = s
    assert np.max(np.abs(y - ref)) < 5e-4


def pin_zero_scale(o):
    for n, p in [(32, 4), (256, 9), (1024, 3)]:
        rng = np.random.default_rng(7 + n)
        w = synth.q8_weights(n, p, rng).reshape(-1, 34)
        w[:, 0:2] = 0
        x = synth.activations(n, rng) * np.float32(1e3)
        y, y64, mag = o.gemv(w, x, n, p)
        assert np.all(y64 == 0.0) and np.all(mag == 0.0)
        w[:, 0:2] = [0x00, 0x80]                          # -0.0
        y, y64, mag = o.gemv(w, x, n, p)
        assert np.all(y64 == 0.0)


def pin_all_ones(o):
    """All quants 1: y = sum_b d_b * sum_j x_{32b+j}, evaluated exactly with
    rationals and rounded once."""
    for n, p in [(32, 3), (96, 4), (512, 5)]:
        rng = np.random.default_rng(11 + n)
        w = synth.q8_weights(n, p, rng).reshape(-1, 34)
        w[:, 2:] = 1
        x = synth.activations(n, rng)
        _, y64, _ = o.gemv(w, x, n, p)
        nb = n // 32
        d = w[:, 0:2].copy().view("<f2")[:, 0]
        for r in range(p):
            exact = Fraction(0)
            for b in range(nb):
                sx = sum(Fraction(float(v)) for v in x[32 * b:32 * b + 32])
                exact += Fraction(float(d[r * nb + b])) * sx
            assert abs(y64[r] - float(exact)) <= 1e-13 * abs(float(exact)) + 1e-300


def pin_integer_exact(o):
    """Scale 0.0625 everywhere, integer x in [-4, 4]: the result is an exact
    multiple of 1/16 that Python integers compute without rounding."""
    for n, p in [(32, 2), (3584, 3), (18944, 2)]:
        rng = np.random.default_rng(23 + n)
        w, x = synth.integer_case(n, p, rng)
        y, y64, _ = o.gemv(w, x, n, p)
        q = w.reshape(p, n // 32, 34)[:, :, 2:].copy().view(np.int8).reshape(p, n).astype(np.int64)
        xi = x.astype(np.int64)
        for r in range(p):
            exact = Fraction(int(np.dot(q[r], xi)), 16)
            assert y64[r] == float(exact) and y[r] == np.float32(float(exact))


def pin_specials(o):
    """Subnormal, largest-finite, infinite and NaN scales by definition."""
    x = np.zeros(32, np.float32)
    x[3] = 2.0
    cases = [(0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14),
             (0x7BFF, 65504.0), (0xFBFF, -65504.0), (0x7C00, math.inf), (0xFC00, -math.inf)]
    for bits, dv in cases:
        w = np.zeros(34, np.uint8)
        w[0], w[1] = bits & 0xFF, bits >> 8
        w[2 + 3] = 5
        _, y64, _ = o.gemv(w, x, 32, 1)
        assert y64[0] == dv * 10.0, (hex(bits), y64[0])
    w = np.zeros(34, np.uint8)
    w[0], w[1] = 0x00, 0x7E
    w[2 + 3] = 5
    _, y64, _ = o.gemv(w, x, 32, 1)
    assert math.isnan(y64[0])


def pin_symmetries(o):
    rng = np.random.default_rng(99)
    n, p = 256, 12
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    y, y64, mag = o.gemv(w, x, n, p)
    yn, yn64, magn = o.gemv(w, -x, n, p)
    assert np.array_equal(yn64, -y64) and np.array_equal(magn, mag)
    y2, y264, _ = o.gemv(w, x * np.float32(4.0), n, p)
    assert np.array_equal(y264, 4.0 * y64)


def pin_gemm_rows(o):
    """Small-batch rows are the independent matvecs (dense reference)."""
    rng = np.random.default_rng(5)
    n, p, m = 128, 9, 4
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m)
    Y, Y64, MAG = o.gemm(w, X, m, n, p)
    for i in range(m):
        ry, rmag = dense_reference(w, X[i], n, p)
        assert np.all(np.abs(Y64[i] - ry) <= 1e-12 * rmag + 1e-300)


ALL_PINS = [pin_f16_exhaustive, pin_page_scale_bytes, pin_hand_worked_row,
            pin_quant_byte_range, pin_brute_force, pin_page_shape, pin_zero_scale,
            pin_all_ones, pin_integer_exact, pin_specials, pin_symmetries, pin_gemm_rows]
