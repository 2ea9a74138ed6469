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


# ---------------------------------------------------------------- activations as Q8_0
def _f16_bits(v):
    return int(np.asarray(v, np.float32).astype(np.float16).view(np.uint16))


def _blocks(xq):
    """(scale as float64, quants as int64) of Q8_0 bytes, decoded with numpy."""
    blk = np.asarray(xq, np.uint8).reshape(-1, 34)
    d = blk[:, 0:2].copy().view("<f2").astype(np.float64)[:, 0]
    q = blk[:, 2:].copy().view(np.int8).astype(np.int64)
    return d, q


def pin_f16_encode(o):
    """float32 -> binary16 against numpy's cast (nearest, ties to even): every
    midpoint between consecutive finite binary16 values (the ties), the
    values themselves, and random magnitudes from below the subnormals to
    past the largest finite value."""
    h = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2.0                  # exact in float32 (12 bits)
    rng = np.random.default_rng(31)
    rand = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 4000))
    vals = np.concatenate([h[::7], mids[::3], mids[-50:], mids[:50], rand, [65504.0, 65519.0, 65520.0, 1e6]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([o.f32_to_f16(float(v)) for v in vals], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "f32 %r -> 0x%04x, numpy 0x%04x" % (float(vals[bad[0]]), got[bad[0]], ref[bad[0]])


def pin_quantize_closed_forms(o):
    """Blocks whose scale is a power of two times 127 quantize to the exact
    integers; halves round away from zero; an all-zero block is all zero
    bytes; each block has its own scale."""
    k = np.arange(-16, 16, dtype=np.float64)
    k[0] = -127.0                                  # the block's largest magnitude
    blk0 = (k * 2.0 ** -3).astype(np.float32)       # d = 2^-3 exactly
    ties = np.zeros(32)
    ties[:7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -126.5]   # d = 1
    blk1 = ties.astype(np.float32)
    blk2 = np.zeros(32, np.float32)
    k3 = np.arange(32, dtype=np.float64) * 4.0 - 3.0
    k3[31] = 127.0
    blk3 = (k3 * 2.0 ** 4).astype(np.float32)       # d = 16
    xq = o.quantize_x(np.concatenate([blk0, blk1, blk2, blk3]))
    b = np.asarray(xq).reshape(4, 34)
    assert int(b[0, 0]) | (int(b[0, 1]) << 8) == _f16_bits(2.0 ** -3)
    assert np.array_equal(b[0, 2:].view(np.int8), k.astype(np.int8))
    assert int(b[1, 0]) | (int(b[1, 1]) << 8) == 0x3C00
    assert list(b[1, 2:9].view(np.int8)) == [127, 3, -3, 1, -1, 2, -127]
    assert not b[2].any()
    assert int(b[3, 0]) | (int(b[3, 1]) << 8) == _f16_bits(16.0)
    assert np.array_equal(b[3, 2:].view(np.int8), k3.astype(np.int8))


def pin_quantize_error_bound(o):
    """On random blocks: the largest magnitude maps to +-127, every quant
    lies in [-127, 127], and dequantizing with the unrounded float32 scale
    d = amax/127 misses x by at most d/2 (plus the scale division's own
    rounding); the stored scale is that d in binary16."""
    rng = np.random.default_rng(32)
    x = (rng.standard_normal(32 * 200) * np.repeat(np.exp(rng.uniform(-6, 6, 200)), 32)).astype(np.float32)
    d16, q = _blocks(o.quantize_x(x))
    xb = x.reshape(200, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=1)
    d = amax / 127.0
    assert np.all(np.abs(q) <= 127) and np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(xb - d[:, None] * q)
    assert np.all(err <= d[:, None] * (0.5 + 1e-6)), float((err / d[:, None]).max())
    assert np.all(np.abs(d16 - d) <= d * 2.0 ** -11 + 2.0 ** -25)
    # the sign of every non-zero quant is the sign of x
    nz = q != 0
    assert np.all(np.sign(q[nz]) == np.sign(xb[nz]))


def pin_q8q8_brute_force(o):
    """The integer matvec against a dense float64 product of the weights and
    the quantized x, both decoded with numpy; the quantized x is the
    oracle's own (pinned above)."""
    rng = np.random.default_rng(33)
    for n, p in [(32, 5), (96, 17), (256, 9)]:
        w = synth.q8_weights(n, p, rng)
        x = synth.activations(n, rng)
        d, q = _blocks(o.quantize_x(x))
        xhat = (d[:, None] * q).reshape(-1)
        ry, rmag = dense_reference(w, xhat.astype(np.float64), n, p)
        y, y64, mag = o.gemv_q8q8(w, x, n, p)
        assert np.all(np.abs(y64 - ry) <= 1e-12 * rmag + 1e-300)
        assert np.allclose(mag, rmag, rtol=1e-12, atol=0)
        assert np.array_equal(y, y64.astype(np.float32))


def pin_q8q8_near_float(o):
    """The integer matvec differs from the float matvec only by x's
    quantization error: |y_q8q8 - y_f32| <= sum_j |w_j| |x_j - xhat_j|."""
    rng = np.random.default_rng(34)
    n, p = 512, 40
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    d, q = _blocks(o.quantize_x(x))
    xhat = (d[:, None] * q).reshape(-1)
    nb = n // 32
    blk = w.reshape(p * nb, 34)
    dw = blk[:, 0:2].copy().view("<f2").astype(np.float64).reshape(p, nb)
    qw = blk[:, 2:].copy().view(np.int8).astype(np.float64).reshape(p, nb, 32)
    absw = np.abs(dw[:, :, None] * qw).reshape(p, n)
    bound = absw @ np.abs(x.astype(np.float64) - xhat)
    _, yq, magq = o.gemv_q8q8(w, x, n, p)
    _, yf, magf = o.gemv(w, x, n, p)
    assert np.all(np.abs(yq - yf) <= bound + 1e-12 * (magq + magf))
    assert np.all(bound < 0.05 * magf)     # and the error is small


def pin_q8q8_integer_exact(o):
    """Unit weight scales and integer activations whose blocks each reach
    127: the quantized x is x itself and y is the exact integer sum."""
    rng = np.random.default_rng(35)
    n, p = 192, 11
    nb = n // 32
    xi = rng.integers(-127, 128, size=n)
    xi[::32] = 127
    qw = rng.integers(-127, 128, size=(p * nb, 32)).astype(np.int8)
    w = synth.pack_blocks(np.full(p * nb, 1.0, np.float16), qw)
    y, y64, mag = o.gemv_q8q8(w, xi.astype(np.float32), n, p)
    exact = qw.astype(np.int64).reshape(p, n) @ xi.astype(np.int64)
    assert np.array_equal(y64, exact.astype(np.float64))
    assert np.array_equal(mag, (np.abs(qw.astype(np.int64).reshape(p, n)) @ np.abs(xi)).astype(np.float64))


ALL_PINS = [pin_f16_exhaustive, pin_page_scale_bytes, pin_hand_worked_row,
            pin_quant_byte_range, pin_brute_force, pin_page_shape, pin_zero_scale,
            pin_all_ones, pin_integer_exact, pin_specials, pin_symmetries, pin_gemm_rows,
            pin_f16_encode, pin_quantize_closed_forms, pin_quantize_error_bound,
            pin_q8q8_brute_force, pin_q8q8_near_float, pin_q8q8_integer_exact]
