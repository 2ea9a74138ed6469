"""Planted mistakes in the oracle must be caught by the pins.

Each mutant is a copy of oracle/q8_0_oracle.c with one plausible mistake
(a dropped term, a wrong sign, a wrong index or offset, a wrong byte order, a
lost sign extension, a single-precision accumulator), compiled with gcc into a
temporary directory.  The real oracle is never modified.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "unsigned_quant": ("int q = (int)(int8_t)blk[2 + j];", "int q = (int)blk[2 + j];"),
    "dropped_block_offset_in_x": ("x[b * Q8O_BLOCK_QUANTS + j]", "x[j]"),
    "big_endian_scale": ("(uint16_t)(blk[0] | ((uint16_t)blk[1] << 8))",
                         "(uint16_t)(blk[1] | ((uint16_t)blk[0] << 8))"),
    "exponent_bias_off_by_one": ("e - 25", "e - 24"),
    "dropped_hidden_bit": ("(double)(1024 + f)", "(double)(f)"),
    "subnormal_scale_wrong": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "sign_dropped": ("return s ? -v : v;", "return v;"),
    "quant_offset": ("blk[2 + j]", "blk[1 + j]"),
    "row_stride": ("w + r * row_bytes", "w + r * (row_bytes - 2)"),
    "subtract_term": ("acc += d * s;", "acc -= d * s;"),
    "scale_dropped": ("acc += d * s;", "acc += s;"),
    "inner_sum_dropped_term": ("s += t;", "s += (j == 31) ? 0.0 : t;"),
    "dropped_last_quant": ("for (int j = 0; j < Q8O_BLOCK_QUANTS; ++j) {",
                           "for (int j = 0; j < Q8O_BLOCK_QUANTS - 1; ++j) {"),
    "float_accumulator": ("double acc = 0.0;", "float acc = 0.0f;"),
    "nan_as_inf": ("(f == 0) ? INFINITY : NAN", "INFINITY"),
    "gemm_x_stride": ("X + i * n", "X + i"),
    "quant_half_even": ("q = (int)roundf(t);", "q = (int)nearbyintf(t);"),
    "quant_truncate": ("q = (int)roundf(t);", "q = (int)t;"),
    "amax_signed": ("float a = fabsf(xb[j]);", "float a = xb[j];"),
    "quant_scale_128": ("amax / 127.0f", "amax / 128.0f"),
    "f16_round_down": ("nearbyint(a / ulp)", "floor(a / ulp)"),
    "f16_spacing": ("ldexp(1.0, e - 10)", "ldexp(1.0, e - 11)"),
    "f16_no_subnormal_floor": ("    if (e < -14)\n        e = -14;\n", ""),
    "xq_scale_bytes_swapped": ("o[0] = (uint8_t)(db & 0xff);", "o[0] = (uint8_t)(db >> 8);"),
    "q8q8_dx_dropped": ("acc += (dw * dx) * (double)isum;", "acc += dw * (double)isum;"),
    "q8q8_unsigned_x": ("(int64_t)(int8_t)xb[2 + j]", "(int64_t)xb[2 + j]"),
    "q8q8_x_block_offset": ("xq + b * Q8O_BLOCK_BYTES", "xq"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, "mutation site vanished: %r" % old
    mutated = src.replace(old, new)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.compile_oracle(path, os.path.join(tmp_path, "libmutant_%s.so" % name),
                                 werror=False)
    o = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % name
