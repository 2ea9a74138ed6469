"""The C-ABI library loads, exports every declared entry point, and refuses
bad arguments before touching any device (no GPU is needed here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8gemv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_0_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def q8():
    import q8_block_quantized_gemv_amd as q8mod
    return q8mod


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("q8_0_gemv", "q8_0_gemm_smallm", "q8_0_decode_chain",
                     "q8_0_chain_create", "q8_0_chain_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol(q8):
    lib = ctypes.CDLL(q8.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(q8.EXPORTS)


def test_status_strings(q8):
    for code in range(0, -9, -1):
        assert q8.lib.q8_0_status_string(code).decode() != "unknown status"
    assert q8.lib.q8_0_status_string(-99).decode() == "unknown status"


# fake, never-dereferenced addresses: validation rejects before any HIP call
X, W, Y = 0x10000000, 0x20000000, 0x30000000


@pytest.mark.parametrize("args,code", [
    ((0, W, Y, 64, 4), -1),            # null x
    ((X, 0, Y, 64, 4), -1),            # null w
    ((X, W, 0, 64, 4), -1),            # null y
    ((X, W, Y, 0, 4), -2),             # n = 0
    ((X, W, Y, 33, 4), -2),            # n not a multiple of 32
    ((X, W, Y, -32, 4), -2),
    ((X, W, Y, (1 << 20) + 32, 4), -2),  # n too large
    ((X, W, Y, 64, 0), -2),            # p = 0
    ((X, W, Y, 64, -1), -2),
    ((X, W, Y, 64, 1 << 31), -2),      # p too large
    ((X, W + 8, Y, 64, 4), -3),        # w not 16-byte aligned
    ((X + 2, W, Y, 64, 4), -3),        # x not 16-byte aligned
    ((X + 4, W, Y, 64, 4), -3),
    ((X, W, Y + 1, 64, 4), -3),
    ((X, W, X + 16, 64, 4), -4),       # y overlaps x
    ((X, W, X - 4, 64, 4), -4),        # y's last element is x[0]
    ((X, W, W + 68, 64, 4), -4),       # y overlaps w
])
def test_gemv_validation(q8, args, code):
    assert q8.gemv_raw(*args) == code
    assert q8.last_error() != ""


@pytest.mark.parametrize("m,code", [(0, -2), (17, -2), (-1, -2)])
def test_gemm_validation(q8, m, code):
    assert q8.gemm_smallm_raw(X, W, Y, m, 64, 4) == code


def test_gemm_alias_counts_all_rows(q8):
    # Y of m rows reaches into x only through its later rows
    assert q8.gemm_smallm_raw(X, W, X - 4 * 4 * 3, 4, 64, 4) == -4


def test_chain_validation(q8):
    h = ctypes.c_void_p()
    ops = (q8.Q8Op * 2)(q8.Q8Op(X, W, Y, 64, 4), q8.Q8Op(X, W, Y, 63, 4))
    assert q8.lib.q8_0_chain_create(ops, 2, 0, ctypes.byref(h)) == -2
    assert h.value is None
    assert "op 1" in q8.last_error()
    assert q8.lib.q8_0_chain_create(ops, 0, 0, ctypes.byref(h)) == -1
    assert q8.lib.q8_0_chain_create(ops, 1, 7, ctypes.byref(h)) == -1
    assert q8.lib.q8_0_chain_create(None, 1, 0, ctypes.byref(h)) == -1
    assert q8.lib.q8_0_decode_chain(None, 0, None) == -1
    assert q8.lib.q8_0_chain_launches(None) == -1
    assert q8.lib.q8_0_chain_destroy(None) == 0


def test_no_device_path(q8):
    """Valid arguments on a machine without a GPU: a clean NO_DEVICE."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is visible")
    assert q8.gemv_raw(X, W, Y, 64, 4) == -5
    assert q8.gemm_smallm_raw(X, W, Y, 2, 64, 4) == -5
