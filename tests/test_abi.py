"""The C-ABI library loads, exports every declared entry point, and refuses
bad arguments before touching any device (no GPU is needed here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("q8gemv.h", "q8step.h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(q8_0_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def q8():
    import q8_block_quantized_gemv_amd as q8mod
    return q8mod


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("q8_0_gemv", "q8_0_gemm_smallm", "q8_0_decode_chain",
                     "q8_0_chain_create", "q8_0_chain_destroy", "q8_0_rms_norm",
                     "q8_0_attention_decode", "q8_0_argmax", "q8_0_step_create",
                     "q8_0_step_run"):
        assert required in names


def test_library_exports_every_declared_symbol(q8):
    lib = ctypes.CDLL(q8.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(q8.EXPORTS)


def test_library_exports_nothing_else(q8):
    """The shared library's exported functions are exactly the C ABI."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm is not installed")
    out = subprocess.run(["nm", "-D", "--defined-only", q8.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {parts[2] for parts in (l.split() for l in out.splitlines())
                if len(parts) == 3 and parts[1] == "T"}
    assert exported == set(declared_functions())


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


@pytest.mark.parametrize("args,code", [
    ((0, W, Y, 64, 4), -1), ((X, W, Y, 33, 4), -2), ((X, W, Y, 64, 0), -2),
    ((X, W + 8, Y, 64, 4), -3), ((X, W, X + 16, 64, 4), -4),
])
def test_gemv_q8q8_validation(q8, args, code):
    assert q8.lib.q8_0_gemv_q8q8(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((0, Y, 64), -1), ((X, 0, 64), -1), ((X, Y, 0), -2), ((X, Y, 48), -2),
    ((X, Y, (1 << 31) + 32), -2), ((X + 2, Y, 64), -3), ((X, X + 100, 64), -4),
])
def test_quantize_validation(q8, args, code):
    assert q8.lib.q8_0_quantize(*args, None) == code


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
    assert q8.lib.q8_0_chain_create(ops, 1, 8, ctypes.byref(h)) == -1   # no flag 8 any more
    assert q8.lib.q8_0_chain_create(ops, 1, 16, ctypes.byref(h)) == -1
    assert "unknown flags" in q8.last_error()
    assert q8.lib.q8_0_chain_create(None, 1, 0, ctypes.byref(h)) == -1
    assert q8.lib.q8_0_decode_chain(None, 0, None) == -1
    assert q8.lib.q8_0_chain_launches(None) == -1
    assert q8.lib.q8_0_chain_destroy(None) == 0


@pytest.mark.parametrize("c,waves,st,n,code", [
    (3, 1, 1, 256, -1), (1, 3, 1, 256, -1), (0, 1, 1, 256, -1), (8, 1, 1, 256, -1),  # not 1, 2, 4
    (1, 1, 0, 256, -1), (1, 1, 3, 256, -1),                                        # stages not 1, 2
    (4, 4, 2, 256, -1),                                                            # LDS past 160 KiB
    (4, 4, 1, 96, -2), (4, 4, 1, 896, -2),                                         # n % 256 != 0
    (4, 4, 1, 0, -2), (1, 1, 1, 33, -2),                                           # as q8_0_gemv
])
def test_gemv_shaped_validation(q8, c, waves, st, n, code):
    assert q8.lib.q8_0_gemv_shaped(X, W, Y, n, 4, c, waves, st, None) == code
    assert q8.last_error() != ""


@pytest.mark.parametrize("m,n,kernel,code", [
    (2, 256, 6, -1), (2, 256, -1, -1),          # unknown kernel
    (2, 896, 5, -2),                            # X held in LDS: rows of whole groups
    (4, 256, 3, -2), (4, 256, 4, -2),           # the row-and-block-pair kernel takes m <= 3
    (2, 896, 3, -2),                            # ... and rows of whole groups (n % 256 == 0)
    (2, 96, 2, -2),                             # the matrix cores take rows of 1 or 2 per super-row
    (1, 256, 2, -2), (1, 256, 1, -2),           # m = 1 is the matvec's
    (17, 256, 0, -2),                           # m as q8_0_gemm_smallm
])
def test_gemm_kernel_validation(q8, m, n, kernel, code):
    assert q8.lib.q8_0_gemm_smallm_kernel(X, W, Y, m, n, 4, kernel, None, 0, None) == code


def test_no_device_path(q8):
    """Valid arguments on a machine without a GPU: a clean NO_DEVICE."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is visible")
    assert q8.gemv_raw(X, W, Y, 64, 4) == -5
    assert q8.gemm_smallm_raw(X, W, Y, 2, 64, 4) == -5
    assert q8.lib.q8_0_rms_norm(X, W, Y, 64, 1, 1e-6, None) == -5
    assert q8.lib.q8_0_argmax(X, 8, Y, WS, 1 << 20, None) == -5
    assert q8.lib.q8_0_attention_decode(X, W, F, Y, 8, 128, 64, 2, 1, WS, 1 << 20, None) == -5
    assert q8.lib.q8_0_gemm_smallm(X, W, Y, 2, 64, 4, WS, 1 << 20, None) == -5
    k = ctypes.c_int(-7)
    assert q8.lib.q8_0_gemm_smallm_choice(2, 256, 4, ctypes.byref(k)) == -5
    layers = (q8.Q8LayerW * 1)(_layer(q8))
    h = ctypes.c_void_p()
    assert q8.lib.q8_0_step_create(ctypes.byref(_model(q8, layers)), ctypes.byref(h)) == -5


# ------------------------------------------------------------------ the decode-step calls
F = 0x40000000   # another fake, 256-B aligned address
WS = 0x50000000  # a fake workspace


@pytest.mark.parametrize("call,code", [
    (lambda L: L.q8_0_rms_norm(0, W, Y, 64, 1, 1e-6, None), -1),
    (lambda L: L.q8_0_rms_norm(X, W, Y, 0, 1, 1e-6, None), -2),
    (lambda L: L.q8_0_rms_norm(X, W, Y, 64, 0, 1e-6, None), -2),
    (lambda L: L.q8_0_rms_norm(X, W, Y, 65537, 1, 1e-6, None), -2),
    (lambda L: L.q8_0_rms_norm(X + 2, W, Y, 64, 1, 1e-6, None), -3),
    (lambda L: L.q8_0_rms_norm(X, W, X + 8, 64, 1, 1e-6, None), -4),   # partial overlap
    (lambda L: L.q8_0_rms_norm(X, W, W + 4, 64, 1, 1e-6, None), -4),
    (lambda L: L.q8_0_rms_norm(X, W, Y, 64, 1, -1.0, None), -1),
    (lambda L: L.q8_0_rope(0, 64, 1, 0, 1e4, None), -1),
    (lambda L: L.q8_0_rope(X, 63, 1, 0, 1e4, None), -2),
    (lambda L: L.q8_0_rope(X, 64, 0, 0, 1e4, None), -2),
    (lambda L: L.q8_0_rope(X, 64, 1, -1, 1e4, None), -2),
    (lambda L: L.q8_0_rope(X, 64, 1, 0, 0.0, None), -1),
    (lambda L: L.q8_0_append_kv(X, 0, Y, F, 64, 0, None), -1),
    (lambda L: L.q8_0_append_kv(X, W, Y, F, 64, 65536, None), -2),
    (lambda L: L.q8_0_append_kv(X, W, Y + 2, F, 64, 0, None), -3),
    (lambda L: L.q8_0_attention_decode(X, W, F, 0, 8, 128, 64, 2, 1, None, 0, None), -1),
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 8, 128, 96, 2, 1, None, 0, None), -2),   # head_dim
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 8, 128, 64, 3, 2, None, 0, None), -2),   # n_heads % group
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 8, 64, 64, 2, 1, None, 0, None), -2),    # kv_width
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 0, 128, 64, 2, 1, None, 0, None), -2),
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 65537, 128, 64, 2, 1, None, 0, None), -2),
    (lambda L: L.q8_0_attention_decode(X, W, F, X + 4, 8, 128, 64, 2, 1, None, 0, None), -4),
    (lambda L: L.q8_0_attention_decode(X + 4, W, F, Y, 8, 128, 64, 2, 1, None, 0, None), -3),  # q not 16-B
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 8, 130, 64, 2, 1, None, 0, None), -3),      # kv_width % 4
    (lambda L: L.q8_0_add_inplace(X, 0, 8, None), -1),
    (lambda L: L.q8_0_add_inplace(X, X + 4, 8, None), -4),
    (lambda L: L.q8_0_add_inplace(X, Y, 0, None), -2),
    (lambda L: L.q8_0_silu_hadamard(X, W, X + 4, 8, None), -4),
    (lambda L: L.q8_0_silu_hadamard(X, W, Y, -3, None), -2),
    (lambda L: L.q8_0_argmax(X, 0, Y, None, 0, None), -2),
    (lambda L: L.q8_0_argmax(X, 8, X + 4, None, 0, None), -4),
    (lambda L: L.q8_0_argmax(X, 8, Y + 1, None, 0, None), -3),
])
def test_step_op_validation(q8, call, code):
    assert call(q8.lib) == code
    assert q8.last_error() != ""


def _layer(q8):
    return q8.Q8LayerW(*([W] * 7 + [X] * 4))


def _model(q8, layers, **kw):
    base = dict(n_layers=1, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, inter=512,
                vocab=1000, max_seq=64, eps=1e-6, theta=1e6)
    base.update(kw)
    return q8.Q8Model(base["n_layers"], base["hidden"], base["n_heads"], base["n_kv_heads"],
                      base["head_dim"], base["inter"], base["vocab"], base["max_seq"],
                      base["eps"], base["theta"], F, F, W, layers)


@pytest.mark.parametrize("kw", [
    dict(n_layers=0), dict(head_dim=96), dict(n_heads=3), dict(n_kv_heads=0),
    dict(hidden=250), dict(inter=0), dict(vocab=0), dict(max_seq=0), dict(max_seq=65537),
    dict(eps=-1.0), dict(theta=0.0),
])
def test_step_create_validation(q8, kw):
    layers = (q8.Q8LayerW * 1)(_layer(q8))
    m = _model(q8, layers, **kw)
    h = ctypes.c_void_p()
    assert q8.lib.q8_0_step_create(ctypes.byref(m), ctypes.byref(h)) in (-1, -2)
    assert h.value is None


def test_step_create_null_weight(q8):
    L = _layer(q8)
    L.wdown = None
    layers = (q8.Q8LayerW * 1)(L)
    m = _model(q8, layers)
    h = ctypes.c_void_p()
    assert q8.lib.q8_0_step_create(ctypes.byref(m), ctypes.byref(h)) == -1
    assert "layer 0" in q8.last_error()
    assert q8.lib.q8_0_step_create(None, ctypes.byref(h)) == -1
    assert q8.lib.q8_0_step_run(None, 0, None) == -1
    assert q8.lib.q8_0_step_reset(None, 0, 0, None) == -1
    assert q8.lib.q8_0_step_launches(None) == -1
    assert q8.lib.q8_0_step_destroy(None) == 0


# ------------------------------------------------------------------ caller-owned workspaces
def _align256(b):
    return (b + 255) // 256 * 256


def _query(fn, *args):
    out = ctypes.c_size_t(0)
    rc = fn(*args, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("seq,hd,nh", [(1, 64, 1), (128, 128, 16), (129, 128, 16), (2048, 128, 28),
                                       (4097, 256, 3)])
def test_attention_workspace_size(q8, seq, hd, nh):
    """Per-head arrival counters, then (m, s, acc[head_dim]) per (head, chunk of 128 rows)."""
    rc, b = _query(q8.lib.q8_0_attention_workspace, seq, hd, nh)
    assert rc == 0
    chunks = -(-seq // 128)
    assert b == _align256(4 * nh) + _align256(4 * nh * chunks * (hd + 2))


@pytest.mark.parametrize("n", [1, 4096, 4097, 151936, 1 << 20, (1 << 31) - 1])
def test_argmax_workspace_size(q8, n):
    """A counter, then one (value, index) per workgroup of up to 4096 values (at most 256)."""
    rc, b = _query(q8.lib.q8_0_argmax_workspace, n)
    assert rc == 0
    wgs = max(1, min(256, -(-n // 4096)))
    assert b == 256 + 2 * _align256(4 * wgs)


def test_workspace_queries_refuse(q8):
    L = q8.lib
    assert L.q8_0_attention_workspace(8, 64, 2, None) == -1
    assert _query(L.q8_0_attention_workspace, 0, 64, 2)[0] == -2
    assert _query(L.q8_0_attention_workspace, 8, 0, 2)[0] == -2
    assert L.q8_0_argmax_workspace(8, None) == -1
    assert _query(L.q8_0_argmax_workspace, 0)[0] == -2
    assert L.q8_0_gemm_smallm_workspace(2, 256, 4, 0, None) == -1
    assert _query(L.q8_0_gemm_smallm_workspace, 17, 256, 4, 0)[0] == -2
    assert _query(L.q8_0_gemm_smallm_workspace, 2, 48, 4, 0)[0] == -2
    assert _query(L.q8_0_gemm_smallm_workspace, 2, 256, 4, 9)[0] == -1     # unknown kernel
    assert _query(L.q8_0_gemm_smallm_workspace, 4, 256, 4, 3)[0] == -2     # kernel does not take m
    k = ctypes.c_int(-7)
    assert L.q8_0_gemm_smallm_choice(2, 256, 4, None) == -1
    assert L.q8_0_gemm_smallm_choice(1, 256, 4, ctypes.byref(k)) == -2 and k.value == 0   # m = 1 is the matvec's
    assert L.q8_0_gemm_smallm_choice(17, 256, 4, ctypes.byref(k)) == -2
    assert L.q8_0_gemm_smallm_choice(2, 48, 4, ctypes.byref(k)) == -2


@pytest.mark.parametrize("call,code", [
    # null, misaligned, too small, overlapping an operand
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 200, 128, 64, 2, 1, None, 1 << 20, None), -3),
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 200, 128, 64, 2, 1, WS + 16, 1 << 20, None), -3),
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 200, 128, 64, 2, 1, WS, 256, None), -1),
    (lambda L: L.q8_0_attention_decode(X, W, F, Y, 200, 128, 64, 2, 1, Y - 256, 1 << 20, None), -4),
    (lambda L: L.q8_0_argmax(X, 8, Y, None, 1 << 20, None), -3),
    (lambda L: L.q8_0_argmax(X, 8, Y, WS + 4, 1 << 20, None), -3),
    (lambda L: L.q8_0_argmax(X, 8, Y, WS, 100, None), -1),
    (lambda L: L.q8_0_argmax(X, 8, Y, X - 512, 1 << 20, None), -4),
])
def test_workspace_validation(q8, call, code):
    assert call(q8.lib) == code
    assert "workspace" in q8.last_error()
