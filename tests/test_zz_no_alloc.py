"""The allocation-free small-batch entry point (q8_0_gemm_smallm_noalloc):
the same results as q8_0_gemm_smallm with a caller workspace, bit for bit,
on two calls in a row (the second smaller, so the scratch holds the first
call's leftovers), no change in free device memory across calls, and a
clear refusal of a shape that needs more scratch than the library holds."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import down, log, parity, up, w_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q8():
    import q8_block_quantized_gemv_amd as mod
    return mod


def _case(q8, m, n, p, seed):
    import torch
    rng = np.random.default_rng(seed)
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m).reshape(m, n)
    return w, X, w_dev(w, n, p), up(X), torch.empty((m, p), dtype=torch.float32, device="cuda")


def _noalloc(q8, Xd, wd, Y, m, n, p):
    s = q8._stream_handle(None)
    return q8.lib.q8_0_gemm_smallm_noalloc(Xd.data_ptr(), wd.data_ptr(), Y.data_ptr(), m, n, p, s)


@pytest.mark.parametrize("first,second", [
    ((16, 18944, 3584), (3, 3584, 300)),      # matrix cores, then two rows on the vector units
    ((4, 3584, 18944), (2, 896, 71)),         # then a width of 28 blocks with a tail row
    ((6, 192, 37), (5, 160, 11)),             # vector units with 4- and 8-row super-rows
])
def test_noalloc_equals_workspace_call(q8, first, second):
    import torch
    for k, (m, n, p) in enumerate((first, second)):
        log("noalloc m=%d n=%d p=%d (call %d)" % (m, n, p, k))
        w, X, wd, Xd, Y = _case(q8, m, n, p, 1000 + 7 * k + m + n + p)
        Y.fill_(float("nan"))
        assert _noalloc(q8, Xd, wd, Y, m, n, p) == 0, q8.last_error()
        got = down(Y).copy()
        ref = torch.full_like(Y, float("nan"))
        q8.gemm_smallm(Xd, wd, ref)
        assert np.array_equal(got.view(np.uint32), down(ref).view(np.uint32))
        if m * n * p <= 16 * 3584 * 300:     # and the oracle, where it is quick
            _, Y64, MAG = oracle.gemm(w, X, m, n, p)
            for i in range(m):
                parity(got[i], Y64[i], MAG[i], "noalloc row %d" % i)


def test_noalloc_keeps_to_its_scratch(q8):
    """The 7B lm_head at m = 16: q8_0_gemm_smallm holds X in LDS and needs
    48.7 MB for its per-range sums; the allocation-free call, whose scratch
    is 32 MiB, runs the stream-K matrix cores instead -- bitwise what that
    kernel gives through a workspace -- and both meet the bar on sampled
    rows."""
    import torch
    m, n, p = 16, 3584, 152064
    log("noalloc m=%d n=%d p=%d (held X needs more than the scratch)" % (m, n, p))
    assert q8.gemm_smallm_choice(m, n, p) == q8.SMALLM_KS
    w, X, wd, Xd, Y = _case(q8, m, n, p, 4242)
    Y.fill_(float("nan"))
    assert _noalloc(q8, Xd, wd, Y, m, n, p) == 0, q8.last_error()
    got = down(Y).copy()
    ref = torch.full_like(Y, float("nan"))
    q8.gemm_smallm(Xd, wd, ref, kernel=q8.SMALLM_MFMA)
    assert np.array_equal(got.view(np.uint32), down(ref).view(np.uint32))
    ks = torch.full_like(Y, float("nan"))
    q8.gemm_smallm(Xd, wd, ks)
    ks = down(ks)
    rows = np.random.default_rng(7).choice(p, 64, replace=False)
    rb = n // 32 * 34
    sub = np.ascontiguousarray(w.reshape(p, rb)[rows]).reshape(-1)
    _, Y64, MAG = oracle.gemm(sub, X, m, n, len(rows))
    for i in range(m):
        parity(got[i, rows], Y64[i], MAG[i], "noalloc lm_head row %d" % i)
        parity(ks[i, rows], Y64[i], MAG[i], "held-X lm_head row %d" % i)


def test_noalloc_allocates_nothing(q8):
    import torch
    cases = [_case(q8, m, n, p, 50 + m) for m, n, p in ((16, 18944, 3584), (2, 3584, 18944), (5, 3584, 4608))]
    for w, X, wd, Xd, Y in cases:
        m, n = Xd.shape
        assert _noalloc(q8, Xd, wd, Y, m, n, Y.shape[1]) == 0
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        for w, X, wd, Xd, Y in cases:
            m, n = Xd.shape
            assert _noalloc(q8, Xd, wd, Y, m, n, Y.shape[1]) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_noalloc_refuses_past_its_scratch(q8):
    """m = 4 at n = 2^20 - 128 (rows of two per super-row) runs on the
    stream-K matrix cores, whose split of X alone takes 96 MiB: refused
    before anything is enqueued."""
    import torch
    m, n, p = 4, (1 << 20) - 128, 64
    need = q8.gemm_smallm_workspace(m, n, p)
    assert need > 32 << 20
    X = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    w = torch.zeros((p, (n // 32) * 34), dtype=torch.uint8, device="cuda")
    Y = torch.full((m, p), 3.0, dtype=torch.float32, device="cuda")
    assert _noalloc(q8, X, w, Y, m, n, p) == q8.Q8_ERR_SHAPE
    assert str(need) in q8.last_error()
    assert bool((down(Y) == 3.0).all())
