"""Calls whose kernels need scratch memory take it from the caller and
allocate nothing of their own: repeated small-batch products across the 7B
projection shapes and m = 2..16 leave the device's free memory unchanged,
and the small-batch product, the standalone attention and argmax record into
a hipGraph under global stream capture (which refuses device allocation,
freeing and synchronization) whose replays equal the eager result bit for
bit, replay after replay, with eager work in between."""
import numpy as np
import pytest

import synth
from tests.gpu_util import down, log, up, w_dev

pytestmark = pytest.mark.gpu

# the 7B projections (q|k|v, gate/up, down) and a ragged row count
SHAPES = [(3584, 4608), (3584, 18944), (18944, 3584), (3584, 300)]


@pytest.fixture(scope="module")
def q8():
    import q8_block_quantized_gemv_amd as mod
    return mod


def _cases(q8, ms, rng):
    import torch
    out = []
    for n, p in SHAPES:
        wd = w_dev(synth.q8_weights(n, p, rng), n, p)
        for m in ms:
            X = up(synth.activations(n, rng, m).reshape(m, n))
            Y = torch.empty((m, p), dtype=torch.float32, device="cuda")
            out.append((wd, X, Y, m, n, p))
    return out


def test_smallm_repeated_calls_allocate_nothing(q8):
    import torch
    log("smallm repeated calls, free device memory before and after")
    cases = _cases(q8, (2, 3, 4, 5, 8, 16), np.random.default_rng(71))
    need = max(q8.gemm_smallm_workspace(m, n, p) for _, _, _, m, n, p in cases)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def run_all():
        for wd, X, Y, m, n, p in cases:
            q8.check(q8.lib.q8_0_gemm_smallm(X.data_ptr(), wd.data_ptr(), Y.data_ptr(), m, n, p,
                                             ws.data_ptr(), ws.numel(), s))

    run_all()                      # first launches of each kernel load their code
    torch.cuda.synchronize()
    first = [down(Y).copy() for _, _, Y, _, _, _ in cases]
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        run_all()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    for (_, _, Y, m, n, p), y0 in zip(cases, first):
        assert np.array_equal(down(Y).view(np.uint32), y0.view(np.uint32)), (m, n, p)


def test_smallm_workspace_too_small_is_refused(q8):
    """Workspace errors, on a call that needs one (n = 18944 at m = 4 cuts the
    columns into several ranges, whose sums the workspace holds)."""
    import torch
    n, p, m = 18944, 300, 4
    rng = np.random.default_rng(5)
    wd = w_dev(synth.q8_weights(n, p, rng), n, p)
    X = up(synth.activations(n, rng, m).reshape(m, n))
    need = q8.gemm_smallm_workspace(m, n, p)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    Y = torch.empty((m, p), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L = q8.lib
    assert L.q8_0_gemm_smallm(X.data_ptr(), wd.data_ptr(), Y.data_ptr(), m, n, p, ws.data_ptr(), need - 1,
                              s) == q8.Q8_ERR_INVALID_ARG
    assert L.q8_0_gemm_smallm(X.data_ptr(), wd.data_ptr(), Y.data_ptr(), m, n, p, None, need,
                              s) == q8.Q8_ERR_ALIGN
    assert L.q8_0_gemm_smallm(X.data_ptr(), wd.data_ptr(), Y.data_ptr(), m, n, p, ws.data_ptr() + 16, need,
                              s) == q8.Q8_ERR_ALIGN
    assert L.q8_0_gemm_smallm(X.data_ptr(), wd.data_ptr(), Y.data_ptr(), m, n, p, Y.data_ptr(), need,
                              s) == q8.Q8_ERR_ALIAS
    # m = 1 is the matvec: no workspace at all
    assert q8.gemm_smallm_workspace(1, n, p) == 0
    assert L.q8_0_gemm_smallm(X.data_ptr(), wd.data_ptr(), Y.data_ptr(), 1, n, p, None, 0, s) == 0
    torch.cuda.synchronize()


def _replays_equal_eager(q8, label, run, outs, replays=3):
    """Record run() under global capture; every replay, with eager work and
    synchronizations between, equals the eager result bit for bit."""
    import torch
    run()
    torch.cuda.synchronize()
    eager = [down(o).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):    # capture_error_mode "global"
        run()
    junk = torch.randn(1 << 20, device="cuda")
    for k in range(replays):
        for o in outs:
            o.fill_(float("nan") if o.dtype.is_floating_point else -7)
        torch.cuda.synchronize()
        g.replay()
        junk.mul_(1.0001)         # eager work between replays
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(down(o).view(np.uint32), e.view(np.uint32)), "%s replay %d" % (label, k)
        run()                     # and an eager call again
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(down(o).view(np.uint32), e.view(np.uint32)), "%s eager %d" % (label, k)


@pytest.mark.parametrize("m,kernel", [(2, "VROW"), (3, "VROW1"), (4, "VALU"), (6, "VALU"), (5, "MFMA"),
                                      (16, "MFMA"), (8, "KS"), (16, "KS"), (2, None), (16, None)])
def test_smallm_under_capture(q8, m, kernel):
    import torch
    log("smallm under capture m=%d kernel=%s" % (m, kernel))
    k = getattr(q8, "SMALLM_" + kernel) if kernel else q8.SMALLM_AUTO
    rng = np.random.default_rng(900 + m)
    runs, outs = [], []
    for n, p in ((3584, 300), (18944, 700)):
        wd = w_dev(synth.q8_weights(n, p, rng), n, p)
        X = up(synth.activations(n, rng, m).reshape(m, n))
        Y = torch.empty((m, p), dtype=torch.float32, device="cuda")
        ws = torch.empty(q8.gemm_smallm_workspace(m, n, p, k), dtype=torch.uint8, device="cuda")
        runs.append(lambda wd=wd, X=X, Y=Y, ws=ws: q8.gemm_smallm(X, wd, Y, kernel=kernel and k,
                                                                    workspace=ws))
        outs.append(Y)
    _replays_equal_eager(q8, "smallm m=%d" % m, lambda: [r() for r in runs], outs)


def test_attention_and_argmax_under_capture(q8):
    import torch
    log("attention and argmax under capture")
    rng = np.random.default_rng(31)
    hd, nh, nkv, seq = 128, 8, 2, 300
    q = up(rng.standard_normal(nh * hd).astype(np.float32))
    kc = up(rng.standard_normal((512, nkv * hd)).astype(np.float32))
    vc = up(rng.standard_normal((512, nkv * hd)).astype(np.float32))
    out = torch.empty(nh * hd, dtype=torch.float32, device="cuda")
    aws = torch.empty(q8.attention_workspace(seq, hd, nh), dtype=torch.uint8, device="cuda")
    x = up(rng.standard_normal(151936).astype(np.float32))
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    mws = torch.empty(q8.argmax_workspace(x.numel()), dtype=torch.uint8, device="cuda")

    def run():
        q8.attention_decode(q, kc, vc, seq, hd, nh // nkv, out=out, workspace=aws)
        q8.argmax(x, idx, workspace=mws)

    _replays_equal_eager(q8, "attention+argmax", run, [out, idx])
    assert int(down(idx)[0]) == int(np.argmax(down(x)))
