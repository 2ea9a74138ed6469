"""The full-size workloads, in the launch configuration the bench times (one
fused launch per token, replayed from a hipGraph), every output against the
oracle (run on host threads), and the same chains launched op by op and
planned for latency giving the same bits; plus the small-batch products at
the 7B shapes on sampled rows."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import down, log, parity, up, w_dev

pytestmark = pytest.mark.gpu


def sample_rows(p, k, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, p // 2, p - 2, p - 1]
    rows = set(r for r in fixed if 0 <= r < p)
    rows.update(rng.integers(0, p, size=k).tolist())
    return np.array(sorted(rows))


@pytest.fixture(scope="module")
def q8():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import q8_block_quantized_gemv_amd as q8mod
    return q8mod


@pytest.mark.parametrize("workload", ["single_1024x3072", "qwen3_0.6b_chain",
                                      "qwen2.5_0.5b_chain", "7b_chain"])
def test_workload_chain(q8, workload):
    import torch
    log("workload %s: generating" % workload)
    data = synth.generate(workload)
    ops = []
    for op, w, x in data:
        ops.append((up(x), w_dev(w, op.n, op.p),
                    torch.full((op.p,), float("nan"), dtype=torch.float32, device="cuda")))
    log("workload %s: chain of %d ops" % (workload, len(ops)))
    chain = q8.Chain(ops, fuse=True)
    assert chain.launches == 1
    chain.run(q8.MODE_GRAPH)
    q8.stream_wait(timeout_ms=120_000)
    got = [down(y).copy() for _, _, y in ops]
    chain.close()
    worst = 0.0
    for i, ((op, w, x), yh) in enumerate(zip(data, got)):
        _, y64, mag = oracle.gemv_threaded(w, x, op.n, op.p)
        worst = max(worst, parity(yh, y64, mag, "%s op %d (%s)" % (workload, i, op.name)))
    log("workload %s: every output within the bar, worst error/bound %.3g" % (workload, worst))
    # one launch per op, planned for latency: the same bits
    for flags in ({"fuse": False}, {"fuse": False, "split_k": True}):
        for _, _, y in ops:
            y.fill_(float("nan"))
        ch = q8.Chain(ops, **flags)
        assert ch.launches == len(ops)
        ch.run(q8.MODE_GRAPH)
        q8.stream_wait(timeout_ms=120_000)
        for i, (_, _, y) in enumerate(ops):
            assert np.array_equal(down(y).view(np.uint32), got[i].view(np.uint32)), (flags, i)
        ch.close()
    del ops
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", synth.SMALLM_SHAPES, ids=lambda s: s.name)
def test_smallm_7b_shapes(q8, shape):
    import torch
    w, _ = synth.generate_smallm(shape, 2)
    wd = w_dev(w, shape.n, shape.p)
    rows = sample_rows(shape.p, 40, 7)
    for m in synth.SMALLM_M:
        log("smallm %s m=%d" % (shape.name, m))
        _, X = synth.generate_smallm(shape, m)
        Y = torch.full((m, shape.p), float("nan"), dtype=torch.float32, device="cuda")
        q8.gemm_smallm(up(X), wd, Y)
        Yh = down(Y)
        assert np.all(np.isfinite(Yh))
        for i in range(m):
            _, y64, mag = oracle.gemv_rows(w, X[i], shape.n, rows)
            parity(Yh[i][rows], y64, mag, "smallm %s m=%d row %d" % (shape.name, m, i))
    del wd
    torch.cuda.empty_cache()
