"""GPU parity of the integer path (x quantized to Q8_0, integer block dots)
against the CPU oracle, through the C ABI.

* q8_0_quantize: byte for byte equal to the oracle's quantization (the codes
  and scales are decided by float32 operations on both sides).
* q8_0_gemv_q8q8 and chains with Q8_CHAIN_XQ: the element bar of the float
  matvec, |y - y_ref| <= 1e-5 * mag + 1e-6, against the oracle's integer
  definition (mag = sum_b |d_w d_x| sum_j |q_w q_x|); and bit for bit equal
  to it where every block share and every partial sum is exact in float32
  (unit scales, small integers), which also checks every code the kernel
  made on the fly.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import down, log, parity, up, w_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q8():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import q8_block_quantized_gemv_amd as q8mod
    return q8mod


def _x_cases():
    rng = np.random.default_rng(900)
    cases = {}
    nb = 4096
    scale = np.exp(rng.uniform(-12, 14, nb))          # scales from subnormal binary16 to large
    cases["wide_scales"] = (rng.standard_normal((nb, 32)) * scale[:, None]).astype(np.float32).reshape(-1)
    x = rng.standard_normal(64 * 32).astype(np.float32)
    x[:32] = 0.0                                          # an all-zero block
    x[32:64] = np.arange(32) - 15.5                       # halves: ties away from zero
    x[64:96] = 0.0
    x[64] = -3.0e-38                                      # a lone tiny value
    x[96:128] = (np.arange(32) * 4 - 60).astype(np.float32) * 2.0 ** -9
    cases["edges"] = x
    cases["n32"] = rng.standard_normal(32).astype(np.float32)
    cases["n_2e20"] = rng.standard_normal(1 << 20).astype(np.float32)
    # values near x/d = k + 1/2 for the block scale d = amax/127
    t = np.zeros((256, 32), np.float32)
    t[:, 0] = 127.0 * 0.37
    t[:, 1:] = ((rng.integers(-126, 126, size=(256, 31)) + 0.5) * 0.37).astype(np.float32)
    cases["near_ties"] = t.reshape(-1)
    return cases


X_CASES = _x_cases()


@pytest.mark.parametrize("name", sorted(X_CASES))
def test_quantize_bytes(q8, name):
    x = X_CASES[name]
    log("quantize %s n=%d" % (name, x.size))
    got = down(q8.quantize(up(x)))
    ref = oracle.quantize_x(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "%s: %d bytes differ, first at %d (block %d): gpu %d oracle %d" % (
        name, bad.size, bad[0], bad[0] // 34, got[bad[0]], ref[bad[0]])


SHAPES = [(32, 7), (96, 67), (160, 9), (256, 65), (512, 300), (896, 130), (1024, 3072),
          (1088, 131), (2080, 67), (3584, 517), (4864, 131), (18944, 70)]


@pytest.mark.parametrize("n,p", SHAPES, ids=str)
def test_gemv_q8q8(q8, n, p):
    import torch
    log("gemv_q8q8 n=%d p=%d" % (n, p))
    rng = np.random.default_rng(20_000 + 7 * n + p)
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    y = torch.full((p,), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemv_q8q8(up(x), w_dev(w, n, p), y)
    _, y64, mag = oracle.gemv_q8q8(w, x, n, p)
    parity(down(y), y64, mag, "gemv_q8q8 %dx%d" % (n, p))


@pytest.mark.parametrize("n,p", [(256, 64), (896, 131), (1024, 300), (4864, 67)], ids=str)
def test_gemv_q8q8_exact(q8, n, p):
    """Unit weight scales, |q_w| <= 15, integer x whose blocks each reach 127
    (so the codes are x itself): every block share and partial sum is an
    integer below 2^24, the result is exact and must match bit for bit."""
    import torch
    log("gemv_q8q8 exact n=%d p=%d" % (n, p))
    rng = np.random.default_rng(21_000 + n + p)
    nb = n // 32
    xi = rng.integers(-15, 16, size=n)
    xi[::32] = 127
    qw = rng.integers(-15, 16, size=(p * nb, 32)).astype(np.int8)
    w = synth.pack_blocks(np.full(p * nb, 1.0, np.float16), qw)
    x = xi.astype(np.float32)
    y = torch.full((p,), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemv_q8q8(up(x), w_dev(w, n, p), y)
    ref, y64, _ = oracle.gemv_q8q8(w, x, n, p)
    assert np.all(np.abs(y64) < 2 ** 24)
    assert np.array_equal(down(y), ref)


@pytest.mark.parametrize("fuse,split", [(True, False), (False, False), (True, True)],
                         ids=["fused", "per_op", "split_k"])
def test_xq_chain(q8, fuse, split):
    import torch
    log("xq chain fuse=%s split=%s" % (fuse, split))
    shapes = [(1024, 2048), (1024, 1024), (2048, 1024), (3072, 1024), (896, 131), (1024, 3000)]
    rng = np.random.default_rng(22_000)
    ws = [synth.q8_weights(n, p, rng) for n, p in shapes]
    xs = [synth.activations(n, rng) for n, p in shapes]
    ys = [torch.full((p,), float("nan"), dtype=torch.float32, device="cuda") for n, p in shapes]
    ch = q8.Chain([(up(x), w_dev(w, n, p), y) for (n, p), w, x, y in zip(shapes, ws, xs, ys)],
                  fuse=fuse, split_k=split, xq=True)
    first = None
    for mode in (q8.MODE_GRAPH, q8.MODE_EAGER, q8.MODE_GRAPH):
        for y in ys:
            y.fill_(float("nan"))
        ch.run(mode)
        q8.stream_wait(timeout_ms=60_000)
        got = [down(y).copy() for y in ys]
        if first is None:
            first = got
        for a, b in zip(first, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for i, (n, p) in enumerate(shapes):
        _, y64, mag = oracle.gemv_q8q8(ws[i], xs[i], n, p)
        parity(first[i], y64, mag, "xq chain op %d" % i)
    ch.close()
