"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Sizes here are small enough for the oracle to check every output; they span
every super-row geometry the kernels have (rows of 1, 2, 4 and 8 per lane),
several row tiles, ragged row counts and the generic tail path.
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


def _gemv(q8, w, x, n, p):
    import torch
    y = torch.full((p,), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemv(up(x), w_dev(w, n, p), y)
    return down(y)


# (n, p): nb = n/32 decides rows per super-row: nb%8==0 -> 1, ==4 -> 2,
# ==2/6 -> 4, odd -> 8; p % rs != 0 leaves tail rows for the generic path.
SHAPES = [
    (32, 1), (32, 7), (32, 9), (64, 3), (96, 50), (96, 67), (160, 9), (224, 13),
    (256, 1), (256, 64), (256, 65), (512, 300), (896, 7), (896, 130), (1024, 3072),
    (1088, 5), (1088, 131), (2080, 67), (3072, 257), (3584, 517), (4864, 131),
    (18944, 70), (256, 1031),
]


@pytest.mark.parametrize("n,p", SHAPES, ids=lambda v: str(v))
def test_gemv_matches_oracle(q8, n, p):
    log("gemv n=%d p=%d" % (n, p))
    rng = np.random.default_rng(10_000 + 7 * n + p)
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    y = _gemv(q8, w, x, n, p)
    _, y64, mag = oracle.gemv(w, x, n, p)
    parity(y, y64, mag, "gemv %dx%d" % (n, p))


def test_page_rung_one_shape(q8):
    """The page's matvec test: 50 x 96, its LCG, weight seed 7, x seed 42;
    it holds its kernel to 5e-4 absolute.  Both that bar and ours."""
    log("page 50x96")
    p, n = 50, 96
    w = synth.page_q8_bytes(p, n, 7)
    x = synth.page_x(n, 42)
    y = _gemv(q8, w, x, n, p)
    _, y64, mag = oracle.gemv(w, x, n, p)
    assert np.max(np.abs(y - y64)) < 5e-4
    parity(y, y64, mag, "page 50x96")


@pytest.mark.parametrize("n,p", [(32, 5), (96, 9), (896, 130), (3584, 512), (18944, 96),
                                 (4864, 33), (1024, 3072)], ids=lambda v: str(v))
def test_integer_case_is_bitwise(q8, n, p):
    """Scale 0.0625, integer x in [-4, 4]: every partial sum is exact in float32
    in any order, so the GPU must equal the oracle bit for bit."""
    log("integer n=%d p=%d" % (n, p))
    w, x = synth.integer_case(n, p, np.random.default_rng(77 + n + p))
    y = _gemv(q8, w, x, n, p)
    yo, _, _ = oracle.gemv(w, x, n, p)
    assert np.array_equal(y.view(np.uint32), yo.view(np.uint32))


def test_every_binary16_scale(q8):
    """Row r has scale bits r, one quant 1 against x = 1: y[r] is the decoded
    scale exactly, for all 65536 patterns (NaN where the pattern is NaN)."""
    log("f16 exhaustive")
    n, p = 32, 65536
    blk = np.zeros((p, 34), np.uint8)
    bits = np.arange(p, dtype=np.uint32)
    blk[:, 0] = bits & 0xFF
    blk[:, 1] = bits >> 8
    blk[:, 2] = 1
    x = np.zeros(n, np.float32)
    x[0] = 1.0
    import torch
    y = torch.empty(p, dtype=torch.float32, device="cuda")
    q8.gemv(up(x), up(blk), y)
    y = down(y)
    ref = np.array([oracle.f16_to_double(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert np.array_equal(y[~nan].astype(np.float64), ref[~nan])


@pytest.mark.parametrize("n", [32, 256, 896])
def test_every_quant_byte(q8, n):
    """Row r: one block of scale 1.0 holds byte r at position r % 32; x is the
    column index + 1, so y[r] = int8(r) * (column + 1) exactly."""
    log("quant bytes n=%d" % n)
    p = 256
    nb = n // 32
    w = np.zeros((p, nb, 34), np.uint8)
    r = np.arange(p)
    b = r % nb
    j = r % 32
    w[r, b, 0:2] = [0x00, 0x3C]
    w[r, b, 2 + j] = r.astype(np.uint8)
    x = (np.arange(n) + 1).astype(np.float32)
    y = _gemv(q8, w.reshape(-1), x, n, p)
    q = r.astype(np.uint8).view(np.int8).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), q * (32 * b + j + 1))


def test_zero_scales_give_zero(q8):
    log("zero scales")
    n, p = 3584, 257
    rng = np.random.default_rng(5)
    w = synth.q8_weights(n, p, rng).reshape(-1, 34)
    w[:, 0:2] = 0
    x = synth.activations(n, rng) * np.float32(100)
    assert np.all(_gemv(q8, w.reshape(-1), x, n, p) == 0.0)


def test_all_ones_quants(q8):
    log("all-ones quants")
    n, p = 896, 66
    rng = np.random.default_rng(6)
    w = synth.q8_weights(n, p, rng).reshape(-1, 34)
    w[:, 2:] = 1
    x = synth.activations(n, rng)
    y = _gemv(q8, w.reshape(-1), x, n, p)
    _, y64, mag = oracle.gemv(w, x, n, p)
    parity(y, y64, mag, "all ones")


@pytest.mark.parametrize("n,p", [(3584, 700), (896, 131), (2080, 67)], ids=lambda v: str(v))
def test_determinism_canaries_and_sign(q8, n, p):
    """Bitwise repeatable; guard bands around y untouched; y(-x) = -y(x) and
    y(4x) = 4y(x) bit for bit (negation and powers of two commute with
    rounding)."""
    import torch
    log("determinism n=%d p=%d" % (n, p))
    rng = np.random.default_rng(8 + n)
    w = w_dev(synth.q8_weights(n, p, rng), n, p)
    x = up(synth.activations(n, rng))
    guard = 1024
    buf = torch.full((p + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    y = buf[guard:guard + p]
    q8.gemv(x, w, y)
    a = down(y).copy()
    q8.gemv(x, w, y)
    b = down(y).copy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    whole = down(buf)
    assert np.all(np.isnan(whole[:guard])) and np.all(np.isnan(whole[guard + p:]))
    q8.gemv(-x, w, y)
    assert np.array_equal(down(y), -a)
    q8.gemv(x * 4, w, y)
    assert np.array_equal(down(y), a * 4)


GEMM_SHAPES = [(256, 130), (896, 70), (896, 71), (3584, 300), (160, 11), (192, 37),
               (18944, 70), (1024, 3072)]

# (m, kernel): by default m = 2..3 runs on the vector units with lanes over
# (row, block pair) where n is a multiple of 256, other m >= 2 on the matrix
# cores where n is a multiple of 128, and the rest on the vector units with a
# lane per row (four rows of X per pass).  The named kernels run where they
# apply and are refused (Q8_ERR_SHAPE) elsewhere; VROW1 is the
# row-and-block-pair kernel with one wave per workgroup instead of two.
GEMM_CASES = ([(m, None) for m in (1, 2, 3, 4, 5, 8, 13, 16)] +
              [(m, "VALU") for m in (2, 3, 4, 5, 8, 13, 16)] +
              [(m, "MFMA") for m in (2, 3)] + [(m, "VROW1") for m in (2, 3)] +
              [(m, "KS") for m in (2, 5, 8, 16)])


def _kernel_takes(kernel, m, n):
    nb = n // 32
    rs = 8 // np.gcd(nb, 8)
    if kernel == "MFMA":
        return rs <= 2 and m >= 2
    if kernel in ("VROW", "VROW1"):
        return rs == 1 and 2 <= m <= 3
    if kernel == "KS":
        return rs == 1 and m >= 2
    return m >= 2


@pytest.mark.parametrize("m,path", GEMM_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("n,p", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_smallm(q8, m, path, n, p):
    """Each row of Y against its own oracle matvec; bitwise repeatable.
    (3584, 300) and (18944, 70) have few row tiles, so a row tile's groups
    are split over workgroups and the last to arrive adds the parts;
    (896, 71) has a tail row; (192, 37) and (160, 11) have 4- and 8-row
    super-rows, which only the vector kernel takes (the others refuse them)."""
    import torch
    log("gemm m=%d n=%d p=%d kernel=%s" % (m, n, p, path or "default"))
    kernel = getattr(q8, "SMALLM_" + path) if path else None
    if path and not _kernel_takes(path, m, n):
        X = torch.zeros((m, n), dtype=torch.float32, device="cuda")
        with pytest.raises(q8.Q8Error) as ei:
            q8.gemm_smallm(X, w_dev(synth.q8_weights(n, p, np.random.default_rng(1)), n, p), kernel=kernel)
        assert ei.value.code == q8.Q8_ERR_SHAPE
        return
    rng = np.random.default_rng(300 + 11 * m + n + p)
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m).reshape(m, n)
    wd = w_dev(w, n, p)
    Xd = up(X)
    Y = torch.full((m, p), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemm_smallm(Xd, wd, Y, kernel=kernel)
    Yh = down(Y).copy()
    _, Y64, MAG = oracle.gemm(w, X, m, n, p)
    for i in range(m):
        parity(Yh[i], Y64[i], MAG[i], "gemm row %d" % i)
    for _ in range(2):       # again: split-K counters must have been left at zero
        Y.fill_(float("nan"))
        q8.gemm_smallm(Xd, wd, Y, kernel=kernel)
        assert np.array_equal(down(Y).view(np.uint32), Yh.view(np.uint32))


def _vrow_sweep_cases():
    rng = np.random.default_rng(2026)
    cases = []
    for k in range(24):
        n = 256 * int(rng.integers(1, 33))               # one row per super-row
        p = int(rng.integers(1, 5000))
        cases.append((n, p, 2 + k % 2, "1" if k % 3 == 0 else "2"))
    return cases


@pytest.mark.parametrize("n,p,m,nw", _vrow_sweep_cases(), ids=lambda v: str(v))
def test_gemm_vrow_sweep(q8, n, p, m, nw):
    """Seeded random shapes on the vector units' row-and-block-pair kernel
    (m = 2, 3; one or two waves per workgroup): every output against the
    oracle, and bitwise repeatable, so that row tiles split over workgroups
    at many different points are checked."""
    import torch
    kernel = q8.SMALLM_VROW1 if nw == "1" else q8.SMALLM_VROW
    log("gemm vrow sweep n=%d p=%d m=%d nw=%s" % (n, p, m, nw))
    rng = np.random.default_rng(n * 7919 + p * 31 + m)
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m).reshape(m, n)
    wd = w_dev(w, n, p)
    Xd = up(X)
    Y = torch.full((m, p), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemm_smallm(Xd, wd, Y, kernel=kernel)
    Yh = down(Y).copy()
    _, Y64, MAG = oracle.gemm(w, X, m, n, p)
    for i in range(m):
        parity(Yh[i], Y64[i], MAG[i], "vrow sweep row %d" % i)
    Y.fill_(float("nan"))
    q8.gemm_smallm(Xd, wd, Y, kernel=kernel)
    assert np.array_equal(down(Y).view(np.uint32), Yh.view(np.uint32))


def _mfma_sweep_cases():
    rng = np.random.default_rng(4242)
    cases = []
    for k in range(20):
        n = 128 * int(rng.integers(1, 65))               # super-rows of one or two rows
        p = int(rng.integers(1, 4000))
        cases.append((n, p, int(rng.integers(4, 17))))
    return cases


@pytest.mark.parametrize("n,p,m", _mfma_sweep_cases(), ids=lambda v: str(v))
def test_gemm_mfma_sweep(q8, n, p, m):
    """Seeded random shapes on the matrix-core kernel (m = 4..16, the split X
    in its block-major layout, the last arriver's batched reduction): every
    output against the oracle, and bitwise repeatable."""
    import torch
    log("gemm mfma sweep n=%d p=%d m=%d" % (n, p, m))
    rng = np.random.default_rng(n * 7919 + p * 31 + m)
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m).reshape(m, n)
    wd = w_dev(w, n, p)
    Xd = up(X)
    Y = torch.full((m, p), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemm_smallm(Xd, wd, Y)
    Yh = down(Y).copy()
    _, Y64, MAG = oracle.gemm(w, X, m, n, p)
    for i in range(m):
        parity(Yh[i], Y64[i], MAG[i], "mfma sweep row %d" % i)
    Y.fill_(float("nan"))
    q8.gemm_smallm(Xd, wd, Y)
    assert np.array_equal(down(Y).view(np.uint32), Yh.view(np.uint32))


@pytest.mark.parametrize("m,n,p,kernel", [
    (2, 18944, 3584, "VROW"), (3, 3584, 18944, "VROW"), (2, 3584, 152064, "KS"), (4, 18944, 3584, "KS"),
    (16, 3584, 18944, "KS"), (16, 3584, 152064, "KS"), (5, 896, 70, "MFMA"), (5, 192, 37, "VALU")])
def test_gemm_choice(q8, m, n, p, kernel):
    """The kernel q8_0_gemm_smallm runs, as q8_0_gemm_smallm_choice reports
    it: the row-and-block-pair vector kernel at m <= 3 below 65536 rows, the
    matrix cores with X held in LDS for other rows of whole groups (unless
    their per-range sums pass 64 MiB; the 7B lm_head at m = 16 needs 48.7
    MB), the
    stream-K matrix cores for super-rows of 1 or 2, else the vector units."""
    log("gemm choice m=%d n=%d p=%d" % (m, n, p))
    assert q8.gemm_smallm_choice(m, n, p) == getattr(q8, "SMALLM_" + kernel)


def _ks_sweep_cases():
    rng = np.random.default_rng(5151)
    cases = []
    for k in range(20):
        n = 256 * int(rng.integers(1, 80))               # rows of whole groups
        p = int(rng.integers(1, 6000))
        cases.append((n, p, int(rng.integers(2, 17))))
    return cases


@pytest.mark.parametrize("n,p,m", _ks_sweep_cases(), ids=lambda v: str(v))
def test_gemm_ks_sweep(q8, n, p, m):
    """Seeded random shapes on the matrix cores with X held in LDS (m =
    2..16; one or several column ranges, so with and without the sum over
    ranges; row blocks ending inside a 32-row sub-tile): every output
    against the oracle, and bitwise repeatable."""
    import torch
    log("gemm ks sweep n=%d p=%d m=%d" % (n, p, m))
    rng = np.random.default_rng(n * 7919 + p * 31 + m)
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m).reshape(m, n)
    wd = w_dev(w, n, p)
    Xd = up(X)
    Y = torch.full((m, p), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemm_smallm(Xd, wd, Y, kernel=q8.SMALLM_KS)
    Yh = down(Y).copy()
    _, Y64, MAG = oracle.gemm(w, X, m, n, p)
    for i in range(m):
        parity(Yh[i], Y64[i], MAG[i], "ks sweep row %d" % i)
    Y.fill_(float("nan"))
    q8.gemm_smallm(Xd, wd, Y, kernel=q8.SMALLM_KS)
    assert np.array_equal(down(Y).view(np.uint32), Yh.view(np.uint32))


@pytest.mark.parametrize("m,n,p", [(8, 18944, 300), (16, 18944, 3584), (16, 18944, 1030), (4, 3584, 700)])
def test_gemm_ks_y_offset(q8, m, n, p):
    """Y only 4-byte aligned (one float past a 256-byte boundary), on the
    matrix cores with X held in LDS: with the ranges' sums added by the last
    workgroup of each row block (n = 18944 at m = 8), by a second launch
    (m = 16: four outputs a thread where p is a multiple of 4, one where it
    is not), and with one range (n = 3584 at m = 4).  Every output against
    the oracle; the floats around Y untouched."""
    import torch
    log("gemm ks y offset m=%d n=%d p=%d" % (m, n, p))
    rng = np.random.default_rng(n + 7 * p + m)
    w = synth.q8_weights(n, p, rng)
    X = synth.activations(n, rng, m).reshape(m, n)
    wd = w_dev(w, n, p)
    buf = torch.full((m * p + 2,), 7.0, dtype=torch.float32, device="cuda")
    Y = buf[1:1 + m * p].view(m, p)
    q8.gemm_smallm(up(X), wd, Y, kernel=q8.SMALLM_KS)
    b = down(buf)
    assert b[0] == 7.0 and b[-1] == 7.0
    Yh = b[1:1 + m * p].reshape(m, p)
    _, Y64, MAG = oracle.gemm(w, X, m, n, p)
    for i in range(m):
        parity(Yh[i], Y64[i], MAG[i], "ks y offset row %d" % i)


@pytest.mark.parametrize("m", [2, 3, 16])
def test_gemm_identical_rows(q8, m):
    """m equal rows of X give m bitwise-equal rows of Y (m = 2, 3 on the
    vector units over rows and block pairs, 16 on the matrix cores)."""
    import torch
    log("gemm identical rows m=%d" % m)
    n, p = 3584, 129
    rng = np.random.default_rng(41)
    wd = w_dev(synth.q8_weights(n, p, rng), n, p)
    x = synth.activations(n, rng)
    Y = q8.gemm_smallm(up(np.tile(x, (m, 1))), wd)
    Yh = down(Y)
    for i in range(1, m):
        assert np.array_equal(Yh[i].view(np.uint32), Yh[0].view(np.uint32))
    del torch


@pytest.mark.parametrize("m,path", [(2, None), (3, None), (5, "VALU"), (5, None), (16, None), (16, "KS")],
                         ids=lambda v: str(v))
def test_gemm_sign_and_scale(q8, m, path):
    """Y(4X) = 4 Y(X) bit for bit on every path, and Y(-X) = -Y(X) bit for
    bit on the vector units, whose roundings are all to nearest even (no
    value here is near overflow or the subnormal range).  The matrix cores
    (m = 5, 16 by default) do not round their internal sums symmetrically
    under negation, so there the sign is checked within the bar.  A row tile
    split over workgroups (p = 300 at n = 3584) is included."""
    import torch
    kernel = getattr(q8, "SMALLM_" + path) if path else None
    log("gemm sign and scale m=%d kernel=%s" % (m, path or "default"))
    n, p = 3584, 300
    rng = np.random.default_rng(77 + m)
    w = synth.q8_weights(n, p, rng)
    wd = w_dev(w, n, p)
    X = synth.activations(n, rng, m).reshape(m, n)
    a = down(q8.gemm_smallm(up(X), wd, kernel=kernel)).copy()
    assert np.array_equal(down(q8.gemm_smallm(up(X * 4), wd, kernel=kernel)), a * 4)
    neg = down(q8.gemm_smallm(up(-X), wd, kernel=kernel))
    if m <= 3 or path == "VALU":
        assert np.array_equal(neg, -a)
    else:
        _, _, MAG = oracle.gemm(w, X, m, n, p)
        for i in range(m):
            assert np.all(np.abs(neg[i].astype(np.float64) + a[i]) <= 2 * (1e-5 * MAG[i] + 1e-6))
    del torch


def _chain_case(seed):
    """Twelve ops of mixed shapes; op 7 reads op 6's output (a dependency)."""
    shapes = [(1024, 2048), (1024, 1024), (896, 128), (896, 130), (2048, 1024), (3584, 512),
              (4864, 896), (896, 4864), (160, 9), (256, 1031), (18944, 64), (3584, 1000)]
    rng = np.random.default_rng(seed)
    ws = [synth.q8_weights(n, p, rng) for n, p in shapes]
    xs = [synth.activations(n, rng) for n, p in shapes]
    return shapes, ws, xs


@pytest.mark.parametrize("fuse", [True, False])
def test_chain_modes_equal_standalone(q8, fuse):
    import torch
    log("chain fuse=%s" % fuse)
    shapes, ws, xs = _chain_case(2024)
    wd = [w_dev(w, n, p) for w, (n, p) in zip(ws, shapes)]
    xd = [up(x) for x in xs]
    ys = [torch.full((p,), float("nan"), dtype=torch.float32, device="cuda") for n, p in shapes]
    xd[7] = ys[6]                      # 4864->896 feeds 896->4864
    chain = q8.Chain(list(zip(xd, wd, ys)), fuse=fuse)
    assert chain.launches == (2 if fuse else len(shapes))
    # standalone reference, in order (op 7 reads op 6's result)
    ref = [torch.empty(p, dtype=torch.float32, device="cuda") for n, p in shapes]
    for i, (n, p) in enumerate(shapes):
        q8.gemv(ref[6] if i == 7 else xd[i], wd[i], ref[i])
    refh = [down(r).copy() for r in ref]
    for mode in (q8.MODE_GRAPH, q8.MODE_EAGER, q8.MODE_SYNC_EACH, q8.MODE_GRAPH):
        for y in ys:
            y.fill_(float("nan"))
        chain.run(mode)
        q8.stream_wait(timeout_ms=60_000)
        for i in range(len(shapes)):
            assert np.array_equal(down(ys[i]).view(np.uint32), refh[i].view(np.uint32)), (mode, i)
    # and against the oracle
    x7 = refh[6]
    for i, (n, p) in enumerate(shapes):
        x = x7 if i == 7 else xs[i]
        _, y64, mag = oracle.gemv(ws[i], x, n, p)
        parity(refh[i], y64, mag, "chain op %d" % i)
    chain.close()


# Shapes for chains planned for latency (Q8_CHAIN_SPLIT_K): row-poor ops
# with many groups per row, super-rows of 2 and 4 rows, a tail row, a 7B
# down projection, more row tiles than the GPU has CUs, and ops of one width
# that share a launch (the 3584-wide q, k, v).
SPLIT_SHAPES = [(2048, 1024), (3072, 1024), (896, 130), (896, 131), (4864, 131), (1088, 5),
                (3584, 512), (96, 67), (18944, 3584), (1024, 16448), (3584, 3584), (3584, 513)]


@pytest.mark.parametrize("per_op", [False, True], ids=["fused", "per_op"])
def test_split_k_chain(q8, per_op):
    """Q8_CHAIN_SPLIT_K on independent ops and on a dependent pair: every
    output equals the standalone q8_0_gemv on the same inputs bit for bit
    (every launch shape sums in the same order), the same bits on every
    replay and in every mode, and within the bar against the oracle."""
    import torch
    log("split-K chain per_op=%s" % per_op)
    rng = np.random.default_rng(77)
    ws = [synth.q8_weights(n, p, rng) for n, p in SPLIT_SHAPES]
    xs = [synth.activations(n, rng) for n, p in SPLIT_SHAPES]
    wd = [w_dev(w, n, p) for w, (n, p) in zip(ws, SPLIT_SHAPES)]
    xd = [up(x) for x in xs]
    ys = [torch.full((p,), float("nan"), dtype=torch.float32, device="cuda") for n, p in SPLIT_SHAPES]
    # a dependent op: 3072 -> 1024 feeds 1024 -> 3072
    w_dep = synth.q8_weights(1024, 3072, rng)
    wd_dep = w_dev(w_dep, 1024, 3072)
    y_dep = torch.full((3072,), float("nan"), dtype=torch.float32, device="cuda")
    ops = list(zip(xd, wd, ys)) + [(ys[1], wd_dep, y_dep)]
    chain = q8.Chain(ops, fuse=not per_op, split_k=True)
    ref = [down(q8.gemv(x, w)).copy() for x, w in zip(xd, wd)]
    ref.append(down(q8.gemv(up(ref[1]), wd_dep)).copy())
    for mode in (q8.MODE_GRAPH, q8.MODE_EAGER, q8.MODE_GRAPH, q8.MODE_SYNC_EACH):
        for y in ys + [y_dep]:
            y.fill_(float("nan"))
        chain.run(mode)
        q8.stream_wait(timeout_ms=60_000)
        for i, y in enumerate(ys + [y_dep]):
            assert np.array_equal(down(y).view(np.uint32), ref[i].view(np.uint32)), (mode, i)
    for i, (n, p) in enumerate(SPLIT_SHAPES):
        _, y64, mag = oracle.gemv(ws[i], xs[i], n, p)
        parity(ref[i], y64, mag, "split-K op %d (%d x %d)" % (i, n, p))
    _, y64, mag = oracle.gemv(w_dep, ref[1], 1024, 3072)
    parity(ref[-1], y64, mag, "split-K dependent op")
    chain.close()


# n multiple of 256: 4, 12, 14, 74 and 37 groups per row (columns that do and
# do not fill 2 and 4 lanes), ragged row counts and rows that leave a last
# tile of one row; (1024, 5000) and (3584, 9000) are planned with tiles
# shorter than a wave's rows (10 of 16, 18 of 32) to even out the CUs
SHAPED = [(1024, 3072), (3072, 1024), (3584, 515), (18944, 70), (9472, 17), (256, 1), (1024, 65),
          (1024, 5000), (3584, 9000)]


@pytest.mark.parametrize("n,p", SHAPED, ids=lambda v: str(v))
def test_every_launch_shape_same_bits(q8, n, p):
    """q8_0_gemv_shaped on every launch shape (1, 2 or 4 lanes per row x 1,
    2 or 4 waves per workgroup x 1 or 2 weight stages, where the LDS fits)
    gives q8_0_gemv's bits exactly, and those are within the bar against the
    oracle."""
    import torch
    log("launch shapes n=%d p=%d plan=%s" % (n, p, q8.gemv_plan(n, p)))
    rng = np.random.default_rng(31 * n + p)
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    wd, xd = w_dev(w, n, p), up(x)
    ref = down(q8.gemv(xd, wd)).copy()
    _, y64, mag = oracle.gemv(w, x, n, p)
    parity(ref, y64, mag, "gemv %dx%d" % (n, p))
    y = torch.empty(p, dtype=torch.float32, device="cuda")
    for c in (1, 2, 4):
        for waves in (1, 2, 4):
            for stages in (1, 2):
                if (c, waves, stages) in ((4, 4, 2),):     # needs more than 160 KiB of LDS
                    continue
                y.fill_(float("nan"))
                q8.gemv(xd, wd, y, shape=(c, waves, stages))
                assert np.array_equal(down(y).view(np.uint32), ref.view(np.uint32)), (c, waves, stages)


def test_shaped_refuses_other_widths(q8):
    """An explicit launch shape needs n % 256 == 0 and lanes/waves in {1,2,4}."""
    import torch
    w = w_dev(synth.q8_weights(896, 8, np.random.default_rng(3)), 896, 8)
    x = torch.zeros(896, dtype=torch.float32, device="cuda")
    with pytest.raises(q8.Q8Error) as ei:
        q8.gemv(x, w, shape=(4, 4, 1))
    assert ei.value.code == q8.Q8_ERR_SHAPE
    w = w_dev(synth.q8_weights(1024, 8, np.random.default_rng(3)), 1024, 8)
    x = torch.zeros(1024, dtype=torch.float32, device="cuda")
    for bad in ((3, 1, 1), (4, 4, 2), (1, 1, 3)):    # (4, 4, 2): 172 KiB of LDS
        with pytest.raises(q8.Q8Error) as ei:
            q8.gemv(x, w, shape=bad)
        assert ei.value.code == q8.Q8_ERR_INVALID_ARG


def test_stream_wait_timeout_and_ok(q8):
    """A bounded wait returns OK on an idle stream; with about 10 ms of
    matvecs queued (40 launches over 72 MB of weights) a wait of 0 ms returns
    Q8_ERR_TIMEOUT without cancelling anything, and an unbounded wait then
    returns OK once they have run (the last output checked)."""
    import torch
    torch.cuda.synchronize()
    assert q8.stream_wait(timeout_ms=1000) == 0
    n, p = 18944, 3584
    rng = np.random.default_rng(12)
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    wd, xd = w_dev(w, n, p), up(x)
    y = torch.empty(p, dtype=torch.float32, device="cuda")
    q8.gemv(xd, wd, y)
    torch.cuda.synchronize()
    ref = down(y).copy()
    for _ in range(40):
        q8.gemv(xd, wd, y)
    with pytest.raises(q8.Q8Error) as ei:
        q8.stream_wait(timeout_ms=0)
    assert ei.value.code == q8.Q8_ERR_TIMEOUT
    assert q8.stream_wait(timeout_ms=-1) == 0
    assert np.array_equal(down(y).view(np.uint32), ref.view(np.uint32))


def test_widest_rows(q8):
    """n at its maximum (2**20 columns, 32768 blocks, 1.1 MB per row): the
    matvec (on every launch shape: the same bits), the small batch on the
    matrix cores (m = 16) and on the vector units (m = 2 over rows and block
    pairs, m = 3 a lane per row), every output against the oracle."""
    import torch
    n, p = 1 << 20, 67
    log("widest rows n=%d p=%d" % (n, p))
    rng = np.random.default_rng(1 << 20)
    w = synth.q8_weights(n, p, rng)
    wd = w_dev(w, n, p)
    x = synth.activations(n, rng)
    y = torch.full((p,), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemv(up(x), wd, y)
    _, y64, mag = oracle.gemv(w, x, n, p)
    ref = down(y).copy()
    parity(ref, y64, mag, "gemv widest")
    for sh in ((1, 1, 2), (4, 4, 1), (2, 2, 1), (4, 2, 2)):
        q8.gemv(up(x), wd, y, shape=sh)
        assert np.array_equal(down(y).view(np.uint32), ref.view(np.uint32)), sh
    for m, kernel in ((16, None), (2, None), (3, q8.SMALLM_VALU)):
        X = synth.activations(n, rng, m)
        Y = torch.full((m, p), float("nan"), dtype=torch.float32, device="cuda")
        q8.gemm_smallm(up(X), wd, Y, kernel=kernel)
        _, Y64, MAG = oracle.gemm(w, X, m, n, p)
        Yh = down(Y)
        for i in range(m):
            parity(Yh[i], Y64[i], MAG[i], "gemm widest m=%d row %d" % (m, i))


def test_most_rows(q8):
    """p = 2**22 + 3 one-block rows (143 MB of W, 16385 row tiles and a tail
    of three rows): sampled rows, the tile boundaries and the tail, against
    the oracle."""
    import torch
    n, p = 32, (1 << 22) + 3
    log("most rows n=%d p=%d" % (n, p))
    rng = np.random.default_rng(22)
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    y = torch.full((p,), float("nan"), dtype=torch.float32, device="cuda")
    q8.gemv(up(x), w_dev(w, n, p), y)
    yh = down(y)
    rows = np.unique(np.concatenate([
        np.arange(0, 130), np.arange(p - 130, p),
        rng.integers(0, p, 2000), np.arange(511, p, 1 << 16), np.arange(512, p, 1 << 16)]))
    _, y64, mag = oracle.gemv_rows(w, x, n, rows)
    parity(yh[rows], y64, mag, "gemv most rows")
    assert not np.isnan(yh).any()
