"""GPU parity of the decode-step kernels and of the whole recorded step
against the CPU oracle (oracle/decode_step.py), through the C ABI.

Bars.  u = 2^-24 is float32's unit roundoff.  Each bar below is the
first-order bound of the kernel's own float32 arithmetic (the oracle is
float64 on the same float32 inputs), written next to the test that uses it:

* add_inplace: one rounding of an exact sum -- bit-exact against the
  oracle's sum rounded to float32.
* argmax: exact (same index, NaN and tie rules).
* append_kv: a copy -- bit-exact.
* rms_norm over dim with at most k = ceil(dim / 64) + 3 fused multiply-adds
  per lane, a 6-level butterfly, then /dim, +eps, sqrt, 1/., two products:
  |err| <= (0.5 (k + 8) + 5) u |ref|.
* rope in double precision, rounded once: |err| <= 2 u |ref| + 1e-10 (|a| + |b|)
  (one float ulp when double rounding error flips a tie, and the angle's
  double-precision error across two libm implementations).
* silu_hadamard: exp to 1 ulp, then +, /, *: |err| <= 8 u |ref|, plus
  2^-120 |up| where g / (1 + e^-g) falls below float32's normal range
  (e^-g overflows for g < -88.7 and the factor becomes 0).
* attention: a score carries at most 13 u sum_i |q_i k_i| / sqrt(hd) of
  error (4 products per lane, up to a 6-level butterfly, the scale and its
  square root and division); the weights then carry twice that plus the
  sums' (64 + chunks) u (rows per thread, row groups, the chunk merge,
  exp); the output's error is bounded by that times sum_t p_t |v_tj|.
* the whole step: each stage above sits far below 1e-5 relative; through
  the stages of a layer (which renormalise their inputs) the logits keep
  |err| <= 1e-4 (mag_i + rms(logits)), mag_i = sum_j |w_ij x_j| of the
  lm_head row.  Tokens must agree wherever the oracle's top two logits are
  further apart than twice that bar.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import decode_step as ods
from tests.gpu_util import down, log, up

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def q8():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import q8_block_quantized_gemv_amd as q8mod
    return q8mod


def _check(gpu, ref, bound, label):
    gpu = np.asarray(gpu, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    bound = np.asarray(bound, np.float64)
    bound = bound.reshape(-1) if bound.size == ref.size else np.broadcast_to(bound, ref.shape)
    assert gpu.shape == ref.shape, label
    assert np.all(np.isfinite(gpu)), "%s: non-finite output" % label
    err = np.abs(gpu - ref)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, "%s: %d over the bar, first %d: gpu %r ref %r bound %r" % (
        label, bad.size, bad[0], gpu[bad[0]], ref[bad[0]], bound[bad[0]])
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0


# ---------------------------------------------------------------- rms_norm
RMS_SHAPES = [(1, 1), (33, 3), (64, 14), (128, 8), (128, 16), (896, 1), (1024, 1), (3584, 1),
              (65536, 1), (256, 300)]


@pytest.mark.parametrize("dim,rows", RMS_SHAPES, ids=str)
@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
def test_rms_norm(q8, dim, rows, inplace):
    log("rms_norm dim=%d rows=%d inplace=%d" % (dim, rows, inplace))
    rng = np.random.default_rng(100 + dim + rows)
    x = (rng.standard_normal(dim * rows) * 3.0).astype(np.float32)
    if rows > 1:
        x[:dim] = 0.0     # an all-zero row: the output is zero
    w = rng.uniform(0.5, 1.5, dim).astype(np.float32)
    xd, wd = up(x), up(w)
    out = q8.rms_norm(xd, wd, xd if inplace else None, eps=1e-6)
    ref = ods.rms_norm_rows(x, w, dim, 1e-6).reshape(-1)
    k = math.ceil(dim / 64) + 3     # fused multiply-adds per lane (float4 path: 4 per load)
    _check(down(out), ref, (0.5 * (k + 8) + 5) * U * np.abs(ref), "rms_norm %dx%d" % (dim, rows))


# ---------------------------------------------------------------- rope
@pytest.mark.parametrize("head_dim,heads", [(64, 14), (128, 16), (128, 8), (192, 3), (256, 2), (2, 5)],
                         ids=str)
@pytest.mark.parametrize("pos", [0, 1, 500, 4095, 32767, 65535])
def test_rope(q8, head_dim, heads, pos):
    log("rope hd=%d heads=%d pos=%d" % (head_dim, heads, pos))
    rng = np.random.default_rng(200 + head_dim + pos)
    x = rng.standard_normal(head_dim * heads).astype(np.float32)
    theta = 1e6 if head_dim >= 128 else 1e4
    xd = up(x)
    q8.rope(xd, head_dim, pos, theta)
    ref = ods.rope_rows(x, head_dim, pos, theta).reshape(-1)
    half = head_dim // 2
    xa = np.abs(x.reshape(heads, 2, half))
    ab = np.concatenate([xa[:, 0] + xa[:, 1], xa[:, 0] + xa[:, 1]], axis=1).reshape(-1)
    _check(down(xd), ref, 2 * U * np.abs(ref) + 1e-10 * ab, "rope")


# ---------------------------------------------------------------- append_kv
def test_append_kv(q8):
    import torch
    log("append_kv")
    rng = np.random.default_rng(300)
    width, rows = 1024, 40
    kc = rng.standard_normal((rows, width)).astype(np.float32)
    vc = rng.standard_normal((rows, width)).astype(np.float32)
    kcd, vcd = up(kc), up(vc)
    for pos in (0, 17, rows - 1):
        k = rng.standard_normal(width).astype(np.float32)
        v = rng.standard_normal(width).astype(np.float32)
        q8.append_kv(up(k), up(v), kcd, vcd, pos)
        kc, vc = ods.append_kv(k, v, kc, vc, width, pos)
    torch.cuda.synchronize()
    assert np.array_equal(down(kcd), kc) and np.array_equal(down(vcd), vc)


# ---------------------------------------------------------------- attention
# (seq, n_heads, kv_group, head_dim, extra kv_width, q scale)
ATTN_CASES = [
    (1, 16, 2, 128, 0, 1.0), (5, 8, 4, 64, 0, 1.0), (127, 4, 1, 64, 0, 1.0),
    (128, 16, 2, 128, 0, 1.0), (129, 14, 7, 64, 0, 1.0), (300, 4, 2, 192, 0, 1.0),
    (1000, 16, 2, 128, 32, 1.0), (1000, 16, 2, 128, 0, 8.0), (4096, 28, 7, 128, 0, 1.0),
    (5000, 2, 1, 256, 0, 1.0), (65536, 2, 2, 256, 0, 1.0),
]


def _attention_case(q8, seq, nh, group, hd, extra, qscale, reps=1):
    rng = np.random.default_rng(400 + seq + nh + hd)
    nkv = nh // group
    kvw = nkv * hd + extra
    q = (rng.standard_normal(nh * hd) * qscale).astype(np.float32)
    kc = rng.standard_normal((seq, kvw), dtype=np.float32)
    vc = rng.standard_normal((seq, kvw), dtype=np.float32)
    if qscale > 1:   # a sharp softmax whose peak sits in the last chunk
        kc[seq - 3] = np.tile(q[:hd] / qscale, kvw // hd + 1)[:kvw]
    qd, kd, vd = up(q), up(kc), up(vc)
    outs = [down(q8.attention_decode(qd, kd, vd, seq, hd, group)) for _ in range(reps)]
    ref, p = ods.attention_decode(q, kc, vc, seq, kvw, hd, nh, group)
    kc64 = kc.astype(np.float64)
    vc64 = vc.astype(np.float64)
    q64 = q.astype(np.float64).reshape(nh, hd)
    chunks = math.ceil(seq / 128)
    bound = np.empty((nh, hd))
    for h in range(nh):
        off = (h // group) * hd
        qk = np.abs(kc64[:, off:off + hd]) @ np.abs(q64[h]) / math.sqrt(hd)
        eps_w = 2 * 13 * U * float(qk.max()) + (64 + chunks) * U
        bound[h] = eps_w * (p[h] @ np.abs(vc64[:, off:off + hd])) + 1e-30
    return outs, ref, bound


@pytest.mark.parametrize("case", ATTN_CASES, ids=str)
def test_attention(q8, case):
    seq, nh, group, hd, extra, qscale = case
    log("attention seq=%d heads=%d group=%d hd=%d extra=%d qscale=%g" % case)
    outs, ref, bound = _attention_case(q8, *case, reps=2)
    worst = _check(outs[0], ref, bound, "attention %s" % (case,))
    assert np.array_equal(outs[0], outs[1]), "attention is not reproducible"
    log("attention worst err/bound %.3g" % worst)


# ---------------------------------------------------------------- add, silu
@pytest.mark.parametrize("n", [1, 255, 256, 1024, 18944, 1 << 20])
def test_add_inplace(q8, n):
    log("add n=%d" % n)
    rng = np.random.default_rng(500 + n)
    x = rng.standard_normal(n).astype(np.float32) * 100
    y = rng.standard_normal(n).astype(np.float32)
    xd = up(x)
    q8.add_inplace(xd, up(y))
    assert np.array_equal(down(xd), ods.add_inplace(x, y).astype(np.float32))


@pytest.mark.parametrize("n", [1, 255, 3072, 18944, 1 << 20])
def test_silu_hadamard(q8, n):
    log("silu n=%d" % n)
    rng = np.random.default_rng(600 + n)
    g = (rng.standard_normal(n) * 6).astype(np.float32)
    if n > 4:
        g[:4] = [-100.0, 100.0, 0.0, -0.0]
    u = rng.standard_normal(n).astype(np.float32)
    out = down(q8.silu_hadamard(up(g), up(u)))
    ref = ods.silu_hadamard(g, u)
    _check(out, ref, 8 * U * np.abs(ref) + 2.0 ** -120 * np.abs(u), "silu n=%d" % n)


# ---------------------------------------------------------------- argmax
def _argmax_inputs():
    rng = np.random.default_rng(700)
    cases = {}
    cases["vocab_151936"] = rng.standard_normal(151936).astype(np.float32)
    cases["n1"] = np.array([3.5], np.float32)
    cases["all_equal"] = np.full(5000, 2.0, np.float32)
    x = rng.standard_normal(4097).astype(np.float32)
    x[4096] = 50.0
    cases["max_last_ragged"] = x
    x = rng.standard_normal(1 << 20 | 3).astype(np.float32)
    x[[5, 300000, (1 << 20) + 1]] = 9.0    # ties in different workgroups
    cases["ties_across_groups"] = x
    x = rng.standard_normal(152064).astype(np.float32)
    x[::7] = np.nan
    cases["nan_sprinkled"] = x
    cases["all_nan"] = np.full(1000, np.nan, np.float32)
    cases["all_neg_inf"] = np.full(777, -np.inf, np.float32)
    x = rng.standard_normal(3000).astype(np.float32)
    x[0] = np.nan
    x[2999] = np.inf
    cases["inf_wins"] = x
    return cases


ARGMAX_CASES = _argmax_inputs()


@pytest.mark.parametrize("name", sorted(ARGMAX_CASES))
def test_argmax(q8, name):
    import torch
    x = ARGMAX_CASES[name]
    log("argmax %s n=%d" % (name, x.size))
    xd = up(x)
    out = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    for _ in range(2):   # the second call checks the arrival counter was reset
        q8.argmax(xd, out)
        got = int(down(out)[0]) & 0xFFFFFFFF
        assert got == ods.argmax_row(x), (name, got, ods.argmax_row(x))


# ---------------------------------------------------------------- the whole step
def _step(q8, name, max_seq):
    import torch
    cfg, w = synth.step_model(name)
    cfg = dict(cfg, max_seq=max_seq)

    def dev_w(a, p=None, n=None):
        if a.dtype == np.uint8:
            return up(a.reshape(p, n // 32 * 34))
        return up(a)

    shapes = dict((nm, (p, n)) for nm, n, p in synth.step_proj_shapes(cfg))
    layers = []
    for L in w["layers"]:
        d = {}
        for k, a in L.items():
            d[k] = dev_w(a, *shapes[k]) if k in shapes else up(a)
        layers.append(d)
    wd = {"embed": up(w["embed"]), "out_norm": up(w["out_norm"]),
          "lm_head": dev_w(w["lm_head"], cfg["vocab"], cfg["hidden"]), "layers": layers}
    torch.cuda.synchronize()
    return cfg, w, q8.Step(cfg, wd)


def _oracle_caches(cfg):
    kvw = cfg["n_kv_heads"] * cfg["head_dim"]
    return ([np.zeros((cfg["max_seq"], kvw), np.float32) for _ in range(cfg["n_layers"])],
            [np.zeros((cfg["max_seq"], kvw), np.float32) for _ in range(cfg["n_layers"])])


def _run_tokens(q8, st, mode, pos, token, count):
    st.reset(pos, token)
    toks, logits, xs = [], [], []
    for _ in range(count):
        st.run(mode)
        toks.append(int(down(st.buffer("token"))[0]) & 0xFFFFFFFF)
        logits.append(down(st.buffer("logits")).copy())
        xs.append(down(st.buffer("x")).copy())
    return toks, logits, xs


def test_step_launch_count(q8):
    log("step launches step_tiny")
    cfg, _, st = _step(q8, "step_tiny", 64)
    # per layer: q|k|v (fused; from the second layer on it also adds the
    # residual and norms), attention, o, gate|up (fused, adds and norms),
    # down; then embed+norm, the lm_head (adds, norms), argmax
    assert st.launches == cfg["n_layers"] * 5 + 1 + 2
    st.close()


def test_step_graph_equals_eager(q8):
    log("step graph vs eager step_tiny")
    _, _, st = _step(q8, "step_tiny", 300)
    a = _run_tokens(q8, st, q8.MODE_EAGER, 0, 7, 6)
    kc_a = down(st.buffer("k_cache")).copy()
    b = _run_tokens(q8, st, q8.MODE_GRAPH, 0, 7, 6)
    kc_b = down(st.buffer("k_cache")).copy()
    assert a[0] == b[0]
    for la, lb in zip(a[1], b[1]):
        assert np.array_equal(la, lb)
    for xa, xb in zip(a[2], b[2]):
        assert np.array_equal(xa, xb)
    assert np.array_equal(kc_a, kc_b)
    assert int(down(st.buffer("pos"))[0]) == 6
    st.close()


STEP_BAR = 1e-4


def _compare_step(cfg, w, kc, vc, tok_in, pos, logits, x, tok_gpu, label, matvec=None):
    tok_ref, y, y64, mag, x_ref = ods.decode_step(cfg, w, kc, vc, tok_in, pos, matvec)
    rms = float(np.sqrt(np.mean(y64 * y64)))
    bar = STEP_BAR * (mag + rms)
    _check(logits, y64, bar, "%s logits pos %d" % (label, pos))
    _check(x, x_ref, STEP_BAR * (np.abs(x_ref) + float(np.sqrt(np.mean(x_ref.astype(np.float64) ** 2)))),
           "%s residual pos %d" % (label, pos))
    order = np.argsort(y64)
    margin = y64[order[-1]] - y64[order[-2]]
    if margin > 2 * bar[order[-1]] + 2 * bar[order[-2]]:
        assert tok_gpu == tok_ref, (label, pos, tok_gpu, tok_ref)
    else:
        assert y64[tok_gpu] >= y64[order[-1]] - 2 * bar[order[-1]] - 2 * bar[tok_gpu]
    return tok_gpu


def _step_vs_oracle(q8, name, max_seq, pos0, count, matvec=None):
    cfg, w, st = _step(q8, name, max_seq)
    kc, vc = _oracle_caches(cfg)
    toks, logits, xs = _run_tokens(q8, st, q8.MODE_GRAPH, pos0, 11, count)
    tok_in = 11
    for i in range(count):
        log("  oracle %s token %d of %d" % (name, i + 1, count))
        _compare_step(cfg, w, kc, vc, tok_in, pos0 + i, logits[i], xs[i], toks[i], name, matvec)
        tok_in = toks[i]    # teacher-forced on the GPU's token
    kvw = cfg["n_kv_heads"] * cfg["head_dim"]
    kc_gpu = down(st.buffer("k_cache")).reshape(cfg["n_layers"], max_seq, kvw)
    for l in range(cfg["n_layers"]):
        ref = kc[l][pos0:pos0 + count].astype(np.float64)
        _check(kc_gpu[l, pos0:pos0 + count], ref,
               STEP_BAR * (np.abs(ref) + float(np.sqrt(np.mean(ref ** 2)))), "k cache layer %d" % l)
        assert not np.any(kc_gpu[l, :pos0]) and not np.any(kc_gpu[l, pos0 + count:])
    st.close()


@pytest.mark.parametrize("name,max_seq,pos0,count", [
    ("step_tiny", 64, 0, 5), ("step_gqa4", 64, 0, 4), ("step_gqa4", 1100, 1000, 3),
    ("step_hd192", 300, 126, 4), ("step_hd256", 200, 0, 3), ("step_hd256", 200, 127, 3),
], ids=str)
def test_step_matches_oracle(q8, name, max_seq, pos0, count):
    log("step vs oracle %s max_seq=%d pos0=%d" % (name, max_seq, pos0))
    _step_vs_oracle(q8, name, max_seq, pos0, count)


@pytest.mark.parametrize("name,max_seq,pos0,count", [
    ("qwen3_0.6b", 1024, 0, 2), ("qwen3_0.6b", 1024, 511, 2), ("7b", 64, 0, 1),
], ids=str)
def test_step_benchmarked_shapes(q8, name, max_seq, pos0, count):
    """The step at the shapes the bench times (page "IV.4: One command buffer
    per token", sections "The correctness ladder" and "Running it"): the
    Qwen3-0.6B shape (28 layers, hidden 1024, 16 query heads on 8 KV heads,
    vocabulary 151936) from position 0 and from 511, and the 7B-class shape
    (hidden 3584, 28 on 4 heads, intermediate 18944) from 0, every logit and
    the residual against the oracle step, whose matvecs run on host threads."""
    import torch
    log("step vs oracle %s max_seq=%d pos0=%d" % (name, max_seq, pos0))
    _step_vs_oracle(q8, name, max_seq, pos0, count, matvec=oracle.gemv_threaded)
    torch.cuda.empty_cache()


def test_step_refuses_past_max_seq(q8):
    log("step max_seq guard")
    _, _, st = _step(q8, "step_tiny", 4)
    st.reset(2, 1)
    st.run(q8.MODE_GRAPH)
    st.run(q8.MODE_EAGER)
    with pytest.raises(q8.Q8Error) as e:
        st.run(q8.MODE_GRAPH)
    assert e.value.code == q8.Q8_ERR_SHAPE
    assert int(down(st.buffer("pos"))[0]) == 4
    with pytest.raises(q8.Q8Error):
        st.reset(4, 0)
    st.close()
