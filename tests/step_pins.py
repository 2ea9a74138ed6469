"""Checks that pin the decode-step oracle (oracle/decode_step.py) to facts
that do not come from it: the hand-worked values in
golden/step_hand_worked.txt, closed forms and invariants of each operation,
and numpy's argmax on data without ties or NaN.

Every check takes a module-like object with the oracle's functions, so the
same checks run on the real oracle (all must pass) and on copies with a
planted mistake (at least one must fail).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "step_hand_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, _, v = line.partition(" ")
                vals[k] = float(v)
    return vals


def _close(a, b, tol=1e-12):
    assert np.allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=tol, atol=tol), (a, b)


# ---------------------------------------------------------------- rms_norm_row
def pin_rms_hand_worked(o):
    g = _golden()
    out = o.rms_norm_rows([3.0, 4.0], [1.0, 2.0], 2, 0.0)
    _close(out[0], [g["rms_out0"], g["rms_out1"]])


def pin_rms_unit_mean_square(o):
    """With unit weights and eps = 0 every row comes out with mean square 1,
    and scaling a row by c > 0 leaves it unchanged."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    out = o.rms_norm_rows(x, np.ones(96, np.float32), 96, 0.0)
    _close(np.mean(out * out, axis=1), np.ones(5), 1e-12)
    out2 = o.rms_norm_rows(x * np.float32(4.0), np.ones(96, np.float32), 96, 0.0)
    _close(out2, out, 1e-12)


def pin_rms_eps(o):
    """A zero row stays zero; eps = 3 on a row of ones divides by 2."""
    assert np.all(o.rms_norm_rows(np.zeros(8, np.float32), np.ones(8, np.float32), 8, 1e-6) == 0)
    _close(o.rms_norm_rows(np.ones(8, np.float32), np.ones(8, np.float32), 8, 3.0)[0],
           np.full(8, 0.5))


# ---------------------------------------------------------------- rope_row
def pin_rope_hand_worked(o):
    g = _golden()
    e = np.eye(4, dtype=np.float32)
    _close(o.rope_rows(e[0], 4, 1, 10000.0)[0], [g["cos1"], 0, g["sin1"], 0])
    _close(o.rope_rows(e[1], 4, 1, 10000.0)[0], [0, g["cos001"], 0, g["sin001"]])
    _close(o.rope_rows(e[2], 4, 1, 10000.0)[0], [-g["sin1"], 0, g["cos1"], 0])


def pin_rope_invariants(o):
    """pos 0 is the identity; every pair keeps its length; turning by a
    then by b equals turning by a + b."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    _close(o.rope_rows(x, 64, 0, 1e6), x.astype(np.float64))
    y = o.rope_rows(x, 64, 37, 1e6)
    n0 = x[:, :32].astype(np.float64) ** 2 + x[:, 32:].astype(np.float64) ** 2
    n1 = y[:, :32] ** 2 + y[:, 32:] ** 2
    _close(n1, n0, 1e-12)
    x2 = np.array([[1.0, 0.5, -2.0, 0.25]], np.float32)
    two = o.rope_rows(o.rope_rows(x2, 4, 3, 100.0).astype(np.float32), 4, 5, 100.0)
    _close(two, o.rope_rows(x2, 4, 8, 100.0), 1e-6)


# ---------------------------------------------------------------- attention_decode
def pin_attention_hand_worked(o):
    g = _golden()
    q = np.array([1, 0, 0, 0], np.float32)
    kc = np.array([[2, 0, 0, 0], [0, 0, 0, 0]], np.float32)
    vc = np.array([[1, 0, 0, 0], [0, 1, 0, 0]], np.float32)
    out, w = o.attention_decode(q, kc, vc, 2, 4, 4, 1, 1)
    _close(w[0], [g["attn_w0"], g["attn_w1"]])
    _close(out[0], [g["attn_w0"], g["attn_w1"], 0, 0])


def pin_attention_special_cases(o):
    """seq 1 returns that V row; a zero query weighs all rows equally (the
    mean of V); only the first seq rows of the cache count."""
    rng = np.random.default_rng(3)
    kc = rng.standard_normal((6, 8)).astype(np.float32)
    vc = rng.standard_normal((6, 8)).astype(np.float32)
    q = rng.standard_normal(8).astype(np.float32)
    out, _ = o.attention_decode(q, kc, vc, 1, 8, 8, 1, 1)
    _close(out[0], vc[0])
    out, _ = o.attention_decode(np.zeros(8, np.float32), kc, vc, 4, 8, 8, 1, 1)
    _close(out[0], vc[:4].astype(np.float64).mean(axis=0))


def pin_attention_gqa(o):
    """Query heads h read KV head h / kv_group: with 4 query heads on 2 KV
    heads, heads 0 and 1 see KV head 0 and heads 2 and 3 KV head 1."""
    rng = np.random.default_rng(4)
    hd, seq = 4, 5
    kc = rng.standard_normal((seq, 2 * hd)).astype(np.float32)
    vc = rng.standard_normal((seq, 2 * hd)).astype(np.float32)
    q1 = rng.standard_normal(hd).astype(np.float32)
    q = np.tile(q1, 4)
    out, _ = o.attention_decode(q, kc, vc, seq, 2 * hd, hd, 4, 2)
    for h, kvh in ((0, 0), (1, 0), (2, 1), (3, 1)):
        ref, _ = o.attention_decode(q1, kc[:, kvh * hd:(kvh + 1) * hd],
                                    vc[:, kvh * hd:(kvh + 1) * hd], seq, hd, hd, 1, 1)
        _close(out[h], ref[0])


def pin_attention_permutation(o):
    """Reordering the cached (key, value) rows together changes nothing."""
    rng = np.random.default_rng(5)
    kc = rng.standard_normal((7, 16)).astype(np.float32)
    vc = rng.standard_normal((7, 16)).astype(np.float32)
    q = rng.standard_normal(32).astype(np.float32)
    perm = rng.permutation(7)
    a, _ = o.attention_decode(q, kc, vc, 7, 16, 16, 2, 2)
    b, _ = o.attention_decode(q, kc[perm], vc[perm], 7, 16, 16, 2, 2)
    _close(a, b, 1e-12)


# ---------------------------------------------------------------- silu, add, append, argmax
def pin_silu_identities(o):
    """silu(g) - silu(-g) = g; silu(0) = 0; and silu(g) = (g/2)(1 + tanh(g/2))."""
    g = np.array([-30.0, -2.5, -0.75, 0.0, 0.5, 1.5, 3.25, 30.0], np.float32)
    up = np.ones_like(g)
    s = o.silu_hadamard(g, up)
    _close(s - o.silu_hadamard(-g, up), g.astype(np.float64), 1e-12)
    assert s[3] == 0
    gd = g.astype(np.float64)
    _close(s, 0.5 * gd * (1.0 + np.tanh(0.5 * gd)), 1e-12)
    _close(o.silu_hadamard(g, np.full_like(g, -3.0)), -3.0 * s, 1e-12)


def pin_add_exact(o):
    """Two float32 values add exactly in float64."""
    x = np.array([1.0, 3.0e38, 1e-45, -7.25], np.float32)
    y = np.array([2.0 ** -30, 3.0e38, 1e-45, 7.25], np.float32)
    got = o.add_inplace(x, y)
    for a, b, c in zip(x.tolist(), y.tolist(), got.tolist()):
        assert Fraction(c) == Fraction(a) + Fraction(b)


def pin_append(o):
    kc = np.zeros((4, 3), np.float32)
    vc = np.ones((4, 3), np.float32)
    k2, v2 = o.append_kv([1, 2, 3], [4, 5, 6], kc, vc, 3, 2)
    ek = np.zeros((4, 3)); ek[2] = [1, 2, 3]
    ev = np.ones((4, 3)); ev[2] = [4, 5, 6]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert np.all(kc == 0) and np.all(vc == 1)   # inputs untouched


def pin_argmax(o):
    """Ties go to the lowest index; NaN never wins; all NaN gives
    0xFFFFFFFF; all -inf gives 0; without ties or NaN it is numpy's argmax."""
    assert o.argmax_row(np.array([1, 3, 3, 2], np.float32)) == 1
    assert o.argmax_row(np.array([np.nan, 1, np.nan, 1], np.float32)) == 1
    assert o.argmax_row(np.array([np.nan, np.nan], np.float32)) == 0xFFFFFFFF
    assert o.argmax_row(np.array([-np.inf, -np.inf], np.float32)) == 0
    assert o.argmax_row(np.array([0.0, -0.0], np.float32)) == 0
    rng = np.random.default_rng(6)
    x = rng.permutation(5000).astype(np.float32)
    assert o.argmax_row(x) == int(np.argmax(x))


# ---------------------------------------------------------------- the composed step
# A one-layer model whose projections are 0/1 (or 0/2) selection matrices
# with unit scales, so each stage's result is a plain function of the
# previous one: the step must reduce to the pinned pieces above, in the
# order and with the weights the step's wiring prescribes.
_S = dict(n_layers=1, hidden=256, n_heads=8, n_kv_heads=2, head_dim=32, inter=512, vocab=8,
          eps=1e-6, theta=1e4)


def _q8(dense):
    """Q8_0 bytes of an integer matrix (|entries| <= 127) with scale 1."""
    import synth
    dense = np.asarray(dense)
    p, n = dense.shape
    nb = p * n // 32
    return synth.pack_blocks(np.ones(nb, np.float16), dense.astype(np.int8).reshape(nb, 32))


def _sel(p, n, k=1):
    m = np.zeros((p, n), np.int64)
    r = min(p, n)
    m[np.arange(r), np.arange(r)] = k
    return m


def _structured(attention: bool):
    c = _S
    hid, qw, kvw, inter = c["hidden"], c["n_heads"] * c["head_dim"], c["n_kv_heads"] * c["head_dim"], c["inter"]
    rng = np.random.default_rng(11)
    z = lambda p, n: np.zeros((p, n), np.int64)
    L = {"wq": _sel(qw, hid) if attention else z(qw, hid),
         "wk": _sel(kvw, hid) if attention else z(kvw, hid),
         "wv": _sel(kvw, hid) if attention else z(kvw, hid),
         "wo": _sel(hid, qw) if attention else z(hid, qw),
         "wgate": z(inter, hid) if attention else _sel(inter, hid),
         "wup": z(inter, hid) if attention else _sel(inter, hid, 2),
         "wdown": z(hid, inter) if attention else _sel(hid, inter)}
    L = {k: _q8(v) for k, v in L.items()}
    for k, lo in (("attn_norm", 0.5), ("ffn_norm", 1.5), ("q_norm", 0.7), ("k_norm", 1.2)):
        dim = c["head_dim"] if k in ("q_norm", "k_norm") else hid
        L[k] = rng.uniform(lo, lo + 0.3, dim).astype(np.float32)
    lm = np.zeros((c["vocab"], hid), np.int64)
    lm[np.arange(c["vocab"]), 3 * np.arange(c["vocab"])] = 1     # logit r = x_final[3 r]
    w = {"embed": rng.standard_normal((c["vocab"], hid)).astype(np.float32),
         "out_norm": rng.uniform(0.9, 1.1, hid).astype(np.float32),
         "lm_head": _q8(lm), "layers": [L]}
    caches = ([np.zeros((4, kvw), np.float32)], [np.zeros((4, kvw), np.float32)])
    return c, w, caches


def _f32(a):
    return np.asarray(a, np.float64).astype(np.float32)


def pin_step_attention_wiring(o):
    """Selection projections, zero FFN: after two tokens the residual is
    embed + attention output (query head h reading KV head h // group),
    the caches hold the normed, rotated keys and the values at rows 0, 1,
    and the logits are the final norm of the residual at the lm_head's
    selected columns."""
    c, w, (kc, vc) = _structured(True)
    L, hd, nh, kvw = w["layers"][0], c["head_dim"], c["n_heads"], c["n_kv_heads"] * c["head_dim"]
    for pos, tok in enumerate((3, 6)):
        tok_out, y, _, _, x = o.decode_step(c, w, kc, vc, tok, pos)
        e = w["embed"][tok]
        xn = _f32(o.rms_norm_rows(e, L["attn_norm"], c["hidden"], c["eps"])).reshape(-1)
        q = _f32(o.rope_rows(_f32(o.rms_norm_rows(xn, L["q_norm"], hd, c["eps"])), hd, pos, c["theta"]))
        k = _f32(o.rope_rows(_f32(o.rms_norm_rows(xn[:kvw], L["k_norm"], hd, c["eps"])), hd, pos,
                             c["theta"])).reshape(-1)
        _close(kc[0][pos], k, 1e-7)
        _close(vc[0][pos], xn[:kvw], 0)
        assert not np.any(kc[0][pos + 1:]) and not np.any(vc[0][pos + 1:])
        keys = kc[0][:pos + 1].astype(np.float64)
        vals = vc[0][:pos + 1].astype(np.float64)
        a = np.empty((nh, hd))
        for h in range(nh):
            g = h // (nh // c["n_kv_heads"])
            sc = keys[:, g * hd:(g + 1) * hd] @ q.reshape(nh, hd)[h].astype(np.float64) / math.sqrt(hd)
            p = np.exp(sc - sc.max())
            a[h] = (p / p.sum()) @ vals[:, g * hd:(g + 1) * hd]
        if pos == 0:   # one cached row: the output is that row's values
            _close(a.reshape(-1), np.repeat(xn[:kvw].reshape(2, 1, hd), 4, axis=1).reshape(-1), 1e-12)
        x_ref = _f32(e.astype(np.float64) + _f32(a).reshape(-1))
        _close(x, x_ref, 1e-6)
        fin = _f32(o.rms_norm_rows(x_ref, w["out_norm"], c["hidden"], c["eps"])).reshape(-1)
        _close(y, fin[3 * np.arange(c["vocab"])], 1e-6)
        assert tok_out == int(np.argmax(fin[3 * np.arange(c["vocab"])]))


def pin_step_ffn_wiring(o):
    """Zero attention, gate = selection, up = 2 x selection, down =
    selection: the residual gains silu(g) * 2 g for g the ffn-normed
    embedding (SiLU on the gate, not on the up projection)."""
    c, w, (kc, vc) = _structured(False)
    L = w["layers"][0]
    _, y, _, _, x = o.decode_step(c, w, kc, vc, 5, 0)
    e = w["embed"][5].astype(np.float64)
    g = _f32(o.rms_norm_rows(e, L["ffn_norm"], c["hidden"], c["eps"])).reshape(-1).astype(np.float64)
    x_ref = _f32(e + _f32(g / (1.0 + np.exp(-g)) * (2.0 * g)))
    _close(x, x_ref, 1e-6)
    assert not np.any(vc[0])    # zero projections leave zero values


ALL_PINS = [
    pin_rms_hand_worked, pin_rms_unit_mean_square, pin_rms_eps,
    pin_rope_hand_worked, pin_rope_invariants,
    pin_attention_hand_worked, pin_attention_special_cases, pin_attention_gqa,
    pin_attention_permutation,
    pin_silu_identities, pin_add_exact, pin_append, pin_argmax,
    pin_step_attention_wiring, pin_step_ffn_wiring,
]
