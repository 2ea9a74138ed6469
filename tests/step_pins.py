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


ALL_PINS = [
    pin_rms_hand_worked, pin_rms_unit_mean_square, pin_rms_eps,
    pin_rope_hand_worked, pin_rope_invariants,
    pin_attention_hand_worked, pin_attention_special_cases, pin_attention_gqa,
    pin_attention_permutation,
    pin_silu_identities, pin_add_exact, pin_append, pin_argmax,
]
