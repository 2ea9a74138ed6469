"""CPU oracle for the rest of a decode step -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this module; the HIP library never does.

The page "IV.4: One command buffer per token" (section "Eight kernels")
defines, besides q8_matvec, the seven kernels one decode step needs:
rms_norm_row, rope_row, append_kv, attention_decode, add_inplace,
silu_hadamard and argmax_row; its section "One command buffer" wires them
into the step (per layer: norm, q/k/v projections, per-head q and k norms,
rotary embedding of q and k, cache append, attention, output projection,
residual add, norm, gate and up projections, SwiGLU, down projection,
residual add; then the final norm, the lm_head and argmax).

Each function below is that definition evaluated in float64 from float32
inputs, in the order the definition is written, and returns float64 (the
step rounds to float32 where the method stores a float32 buffer).  numpy
supplies the elementary operations (exp, sin, cos, sqrt, power) and sums.
Readings taken where the page leaves a step open:

* rope_row: the rotation angle is pos * theta**(-i / half) exactly (the
  page evaluates it in float32 with correctly rounded pow/cos/sin; the
  exact angle is what those calls approximate).
* argmax_row: comparisons as the page writes them -- a value wins if it is
  greater, or equal with a lower index; NaN never wins, and a row of only
  NaN gives 0xFFFFFFFF, the page's initial index.
* decode_step: the embedding row is looked up from the token id (the page
  does it on the host before encoding); a token id outside the vocabulary
  (only the all-NaN argmax produces one) gives a zero row.  Every buffer
  the method keeps in float32 is rounded to float32 between the steps.
"""
from __future__ import annotations

import numpy as np

from oracle import gemv as _q8_gemv

NO_INDEX = 0xFFFFFFFF


def _f64(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def rms_norm_rows(x, w, dim: int, eps: float) -> np.ndarray:
    """Each row of x (rows x dim): x * (mean(x^2) + eps)^(-1/2) * w."""
    x = _f64(x).reshape(-1, dim)
    w = _f64(w).reshape(dim)
    ms = np.sum(x * x, axis=1) / dim
    inv = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    return x * inv[:, None] * w[None, :]


def rope_rows(x, head_dim: int, pos: int, theta: float) -> np.ndarray:
    """Each head of x (heads x head_dim): pairs (i, i + head_dim/2) rotated
    by the angle pos * theta^(-i / (head_dim/2))."""
    x = _f64(x).reshape(-1, head_dim)
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(np.float32(theta)), -i / half)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def append_kv(k, v, kc, vc, width: int, pos: int):
    """Copies of the caches with row `pos` set to k and v."""
    kc = np.array(kc, dtype=np.float32, copy=True).reshape(-1, width)
    vc = np.array(vc, dtype=np.float32, copy=True).reshape(-1, width)
    kc[pos] = np.asarray(k, dtype=np.float32).reshape(width)
    vc[pos] = np.asarray(v, dtype=np.float32).reshape(width)
    return kc, vc


def attention_decode(q, kc, vc, seq: int, kv_width: int, head_dim: int, n_heads: int,
                     kv_group: int):
    """Per query head h, on KV head h / kv_group: scores over the first seq
    cached rows scaled by 1/sqrt(head_dim), softmax, weighted sum of V.
    Returns (out, weights): out is n_heads x head_dim, weights n_heads x seq
    (the softmax, for the tests' bars)."""
    q = _f64(q).reshape(n_heads, head_dim)
    kc = _f64(kc).reshape(-1, kv_width)[:seq]
    vc = _f64(vc).reshape(-1, kv_width)[:seq]
    out = np.empty((n_heads, head_dim))
    weights = np.empty((n_heads, seq))
    scale = 1.0 / np.sqrt(float(head_dim))
    for h in range(n_heads):
        off = (h // kv_group) * head_dim
        k = kc[:, off:off + head_dim]
        v = vc[:, off:off + head_dim]
        scores = (k @ q[h]) * scale
        e = np.exp(scores - np.max(scores))
        p = e / np.sum(e)
        weights[h] = p
        out[h] = p @ v
    return out, weights


def add_inplace(x, y) -> np.ndarray:
    return _f64(x) + _f64(y)


def silu_hadamard(gate, up) -> np.ndarray:
    """(g / (1 + e^-g)) * up, elementwise."""
    g = _f64(gate)
    return (g / (1.0 + np.exp(-g))) * _f64(up)


def argmax_row(x) -> int:
    """The index of the largest value, ties to the lowest index, NaN never
    winning (a linear scan with the page's comparison)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    best, besti = -np.inf, NO_INDEX
    for i, v in enumerate(x.tolist()):
        if v > best or (v == best and i < besti):
            best, besti = v, i
    return besti


def _r32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def decode_step(cfg: dict, w: dict, kc: list, vc: list, token: int, pos: int, matvec=None):
    """One decode step of a Qwen3-style model in the order of section "One
    command buffer": per layer norm, q/k/v projections, per-head q and k
    norms, rotary embedding at pos, cache append at pos, attention over pos + 1
    rows, output projection, residual add, norm, gate and up projections,
    SwiGLU, down projection, residual add; then the final norm, the lm_head
    and argmax.  The Q8_0 projections are the oracle's matvec.

    kc, vc: per layer float32 (max_seq, kv_width) caches, updated in place.
    matvec: the Q8_0 matvec to use, (w, x, n, p) -> (y, y64, mag) (default
    the serial oracle; oracle.gemv_threaded gives the same results).
    Returns (next token, logits float32, logits float64, logits magnitude
    sum_j |w_j x_j| per row, final residual x float32).
    """
    hid, hd = cfg["hidden"], cfg["head_dim"]
    nh, nkv, inter = cfg["n_heads"], cfg["n_kv_heads"], cfg["inter"]
    eps, theta, vocab = cfg["eps"], cfg["theta"], cfg["vocab"]
    qw, kvw = nh * hd, nkv * hd

    gemv = matvec or _q8_gemv

    def mv(wt, x, n, p):
        return gemv(wt, x, n, p)[0]

    x = (np.asarray(w["embed"], np.float32).reshape(vocab, hid)[token].copy()
         if 0 <= token < vocab else np.zeros(hid, np.float32))
    for l, L in enumerate(w["layers"]):
        xn = _r32(rms_norm_rows(x, L["attn_norm"], hid, eps)).reshape(-1)
        q = mv(L["wq"], xn, hid, qw)
        k = mv(L["wk"], xn, hid, kvw)
        v = mv(L["wv"], xn, hid, kvw)
        q = _r32(rms_norm_rows(q, L["q_norm"], hd, eps))
        k = _r32(rms_norm_rows(k, L["k_norm"], hd, eps))
        q = _r32(rope_rows(q, hd, pos, theta)).reshape(-1)
        k = _r32(rope_rows(k, hd, pos, theta)).reshape(-1)
        kc[l], vc[l] = append_kv(k, v, kc[l], vc[l], kvw, pos)
        a = _r32(attention_decode(q, kc[l], vc[l], pos + 1, kvw, hd, nh, nh // nkv)[0]).reshape(-1)
        x = _r32(add_inplace(x, mv(L["wo"], a, qw, hid)))
        xn = _r32(rms_norm_rows(x, L["ffn_norm"], hid, eps)).reshape(-1)
        h = _r32(silu_hadamard(mv(L["wgate"], xn, hid, inter), mv(L["wup"], xn, hid, inter)))
        x = _r32(add_inplace(x, mv(L["wdown"], h, inter, hid)))
    xn = _r32(rms_norm_rows(x, w["out_norm"], hid, eps)).reshape(-1)
    y, y64, mag = gemv(w["lm_head"], xn, hid, vocab)
    return argmax_row(y), y, y64, mag, x
