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
"""
from __future__ import annotations

import numpy as np

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
