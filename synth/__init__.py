"""Seeded synthetic inputs for the Q8_0 decode matvec.

This module is shared by the tests, the bench and the smoke check: it feeds
the HIP library and the CPU oracle the same bytes.  It holds none of the
matvec's arithmetic: it only draws random numbers, rounds scales to binary16
with numpy's own cast, and lays the bytes out in the Q8_0 block format
(page "IV.4: One command buffer per token", section "Eight kernels": a block
is a little-endian binary16 scale followed by 32 int8 quants, 34 bytes; a
row is n/32 consecutive blocks; rows follow each other).

Workload shapes follow the decode step of that page's section "One command
buffer" (per layer: q, k, v, o, gate, up, down, then one lm_head after the
last layer) at three model sizes.  Value distributions: scale uniform in
[0.001, 0.02] rounded to binary16 (round to nearest even), quants uniform
over the 255 integers in [-127, 127], activations float32 N(0, 1).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np

BLOCK_QUANTS = 32
BLOCK_BYTES = 34
SEED_BASE = 0x51385F30

ROLE_W = 0
ROLE_X = 1
ROLE_NORM = 2
ROLE_EMBED = 3


def row_bytes(n: int) -> int:
    return (n // BLOCK_QUANTS) * BLOCK_BYTES


def rng_for(cfg: int, op: int, role: int) -> np.random.Generator:
    """Independent PCG64 stream for (workload, op index in encode order, role)."""
    return np.random.default_rng(np.random.SeedSequence([SEED_BASE, cfg, op, role]))


def pack_blocks(scale_f16: np.ndarray, quants: np.ndarray) -> np.ndarray:
    """Lay out blocks: scale_f16 (nblocks,) float16, quants (nblocks, 32) int8."""
    nb = scale_f16.size
    out = np.empty((nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(scale_f16.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 2:] = quants.reshape(nb, BLOCK_QUANTS).view(np.uint8)
    return out.reshape(-1)


def q8_weights(n: int, p: int, rng: np.random.Generator,
               scale_lo: float = 0.001, scale_hi: float = 0.02) -> np.ndarray:
    """p x n Q8_0 matrix as a flat uint8 array of p*(n/32)*34 bytes."""
    if n % BLOCK_QUANTS:
        raise ValueError("n must be a multiple of 32")
    nb = p * (n // BLOCK_QUANTS)
    scale = rng.uniform(scale_lo, scale_hi, size=nb).astype(np.float16)
    quants = rng.integers(-127, 128, size=(nb, BLOCK_QUANTS), dtype=np.int8)
    return pack_blocks(scale, quants)


def activations(n: int, rng: np.random.Generator, m: int = 1) -> np.ndarray:
    """float32 N(0,1); shape (n,) for m == 1, else (m, n) row-major."""
    x = rng.standard_normal(n * m, dtype=np.float32)
    return x if m == 1 else x.reshape(m, n)


def integer_case(n: int, p: int, rng: np.random.Generator,
                 scale_bits: int = 0x2C00, xmax: int = 4):
    """Every scale the bit pattern 0x2C00 (the page's fabricator bytes 0x00
    0x2c), quants uniform in [-127, 127], x integers in [-xmax, xmax]."""
    nb = p * (n // BLOCK_QUANTS)
    scale = np.full(nb, scale_bits, dtype=np.uint16).view(np.float16)
    quants = rng.integers(-127, 128, size=(nb, BLOCK_QUANTS), dtype=np.int8)
    x = rng.integers(-xmax, xmax + 1, size=n).astype(np.float32)
    return pack_blocks(scale, quants), x


# ---------------------------------------------------------------------------
# The page's own test-input generator (section "The correctness ladder",
# rung one): a 64-bit linear congruential generator whose state advances as
# s = s * 6364136223846793005 + 1442695040888963407 (mod 2^64); each draw is
# float32((s >> 33)) / 2^31 - 1 in float32.  Its weight fabricator writes
# scale bytes 0x00 0x2c for every block and quant = trunc(draw * 127) as i8.
# ---------------------------------------------------------------------------
_LCG_A = 6364136223846793005
_LCG_C = 1442695040888963407
_M64 = (1 << 64) - 1


def page_lcg_f32(seed: int, count: int) -> Tuple[np.ndarray, int]:
    """`count` draws of the page's generator; returns (draws, final state)."""
    s = seed & _M64
    hi = np.empty(count, dtype=np.float64)
    for i in range(count):
        s = (s * _LCG_A + _LCG_C) & _M64
        hi[i] = s >> 33
    v = (hi.astype(np.float32) / np.float32(2.0 ** 31)) - np.float32(1.0)
    return v.astype(np.float32), s


def page_q8_bytes(rows: int, cols: int, seed: int) -> np.ndarray:
    nb = rows * (cols // BLOCK_QUANTS)
    draws, _ = page_lcg_f32(seed, nb * BLOCK_QUANTS)
    q = np.trunc(draws * np.float32(127.0)).astype(np.int8).reshape(nb, BLOCK_QUANTS)
    scale = np.full(nb, 0x2C00, dtype=np.uint16).view(np.float16)
    return pack_blocks(scale, q)


def page_x(n: int, seed: int = 42) -> np.ndarray:
    return page_lcg_f32(seed, n)[0]


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class OpShape:
    name: str
    n: int   # input width
    p: int   # output rows


def _decoder_chain(layers: int, proj: Sequence[Tuple[str, int, int]],
                   lm: Tuple[int, int]) -> List[OpShape]:
    ops = []
    for li in range(layers):
        for nm, n, p in proj:
            ops.append(OpShape("L%d.%s" % (li, nm), n, p))
    ops.append(OpShape("lm_head", lm[0], lm[1]))
    return ops


WORKLOADS: Dict[str, List[OpShape]] = {
    # a single matvec at the Qwen3-0.6B FFN-up shape
    "single_1024x3072": [OpShape("ffn_up", 1024, 3072)],
    # Qwen3-0.6B decode step: 28 layers x 7 projections + lm_head = 197 matvecs
    "qwen3_0.6b_chain": _decoder_chain(28, [("q", 1024, 2048), ("k", 1024, 1024),
                                            ("v", 1024, 1024), ("o", 2048, 1024),
                                            ("gate", 1024, 3072), ("up", 1024, 3072),
                                            ("down", 3072, 1024)], (1024, 151936)),
    # Qwen2.5-0.5B-shaped decode step: 24 x 7 + lm_head = 169 matvecs
    "qwen2.5_0.5b_chain": _decoder_chain(24, [("q", 896, 896), ("k", 896, 128),
                                              ("v", 896, 128), ("o", 896, 896),
                                              ("gate", 896, 4864), ("up", 896, 4864),
                                              ("down", 4864, 896)], (896, 151936)),
    # 7B-class decode step: 28 x 7 + lm_head = 197 matvecs
    "7b_chain": _decoder_chain(28, [("q", 3584, 3584), ("k", 3584, 512),
                                    ("v", 3584, 512), ("o", 3584, 3584),
                                    ("gate", 3584, 18944), ("up", 3584, 18944),
                                    ("down", 18944, 3584)], (3584, 152064)),
}

# workload number used in the seeds, in the order the workloads are listed
WORKLOAD_ID = {"single_1024x3072": 0, "qwen3_0.6b_chain": 1,
               "qwen2.5_0.5b_chain": 2, "7b_chain": 3, "smallm_7b": 4,
               "step_tiny": 5, "step_gqa4": 6, "step_hd192": 7, "step_hd256": 8}

# small-batch products: X is m x n, m in {2, 4, 8, 16}, at three 7B shapes
SMALLM_SHAPES = [OpShape("down", 18944, 3584), OpShape("gate", 3584, 18944),
                 OpShape("lm_head", 3584, 152064)]
SMALLM_M = (2, 4, 8, 16)


def workload_bytes(ops: Sequence[OpShape], m: int = 1) -> int:
    """Algorithmic bytes: every weight byte once, x once, y once."""
    return sum(op.p * row_bytes(op.n) + 4 * m * op.n + 4 * m * op.p for op in ops)


def _gen_op(cfg: int, i: int, op: OpShape, m: int):
    w = q8_weights(op.n, op.p, rng_for(cfg, i, ROLE_W))
    x = activations(op.n, rng_for(cfg, i, ROLE_X), m)
    return w, x


def generate(workload: str, m: int = 1, threads: int | None = None):
    """Weights and activations of every op of a workload, in encode order.

    Returns a list of (OpShape, w uint8[...], x float32[...]).
    """
    ops = WORKLOADS[workload] if workload in WORKLOADS else None
    if ops is None:
        raise KeyError(workload)
    cfg = WORKLOAD_ID[workload]
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(_gen_op, cfg, i, op, m) for i, op in enumerate(ops)]
        res = [f.result() for f in futs]
    return [(op, w, x) for op, (w, x) in zip(ops, res)]


def generate_smallm(shape: OpShape, m: int):
    """Weights and an m x n activation matrix for one small-batch case."""
    k = [s.name for s in SMALLM_SHAPES].index(shape.name)
    w = q8_weights(shape.n, shape.p, rng_for(WORKLOAD_ID["smallm_7b"], k, ROLE_W))
    x = activations(shape.n, rng_for(WORKLOAD_ID["smallm_7b"], 16 * k + m, ROLE_X), m)
    return w, x


# ------------------------------------------------------------------ whole decode-step models
# Qwen3-style decoders (the step of page "IV.4: One command buffer per token",
# section "One command buffer").  "qwen3_0.6b" has Qwen3-0.6B's shape and the
# very projection bytes of the qwen3_0.6b_chain workload, "7b" the 7B-class
# shape (28 query heads on 4 KV heads of 128) and the 7b_chain bytes; the small ones
# are test models: "step_tiny" (2 layers, head_dim 64, two query heads per
# KV head), "step_gqa4" (head_dim 128, four query heads per KV head, an
# intermediate width and a vocabulary that are not powers of two),
# "step_hd192" (three query heads on one KV head; rows of 12 blocks pair into
# two-row super-rows and the odd vocabulary leaves the lm_head a tail row)
# and "step_hd256".
STEP_MODELS = {
    "qwen3_0.6b": dict(n_layers=28, hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128,
                       inter=3072, vocab=151936, eps=1e-6, theta=1e6),
    "7b": dict(n_layers=28, hidden=3584, n_heads=28, n_kv_heads=4, head_dim=128,
               inter=18944, vocab=152064, eps=1e-6, theta=1e6),
    "step_tiny": dict(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                      inter=512, vocab=1000, eps=1e-6, theta=1e6),
    "step_gqa4": dict(n_layers=1, hidden=512, n_heads=8, n_kv_heads=2, head_dim=128,
                      inter=1376, vocab=4099, eps=1e-6, theta=1e4),
    "step_hd192": dict(n_layers=1, hidden=384, n_heads=3, n_kv_heads=1, head_dim=192,
                       inter=640, vocab=501, eps=1e-5, theta=1e6),
    "step_hd256": dict(n_layers=2, hidden=512, n_heads=4, n_kv_heads=2, head_dim=256,
                       inter=768, vocab=700, eps=1e-6, theta=1e6),
}
STEP_SEED = {"qwen3_0.6b": WORKLOAD_ID["qwen3_0.6b_chain"], "7b": WORKLOAD_ID["7b_chain"],
             "step_tiny": WORKLOAD_ID["step_tiny"],
             "step_gqa4": WORKLOAD_ID["step_gqa4"], "step_hd192": WORKLOAD_ID["step_hd192"],
             "step_hd256": WORKLOAD_ID["step_hd256"]}
PROJ = ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown")
NORMS = ("attn_norm", "ffn_norm", "q_norm", "k_norm")


def step_proj_shapes(cfg: dict):
    """(name, n, p) of the seven projections of one layer, in encode order."""
    hid, inter = cfg["hidden"], cfg["inter"]
    qw, kvw = cfg["n_heads"] * cfg["head_dim"], cfg["n_kv_heads"] * cfg["head_dim"]
    return [("wq", hid, qw), ("wk", hid, kvw), ("wv", hid, kvw), ("wo", qw, hid),
            ("wgate", hid, inter), ("wup", hid, inter), ("wdown", inter, hid)]


def step_model(name: str, threads: int | None = None):
    """(cfg, weights) of a step model.  weights: "embed" float32 (vocab,
    hidden) N(0, 1); "out_norm" and per layer the four norm gains, float32
    uniform in [0.5, 1.5]; "lm_head" and the seven projections per layer as
    flat uint8 Q8_0 (drawn like every other weight here: op index i of the
    encode order -- layer l's projections are 7 l .. 7 l + 6, the lm_head
    7 n_layers -- on the model's seed); "layers" a list of dicts."""
    cfg = dict(STEP_MODELS[name])
    seed = STEP_SEED[name]
    L = cfg["n_layers"]
    shapes = step_proj_shapes(cfg)
    jobs = [(7 * l + j, n, p) for l in range(L) for j, (_, n, p) in enumerate(shapes)]
    jobs.append((7 * L, cfg["hidden"], cfg["vocab"]))
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        ws = list(ex.map(lambda j: q8_weights(j[1], j[2], rng_for(seed, j[0], ROLE_W)), jobs))
    layers = []
    for l in range(L):
        d = {nm: ws[7 * l + j] for j, (nm, _, _) in enumerate(shapes)}
        r = rng_for(seed, l, ROLE_NORM)
        for nm in NORMS:
            dim = cfg["head_dim"] if nm in ("q_norm", "k_norm") else cfg["hidden"]
            d[nm] = r.uniform(0.5, 1.5, size=dim).astype(np.float32)
        layers.append(d)
    r = rng_for(seed, L, ROLE_NORM)
    weights = {"embed": rng_for(seed, 0, ROLE_EMBED).standard_normal(
                   cfg["vocab"] * cfg["hidden"], dtype=np.float32).reshape(cfg["vocab"], cfg["hidden"]),
               "out_norm": r.uniform(0.5, 1.5, size=cfg["hidden"]).astype(np.float32),
               "lm_head": ws[7 * L], "layers": layers}
    return cfg, weights
