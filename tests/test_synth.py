"""The seeded input generators: shapes, ranges, determinism, workload sizes."""
import numpy as np

import synth


def test_weights_layout_and_ranges():
    rng = np.random.default_rng(3)
    n, p = 1024, 300
    w = synth.q8_weights(n, p, rng)
    assert w.dtype == np.uint8 and w.size == p * (n // 32) * 34
    blk = w.reshape(-1, 34)
    d = blk[:, 0:2].copy().view("<f2")[:, 0].astype(np.float64)
    assert d.min() >= np.float16(0.001) and d.max() <= np.float16(0.02)
    q = blk[:, 2:].copy().view(np.int8)
    assert q.min() == -127 and q.max() == 127          # -128 never drawn
    counts = np.bincount(q.reshape(-1).astype(np.int64) + 127, minlength=255)
    assert counts.size == 255 and counts.min() > 0.8 * counts.mean()


def test_activations_distribution():
    x = synth.activations(1 << 16, np.random.default_rng(4))
    assert x.dtype == np.float32
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02


def test_determinism():
    a = synth.generate("single_1024x3072")
    b = synth.generate("single_1024x3072")
    assert np.array_equal(a[0][1], b[0][1]) and np.array_equal(a[0][2], b[0][2])
    w0, x0 = synth.generate_smallm(synth.SMALLM_SHAPES[0], 2)
    assert x0.shape == (2, 18944)


def test_workload_sizes():
    # per-token algorithmic bytes (weights + x + y) of each decode chain
    expect = {"single_1024x3072": (1, 3358720), "qwen3_0.6b_chain": (197, 636368384),
              "qwen2.5_0.5b_chain": (169, 527644672), "7b_chain": (197, 7522893824)}
    for name, (count, nbytes) in expect.items():
        ops = synth.WORKLOADS[name]
        assert len(ops) == count and synth.workload_bytes(ops) == nbytes


def test_page_lcg_first_draws():
    # first draw for seed 7 worked with Python integers
    s = (7 * 6364136223846793005 + 1442695040888963407) % (1 << 64)
    first = np.float32(np.float32(s >> 33) / np.float32(2.0 ** 31)) - np.float32(1.0)
    v, _ = synth.page_lcg_f32(7, 3)
    assert v[0] == first and v.dtype == np.float32
    w = synth.page_q8_bytes(50, 96, 7)
    assert w.size == 50 * 3 * 34
    assert np.all(w.reshape(-1, 34)[:, 0] == 0x00) and np.all(w.reshape(-1, 34)[:, 1] == 0x2C)
