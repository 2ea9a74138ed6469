"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the CPU
baseline records, and the traffic record's match on workload and kernel."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baselines_are_records_of_the_oracle():
    import bench
    import synth
    data = synth.generate("qwen3_0.6b_chain")[:3]
    for rec, cores in ((bench.cpu_baseline(data, 0.05), 1),
                       (bench.cpu_baseline_threaded(data, 0.05, 3), 3)):
        assert rec["kind"] == "oracle" and rec["unit"] == "GB/s"
        assert rec["cores"] == cores and rec["value"] > 0
        json.dumps(rec)


def test_row_ranges_reproduce_the_whole_op():
    """The all-cores baseline runs the oracle on contiguous row ranges; the
    ranges' rows are the whole op's rows, bit for bit."""
    import oracle
    import synth
    rng = np.random.default_rng(5)
    n, p = 256, 67
    w = synth.q8_weights(n, p, rng)
    x = synth.activations(n, rng)
    _, y64, mag = oracle.gemv(w, x, n, p)
    rb = synth.row_bytes(n)
    wf = w.reshape(-1)
    cuts = [p * k // 4 for k in range(5)]
    parts = [oracle.gemv(wf[a * rb:b * rb], x, n, b - a) for a, b in zip(cuts, cuts[1:])]
    assert np.array_equal(np.concatenate([q[1] for q in parts]), y64)
    assert np.array_equal(np.concatenate([q[2] for q in parts]), mag)


def test_traffic_record_needs_its_kernel():
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert bench.measured_traffic(rec["workload"], rec["kernel"] + "x") is None
    assert bench.measured_traffic("no_such_workload", rec["kernel"]) is None
    got = bench.measured_traffic(rec["workload"], rec["kernel"])
    if rec["kernel_digest"] == bench.kernel_digest():
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None
