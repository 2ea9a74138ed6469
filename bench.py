#!/usr/bin/env python3
"""Benchmark of the Q8_0 decode matvec chain on one MI355X.

One step = one token's chain of matvecs (197 for the 7B-class decode step),
replayed from the recorded hipGraph on torch's current stream, with every
weight and activation already resident in HBM.  Prints ONE JSON line:

  metric / value / unit : achieved HBM GB/s of algorithmic bytes (weights
                          once + x once + y once per op) over the timed steps
  ms_per_step           : milliseconds per token
  roofline              : the dominant (only) kernel of a step, measured with
                          HIP events on the launch stream, against 8 TB/s
  cpu_baseline          : the CPU oracle on a bounded sample of the same
                          workload, on this host (single thread)

Progress goes to stderr.  Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the sources of the chain's kernel: counters taken on other sources are stale
KERNEL_SOURCES = [os.path.join(ROOT, "q8_block_quantized_gemv_amd", "csrc", f)
                  for f in ("q8_gemv_rc.hip", "q8_rc.h", "q8_block.h", "q8_device.h", "q8_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_7b_chain.json")


def say(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the baselines."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on this workload's kernel (same template arguments) and the
    current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("workload") != workload or rec.get("kernel") != kernel
            or rec.get("kernel_digest") != kernel_digest()):
        return None
    return rec.get("hbm_bytes_per_launch")


SETTLE_S = 0.3


def settle(run, sync, seconds: float = SETTLE_S) -> int:
    """Untimed work before the counted warm-up: `run` again and again until
    `seconds` have passed, so that the timed steps find the GPU in its steady
    state (a few milliseconds of warm-up leave the first ~100 replays of a
    100 us chain about 10 % slow).  Returns the number of runs."""
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            run()
        sync()
        n += 8
    return n


def cpu_baseline(data, budget_s: float):
    """The oracle, as it is, on ops in encode order, passing over the workload
    again until the time budget is spent (at least one op); returns the
    baseline record."""
    import oracle
    import synth
    done_bytes, t_used, ops_done = 0, 0.0, 0
    while t_used < budget_s:
        for op, w, x in data:
            t0 = time.perf_counter()
            oracle.gemv(w, x, op.n, op.p)
            t_used += time.perf_counter() - t0
            done_bytes += synth.workload_bytes([op])
            ops_done += 1
            if t_used >= budget_s:
                break
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d ops of the %d-op workload in encode order, %.2f passes (%.1f MB, %.1f s), "
                      "serial float64 C oracle, one host thread" % (
                          ops_done, len(data), ops_done / len(data), done_bytes / 1e6, t_used)}


def cpu_baseline_threaded(data, budget_s: float, threads: int):
    """The same serial oracle, unchanged, on contiguous row ranges of each op
    run by `threads` host threads at once (the C call releases the
    interpreter lock), passing over the workload until the budget is spent."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import synth
    done_bytes, t_used, ops_done = 0, 0.0, 0
    with ThreadPoolExecutor(max_workers=threads) as pool:
        while t_used < budget_s:
            for op, w, x in data:
                rb = synth.row_bytes(op.n)
                cuts = [op.p * k // threads for k in range(threads + 1)]
                parts = [(cuts[k], cuts[k + 1]) for k in range(threads) if cuts[k + 1] > cuts[k]]
                wf = w.reshape(-1)
                t0 = time.perf_counter()
                list(pool.map(lambda r: oracle.gemv(wf[r[0] * rb:r[1] * rb], x, op.n, r[1] - r[0]),
                              parts))
                t_used += time.perf_counter() - t0
                done_bytes += synth.workload_bytes([op])
                ops_done += 1
                if t_used >= budget_s:
                    break
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d ops of the %d-op workload in encode order, %.2f passes (%.1f MB, %.1f s), "
                      "serial float64 C oracle on contiguous row ranges, %d host threads" % (
                          ops_done, len(data), ops_done / len(data), done_bytes / 1e6, t_used,
                          threads)}


def bench_smallm(args, q8, synth, torch, np):
    """Small-batch products at the 7B shapes.  Each case cycles through enough
    distinct copies of W (>= 1 GiB in all) that no copy is still cached when it
    comes round again.  m <= 3 runs on the vector units (one conversion and m
    multiply-adds per weight, one lane-instruction each); larger m on bfloat16
    matrix cores with x split into three exact parts and the batch padded to
    16 rows: 3 * 16 * n * p multiply-adds.  Reported against max(HBM time,
    the path's compute time)."""
    MFMA_BF16_FLOPS = 2.5e15                # MI355X dense bf16
    VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9    # CUs x SIMDs x lanes x clock (no packed FP32)
    stream = torch.cuda.current_stream()
    cases = []
    kernel_arg = getattr(q8, "SMALLM_" + args.smallm_kernel) if args.smallm_kernel else None
    kernel_id = q8.SMALLM_AUTO if kernel_arg is None else kernel_arg
    only = {tuple(c.split(":")) for c in args.smallm_cases.split(",") if c}
    want = lambda shape, m: not only or (shape.name, str(m)) in only
    for shape in synth.SMALLM_SHAPES:
        if not any(want(shape, m) for m in synth.SMALLM_M):
            continue
        w, _ = synth.generate_smallm(shape, 2)
        wbytes = w.size
        copies = max(1, -(-(1 << 30) // wbytes))
        say("smallm %s: %d copies of %.1f MB" % (shape.name, copies, wbytes / 1e6))
        wd = [torch.from_numpy(w.reshape(shape.p, -1)).to("cuda") for _ in range(copies)]
        for m in synth.SMALLM_M:
            if not want(shape, m):
                continue
            _, X = synth.generate_smallm(shape, m)
            Xd = torch.from_numpy(X).to("cuda")
            Y = torch.empty((m, shape.p), dtype=torch.float32, device="cuda")
            # the caller-owned workspace, allocated once per case
            ws = torch.empty(max(1, q8.gemm_smallm_workspace(m, shape.n, shape.p, kernel_id)), dtype=torch.uint8,
                             device="cuda")
            if not cases:   # the first case: settle the GPU before anything is timed
                ring = iter(range(1 << 62))
                settle(lambda: q8.gemm_smallm(Xd, wd[next(ring) % copies], Y, stream, workspace=ws, kernel=kernel_arg),
                       torch.cuda.synchronize)
            for i in range(copies):
                q8.gemm_smallm(Xd, wd[i], Y, stream, workspace=ws, kernel=kernel_arg)
            k = max(copies * 4, 20)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(k):
                q8.gemm_smallm(Xd, wd[i % copies], Y, stream, workspace=ws, kernel=kernel_arg)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / k
            nbytes = synth.workload_bytes([shape], m)
            t_hbm = nbytes / 8e12
            chosen = q8.gemm_smallm_choice(m, shape.n, shape.p) if kernel_arg is None else kernel_arg
            if chosen == q8.SMALLM_VROW:
                kernel, unit = "k_q8_gemm_vrow<%d,2>" % m, "alu"
                t_cmp = (1 + m) * shape.n * shape.p / VALU_LANE_OPS
            elif chosen == q8.SMALLM_KS:
                kernel, unit = "k_q8_gemm_ks<8> (+ k_ks_reduce)", "mfma"
                t_cmp = 2 * 3 * 16 * shape.n * shape.p / MFMA_BF16_FLOPS
            else:
                kernel, unit = "k_split_x + k_q8_gemm_mfma<1>", "mfma"
                t_cmp = 2 * 3 * 16 * shape.n * shape.p / MFMA_BF16_FLOPS
            cases.append({"shape": shape.name, "n": shape.n, "p": shape.p, "m": m,
                          "kernel": kernel,
                          "us": round(t * 1e6, 2), "GB_s": round(nbytes / t / 1e9, 1),
                          "bound": "hbm" if t_hbm >= t_cmp else unit,
                          "frac_of_roof": round(max(t_hbm, t_cmp) / t, 4)})
            say("smallm %s m=%d: %.1f us, %.0f GB/s, %.1f%% of the %s roof" % (
                shape.name, m, t * 1e6, nbytes / t / 1e9, 100 * max(t_hbm, t_cmp) / t,
                cases[-1]["bound"]))
        del wd
        torch.cuda.empty_cache()
    return {"metric": "q8_0_gemm_smallm at 7B shapes", "unit": "us", "n_gpus": 1,
            "dtype": "f32", "data": "synthetic",
            "roof_note": "HBM 8 TB/s; vector units: FP32 lanes 39.3e12 instr/s (1 + m per weight); "
                         "matrix cores: bf16 MFMA 2.5 PFLOP/s dense (3 exact x parts, 16 padded rows)",
            "cases": cases}


def single_cold(op, nbytes, q8, torch, stream, time_steps):
    """Per-launch time of a one-op workload with W not in any cache: launches
    rotate through distinct copies of W (>= 2 x 256 MiB together), each copy
    once per pass, as direct launches and as a per-op chain (one launch per
    copy) replayed from one hipGraph."""
    x, w, _ = op
    copies = max(2, -(-(512 << 20) // w.numel()))
    ws = [w.clone() for _ in range(copies)]
    ys = [torch.empty(w.shape[0], dtype=torch.float32, device="cuda") for _ in range(copies)]
    for i in range(copies):
        q8.gemv(x, ws[i], ys[i], stream)
    passes = 3
    eager_s = time_steps(lambda: [q8.gemv(x, ws[i], ys[i], stream) for i in range(copies)],
                         passes) / passes / copies
    chain = q8.Chain([(x, ws[i], ys[i]) for i in range(copies)], fuse=False)
    chain.run(q8.MODE_GRAPH, stream)
    graph_s = time_steps(lambda: chain.run(q8.MODE_GRAPH, stream), passes) / passes / copies
    chain.close()
    return {"copies": copies, "distinct_weight_bytes": copies * w.numel(),
            "per_launch_eager_us": round(eager_s * 1e6, 2),
            "per_launch_graph_us": round(graph_s * 1e6, 2),
            "GB_s_graph": round(nbytes / graph_s / 1e9, 1)}


def bench_step(args, q8, synth, torch, np):
    """A whole decode token of a Qwen3-style model (embedding, per layer the
    norms, projections, rotary embedding, cache append, attention, SwiGLU and
    residual adds, then the final norm, the lm_head and argmax) replayed from
    its recorded hipGraph, greedy: each token feeds the next on the device.
    Timed from two starting positions (a short and a 511-token context).
    Also reports the matvec weight bytes a token streams, per second."""
    cfg, w = synth.step_model(args.step_model)
    wbytes = sum(synth.row_bytes(n) * p for _, n, p in synth.step_proj_shapes(cfg)) * cfg["n_layers"]
    wbytes += synth.row_bytes(cfg["hidden"]) * cfg["vocab"]
    cfg["max_seq"] = args.step_max_seq
    shapes = dict((nm, (p, n)) for nm, n, p in synth.step_proj_shapes(cfg))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    layers = [{k: (dev(a.reshape(shapes[k][0], -1)) if k in shapes else dev(a)) for k, a in L.items()}
              for L in w["layers"]]
    wd = {"embed": dev(w["embed"]), "out_norm": dev(w["out_norm"]),
          "lm_head": dev(w["lm_head"].reshape(cfg["vocab"], -1)), "layers": layers}
    del w
    torch.cuda.synchronize()
    st = q8.Step(cfg, wd)
    stream = torch.cuda.current_stream()
    launches = st.launches
    say("step: %d launches per token, %.2f GB resident" % (launches, torch.cuda.memory_allocated() / 1e9))

    def timed(mode, k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            st.run(mode, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / k

    # settle the GPU with untimed tokens (32 at a time from position 0)
    count = iter(range(1 << 62))

    def settle_token():
        if next(count) % 32 == 0:
            st.reset(0, 1, stream)
        st.run(q8.MODE_GRAPH, stream)
    settle(settle_token, torch.cuda.synchronize)

    cases = []
    for pos0 in (0, 511):
        rec = {"start_pos": pos0, "tokens": args.steps}
        for mode, name in ((q8.MODE_GRAPH, "graph"), (q8.MODE_EAGER, "eager")):
            st.reset(pos0, 1, stream)
            for _ in range(args.warmup):
                st.run(mode, stream)
            st.reset(pos0, 1, stream)
            t = timed(mode, args.steps)
            rec[name + "_us_per_token"] = round(t * 1e6, 2)
            rec[name + "_tokens_per_s"] = round(1.0 / t, 1)
            rec[name + "_weight_GB_per_s"] = round(wbytes / t / 1e9, 1)
            say("step from pos %d, %s: %.1f us/token, %.0f tokens/s" % (pos0, name, t * 1e6, 1.0 / t))
        cases.append(rec)
    st.close()
    short = cases[0]
    return {"metric": "%s-shaped greedy decode step (whole token, one hipGraph)" % args.step_model,
            "value": short["graph_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(short["graph_us_per_token"] / 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "%s decode step" % args.step_model, "launches_per_token": launches,
                       "weight_bytes_per_token": wbytes,
                       "max_seq": cfg["max_seq"],
                       "weights": "the %s chain's projection bytes; f32 embedding N(0,1), "
                                  "norm gains U[0.5,1.5]" % args.step_model},
            "cases": cases}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="7b_chain")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the per-op / eager / sync-each comparison")
    ap.add_argument("--smallm", action="store_true",
                    help="instead of the chain: time q8_0_gemm_smallm at the 7B shapes, "
                         "m in {2,4,8,16}, rotating weight copies past the 256 MB cache")
    ap.add_argument("--smallm-kernel", default="", metavar="NAME",
                    help="with --smallm: run this kernel (VALU, MFMA, VROW, VROW1, KS) instead of the library's choice")
    ap.add_argument("--smallm-cases", default="", metavar="SHAPE:M,...",
                    help="with --smallm: only these cases (e.g. down:2,lm_head:16), in the bench's order")
    ap.add_argument("--xq", action="store_true",
                    help="the chain's ops quantize x to Q8_0 and multiply integers "
                         "(q8_0_gemv_q8q8 semantics) instead of multiplying float x")
    ap.add_argument("--step", action="store_true",
                    help="instead of the chain: time a whole Qwen3-0.6B-shaped decode token "
                         "(every kernel of the step, one hipGraph) from positions 0 and 511")
    ap.add_argument("--step-max-seq", type=int, default=2048)
    ap.add_argument("--step-model", default="qwen3_0.6b", choices=("qwen3_0.6b", "7b"))
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the bench: copy MIB MiB device-to-device 5 times "
                         "(the known-size kernel that scales the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the matvec chain runs on a single "
              "MI355X (rows shard across GPUs without exchange, but no multi-GPU "
              "path is built here); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import q8_block_quantized_gemv_amd as q8
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": nb, "launches": 5}), flush=True)
        return
    if args.smallm:
        print(json.dumps(bench_smallm(args, q8, synth, torch, np)), flush=True)
        return
    if args.step:
        print(json.dumps(bench_step(args, q8, synth, torch, np)), flush=True)
        return
    ops_shape = synth.WORKLOADS[args.workload]
    nbytes = synth.workload_bytes(ops_shape)

    say("generating %s (%d ops, %.3f GB per token)" % (args.workload, len(ops_shape), nbytes / 1e9))
    t0 = time.time()
    data = synth.generate(args.workload)
    say("generated in %.1f s; uploading" % (time.time() - t0))
    dev_ops = []
    for op, w, x in data:
        dev_ops.append((torch.from_numpy(x).to("cuda"),
                        torch.from_numpy(w.reshape(op.p, -1)).to("cuda"),
                        torch.empty(op.p, dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    say("resident in HBM: %.2f GB" % (torch.cuda.memory_allocated() / 1e9))

    chain = q8.Chain(dev_ops, fuse=True, xq=args.xq)
    stream = torch.cuda.current_stream()

    def time_steps(run, k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3  # seconds

    run_graph = lambda: chain.run(q8.MODE_GRAPH, stream)
    cold = time_steps(run_graph, 1)
    settle_runs = settle(run_graph, torch.cuda.synchronize)
    for _ in range(args.warmup):
        run_graph()
    torch.cuda.synchronize()
    say("warm; timing %d steps" % args.steps)

    # the timed region: K graph-mode tokens (one launch, or one graph replay)
    # between a synchronize on each side
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    sec = time_steps(run_graph, args.steps)
    t_wall = time.perf_counter() - t_wall0
    per_step = sec / args.steps
    value = nbytes * args.steps / sec / 1e9
    say("fused graph: %.1f us/token, %.1f GB/s (%.1f%% of 8 TB/s); wall %.3f s" % (
        per_step * 1e6, value, 100 * value / HBM_PEAK_GBS, t_wall))

    # per-launch view of the dominant kernel: the fused chain is one kernel.
    # K launches of it issued directly (no graph around them), back to back on
    # the launch stream between one pair of events: the average is that
    # kernel's duration plus the dispatch gap between consecutive launches.
    launches = chain.launches
    kernel_s = time_steps(lambda: chain.run(q8.MODE_EAGER, stream), args.steps) / args.steps / launches
    achieved = nbytes / launches / kernel_s / 1e9
    # The kernel, named from the library's own plan of this chain
    # (q8_0_chain_plan): a chain of one op is that op's standalone launch
    # (its latency plan); more independent ops share one fused launch, of
    # the rows-and-group-slots tile where every width is whole groups, else
    # of the mixed-width kernel.  Template arguments: lanes per row, waves
    # per workgroup, weight stages in LDS, build mode (0 float activations,
    # 1 activations quantized to Q8_0).
    mode = 1 if args.xq else 0
    plan, _, _ = q8.chain_plan([(x.data_ptr(), w.data_ptr(), y.data_ptr(), o.n, o.p)
                                for (x, w, y), o in zip(dev_ops, ops_shape)],
                               q8.Q8_CHAIN_XQ if args.xq else 0,
                               torch.cuda.get_device_properties(0).multi_processor_count)
    lp = plan[0]
    if len(ops_shape) == 1:
        kernel = "k_q8_gemv_rc<%d,%d,%d,%d> (the op's latency plan)" % (
            lp["lanes_per_row"], lp["waves"], lp["stages"], mode)
    elif lp["kind"] == 2:
        kernel = "k_q8_gemv_rc_fused<%d,%d,%d,%d>" % (lp["lanes_per_row"], lp["waves"], lp["stages"], mode)
    else:
        kernel = "k_q8_gemv_mixed<%d>" % mode
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(args.workload, kernel),
                "kernel": kernel,
                "launches_per_step": launches,
                "algorithmic_bytes_per_launch": nbytes // launches,
                "kernel_us": round(kernel_s * 1e6, 2),
                "timing": "%d back-to-back launches between HIP events on the launch stream" % args.steps}

    modes = {"fused_graph_us": round(per_step * 1e6, 2), "fused_graph_cold_first_us": round(cold * 1e6, 2),
             "settle": {"seconds": SETTLE_S, "untimed_replays": settle_runs}}
    # spread: R more regions of graph replays after the timed one
    reps = sorted(time_steps(run_graph, 20) / 20 * 1e6 for _ in range(5))
    modes["fused_graph_repeats_us"] = {"regions": 5, "steps_each": 20, "min": round(reps[0], 2),
                                       "median": round(reps[2], 2), "max": round(reps[-1], 2)}
    if not args.no_modes:
        k = max(3, args.steps // 10)
        modes["fused_eager_us"] = round(time_steps(lambda: chain.run(q8.MODE_EAGER, stream), k) / k * 1e6, 2)
        per_op = q8.Chain(dev_ops, fuse=False, xq=args.xq)
        for m, name in ((q8.MODE_GRAPH, "per_op_graph_us"), (q8.MODE_EAGER, "per_op_eager_us"),
                        (q8.MODE_SYNC_EACH, "per_op_sync_each_us")):
            per_op.run(m, stream)
            torch.cuda.synchronize()
            modes[name] = round(time_steps(lambda: per_op.run(m, stream), k) / k * 1e6, 2)
            say("%s: %.1f us/token" % (name, modes[name]))
        per_op.close()

    if 1 < len(ops_shape) and nbytes < (4 << 30):
        # a chain of a few hundred MB against the 256 MB Infinity Cache: a
        # second copy of every weight, the two chains replayed in turn, shows
        # whether any part of a token is served from the cache when it repeats
        twin = q8.Chain([(x, w.clone(), y) for x, w, y in dev_ops], fuse=True, xq=args.xq)
        twin.run(q8.MODE_GRAPH, stream)
        k = max(10, args.steps // 2)

        def alternate():
            chain.run(q8.MODE_GRAPH, stream)
            twin.run(q8.MODE_GRAPH, stream)
        alt_us = time_steps(alternate, k) / (2 * k) * 1e6
        one_us = time_steps(run_graph, 2 * k) / (2 * k) * 1e6
        modes["two_weight_sets"] = {"alternating_us": round(alt_us, 2), "one_set_us": round(one_us, 2),
                                    "tokens_each": 2 * k}
        twin.close()
        say("two weight sets in turn: %.1f us/token, one set: %.1f" % (alt_us, one_us))

    if len(ops_shape) == 1:
        # one op of a few MB stays in the 256 MB Infinity Cache when it repeats:
        # the figures above are hot-cache.  Cold: the same op on distinct copies
        # of W (>= 2 x 256 MiB in all), each copy used once per pass.
        modes["cold_rotation"] = single_cold(dev_ops[0], nbytes, q8, torch, stream, time_steps)
        say("cold rotation: %s" % json.dumps(modes["cold_rotation"]))

    base = base_mt = None
    if not args.no_cpu_baseline:
        say("timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        base = cpu_baseline(data, args.cpu_budget)
        # the host's cores, at most the 16 a one-GPU share of the machine has
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        say("timing the CPU oracle on %d threads (budget %.0f s)" % (threads, args.cpu_budget / 2))
        base_mt = cpu_baseline_threaded(data, args.cpu_budget / 2, threads)

    out = {
        "metric": "Q8_0 GEMV achieved HBM GB/s (% of 8 TB/s); decode-chain matvec us/token",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(per_step * 1e3, 5),
        "us_per_token": round(per_step * 1e6, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8xi8->f32" if args.xq else "f32", "data": "synthetic",
        "config": {"workload": args.workload, "ops_per_token": len(ops_shape),
                   "bytes_per_token": nbytes,
                   "mode": "q8_0_decode_chain in graph mode, %d launch(es) per token (%s)" % (
                       chain.launches, "issued directly" if chain.launches == 1 else "one hipGraph replay"),
                   "activations_as": "Q8_0, integer dots" if args.xq else "float32",
                   "weights": "Q8_0, scale U[0.001,0.02] as f16, quants U{-127..127}",
                   "activations": "f32 N(0,1), independent per op",
                   "cache": ("hot: one %.1f MB copy of W, resident in the 256 MB Infinity Cache "
                             "(cold figures: modes_us_per_token.cold_rotation)" % (nbytes / 1e6)
                             if nbytes < (256 << 20) else
                             "partly warm: %.0f MB of weights per step against the 256 MB Infinity "
                             "Cache, part of which is still cached when the step repeats (two "
                             "weight sets in turn: modes_us_per_token.two_weight_sets)" % (nbytes / 1e6)
                             if nbytes < (4 << 30) else
                             "cold: %.0f MB of weights per step, far past the 256 MB Infinity Cache"
                             % (nbytes / 1e6))},
        "roofline": roofline,
        "modes_us_per_token": modes,
        "cpu_baseline": base,
        "cpu_baseline_all_cores": base_mt,
    }
    print(json.dumps(out), flush=True)
    chain.close()


if __name__ == "__main__":
    main()
