"""Build the HIP library in-tree: q8_block_quantized_gemv_amd/libq8gemv.so.

gfx950 only; packed FP32 instructions are switched off in device code.  Each
source (and each build mode of q8_gemv_rc.hip) compiles to an object of
its own, in parallel, under _build/; the objects are then linked.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq8gemv.so")
OBJ_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (source, extra flags, object name)
UNITS = [("q8_gemv.hip", (), "q8_gemv")] + \
        [("q8_gemv_rc.hip", ("-DQ8_RC_MODE=%d" % m,), "q8_gemv_rc_%d" % m) for m in range(7)] + \
        [("q8_gemm.hip", (), "q8_gemm"), ("q8_step.hip", (), "q8_step"),
         ("q8_api.hip", (), "q8_api"), ("q8_step_api.hip", (), "q8_step_api")]
SOURCES = sorted({os.path.join(CSRC, u[0]) for u in UNITS})

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Werror", "-Wno-unused-command-line-argument", "-Wno-inline-asm"]


def compile_command(src: str, out: str, extra=()):
    return [HIPCC, *COMMON, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
            "-c", os.path.join(CSRC, src), "-o", out]


def link_command(objs, out: str):
    return [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature name; that is harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or max(1, min(len(UNITS), os.cpu_count() or 1))
    tag = ".%d" % os.getpid()
    cmds = []
    objs = []
    for src, extra, name in UNITS:
        obj = os.path.join(OBJ_DIR, name + tag + ".o")
        objs.append(obj)
        cmds.append(compile_command(src, obj, extra))
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(_run, cmds))
        failed = [(c, e) for c, (rc, e) in zip(cmds, results) if rc != 0]
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(" ".join(c) + "\n" + e for c, e in failed))
        tmp = LIB + ".tmp%d" % os.getpid()
        rc, err = _run(link_command(objs, tmp))
        if rc != 0:
            raise RuntimeError("link failed:\n" + err)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
