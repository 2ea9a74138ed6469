"""Build the HIP library in-tree: q8_block_quantized_gemv_amd/libq8gemv.so.

gfx950 only; packed FP32 instructions are switched off in device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq8gemv.so")
SOURCES = [os.path.join(CSRC, f)
           for f in ("q8_gemv.hip", "q8_gemm.hip", "q8_step.hip", "q8_api.hip", "q8_step_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_command(out: str, extra=()):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Werror", "-Wno-unused-command-line-argument", "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra, *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature name; that is harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
