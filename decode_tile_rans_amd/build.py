"""Build libentropack_hip.so in-tree (gfx950).

Host C++ (encoder, model, blob code) is compiled with g++ and -ffp-contract=off
(the encoder's float64 arithmetic must not be contracted into FMAs); the HIP
units with hipcc for gfx950.  Run ``python -m decode_tile_rans_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libentropack_hip.so")
BUILD = os.path.join(ROOT, "_build")

HOST_SRCS = ["model.cpp", "encoder.cpp", "blob.cpp", "plan.cpp"]
HIP_SRCS = ["decode.hip", "gemm.hip", "encode_gpu.hip"]
ARCH = os.environ.get("EP_OFFLOAD_ARCH", "gfx950")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + os.path.basename(cmd[-1]))
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    procs = []
    for s in HOST_SRCS:
        o = os.path.join(BUILD, s + ".o")
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-pthread",
               "-Wall", "-Wno-unused-function", *inc, "-c", os.path.join(CSRC, s), "-o", o]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(o)
    for s in HIP_SRCS:
        o = os.path.join(BUILD, s + ".o")
        cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
               *inc, "-c", os.path.join(CSRC, s), "-o", o]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(o)
    for cmd, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + out + err)
            raise RuntimeError("build step failed: " + os.path.basename(cmd[-3]))
        if verbose and err.strip():
            errs = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            if errs:
                sys.stderr.write("\n".join(errs) + "\n")
    tmp = OUT + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
