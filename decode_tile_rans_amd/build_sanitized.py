"""Host-only build of the library's CPU code with AddressSanitizer and UBSan.

Compiles the encoder, model, blob and planning units (everything the C ABI runs on the
host, including the parser of untrusted blob bytes) with g++ ``-fsanitize=address,
undefined`` into one shared library that exports the host entry points only (no HIP
units; blobs cannot be uploaded).  Python loads it through ``EP_LIB_PATH`` with the
ASan runtime preloaded; ``runtime_env()`` gives that environment.

    python -m decode_tile_rans_amd.build_sanitized [out.so]
"""
from __future__ import annotations

import os
import subprocess
import sys

from decode_tile_rans_amd.build import CSRC, HOST_SRCS, ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build(out: str) -> str:
    """Compile and link the sanitized host library at `out`; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in HOST_SRCS + ["host_only.cpp"]]
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-pthread", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs,
           "-Wl,--no-undefined", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    return out


def asan_runtime() -> str | None:
    """Path of g++'s ASan runtime, or None when the toolchain has none."""
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def runtime_env(lib_path: str) -> dict:
    """Environment for a Python process that loads the sanitized library: the ASan
    runtime preloaded (Python itself is not instrumented, so leak reports are off),
    any sanitizer finding fatal."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime() or ""
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["EP_LIB_PATH"] = lib_path
    return env


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "libentropack_host_san.so")))
