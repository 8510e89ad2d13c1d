"""The library's host code under AddressSanitizer and UBSan: the encoder, model, blob
parser and bit-rate planner are built into a host-only library with g++
-fsanitize=address,undefined, and the C-ABI CPU tests (byte parity with the oracle,
validation, the parser on corrupted bytes, the planner, CompressedLinear state loading)
run against it in a child process with the ASan runtime preloaded.  Any sanitizer
finding aborts the child, so the test passes only on a clean run."""
import os
import subprocess
import sys

import pytest

from decode_tile_rans_amd import build_sanitized as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    if bs.asan_runtime() is None:
        pytest.skip("g++ has no ASan runtime here")
    lib = bs.build(str(tmp_path / "libentropack_host_san.so"))
    env = bs.runtime_env(lib)
    # the child really runs the sanitized library: ASan is mapped and the loader took EP_LIB_PATH
    probe = ("import decode_tile_rans_amd._lib as L; L.lib(); "
             "m = open('/proc/self/maps').read(); assert 'libasan' in m and L.LIB_PATH in m; print('ok')")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-n", "4",
           "tests/test_capi_cpu.py", "tests/test_api_cpu.py", "-m", "not gpu",
           "-k", "not exports_every_declared_symbol"]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=1500)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
