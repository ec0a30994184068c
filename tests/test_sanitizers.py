"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The fp64 oracle (oracle/nsa_oracle.c), built with gcc and both sanitizers,
  run by tests/sanitize/oracle_driver.c over every entry point on small inputs
  with padding, future, out-of-range and repeated entries, empty rows, M != N
  and ragged blocks.
- The host side of the C-ABI library (argument checks, aliasing checks,
  workspace planning, status strings), built from the library's HIP sources
  with the sanitizers on the host half only (the device half is compiled but
  never run), driven by tests/sanitize/host_checks.cpp through calls that every
  check must reject before any HIP call.
"""

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_attention_sel_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer"]


def _run(exe, tmp):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, cwd=tmp, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_driver")
        cmd = ["gcc", "-std=c11", *SAN_FLAGS, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-pthread", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
               os.path.join(ROOT, "oracle", "nsa_oracle.c"), "-lm"]
        subprocess.run(cmd, check=True, capture_output=True)
        assert "oracle sanitizer driver: ok" in _run(exe, tmp)


def test_library_host_checks_under_asan_and_ubsan():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    # Sanitizers on the host half only: each -fsanitize= behind -Xarch_host.
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["--offload-arch=gfx950", "-std=c++17", *SAN_FLAGS, *host_san, "-I", hip_build.INCLUDE,
              "-I", hip_build.CSRC]
    srcs = [os.path.join(SAN, "host_checks.cpp"), hip_build.SRC, hip_build.BWD_SRC, hip_build.DENSE_SRC,
            hip_build.TOPK_SRC]
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            subprocess.run([hipcc, *common, "-x", "hip", "-c", "-o", obj, src], check=True, capture_output=True)
            return obj
        with ThreadPoolExecutor(len(srcs)) as ex:
            objs = list(ex.map(compile_one, srcs))
        exe = os.path.join(tmp, "host_checks")
        subprocess.run([hipcc, "--offload-arch=gfx950", *host_san, "-o", exe, *objs], check=True,
                       capture_output=True)
        assert "host checks: ok" in _run(exe, tmp)
