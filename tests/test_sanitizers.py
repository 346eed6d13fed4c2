"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- The fp64 oracle (oracle/ssm_oracle.c), every function on tiny shapes
  (tests/oracle_san_check.c), built with gcc.
- The C ABI's host side -- size queries, workspace planning and argument
  validation -- on tiny and full-size shapes (tests/abi_san_check.cpp),
  linked against the library's sources built with the sanitizers on the host
  side only (device code is built as usual and never launched: every call the
  driver makes is rejected by validation).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    proc = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert proc.returncode == 0, f"{' '.join(cmd)}\n{proc.stdout[-4000:]}\n{proc.stderr[-4000:]}"
    return proc


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", "-o", exe, os.path.join(ROOT, "oracle", "ssm_oracle.c"),
          os.path.join(ROOT, "tests", "oracle_san_check.c"), "-lm"])
    out = _run([exe], env=ENV, timeout=300).stdout
    assert "oracle sanitizer run OK" in out


def test_abi_host_paths_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops"]
    csrc = os.path.join(ROOT, "adjoint_gradients_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    srcs.append(os.path.join(ROOT, "tests", "abi_san_check.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *common, *san, "-c", "-o", obj, src])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", *san, "-o", exe, *objs])
    out = _run([exe], env=ENV, timeout=300).stdout
    assert "ABI sanitizer run OK" in out
