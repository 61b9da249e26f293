"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the C oracle (oracle/recurrence.c), forward and backward, in every gate,
  key and preconditioner mode, built with gcc's sanitizers and driven by
  tests/sanitize/oracle_driver.c;
* the argument validation and workspace sizing of libpdn.so, from a build of
  every library source with the sanitizers on the host side only (the device
  code is built as usual and never launched here), driven by
  tests/sanitize/api_driver.c: every mode, each field out of range, and sizes
  at and beyond the limits where the size arithmetic could overflow.

The sanitizers abort the process on a finding, so a zero exit status and an
empty sanitizer report are the pass condition.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_77_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    # OpenMP left out: the loops over (b, h) run serially, the arithmetic is the same
    _run(["gcc", "-O1", "-g", "-std=c99", "-fno-omit-frame-pointer", *SAN,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "recurrence.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=600)
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.timeout(900)
def test_api_validation_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("the ROCm toolchain is needed for the host-only library build")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "pdn_api.cpp")]
    host_san = []
    for f in SAN:                       # host side only: no sanitizer in device code
        host_san += ["-Xarch_host", f]
    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *host_san, "-c", src, "-o", obj])
        return obj
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(len(srcs), 4)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libpdn_san.so")
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", *host_san, *objs, "-o", lib])
    exe = str(tmp_path / "api_driver")
    _run([clang, "-O1", "-g", "-std=c11", *SAN, os.path.join(HERE, "api_driver.c"),
          "-I" + os.path.join(ROOT, "include"), lib, "-Wl,-rpath," + str(tmp_path),
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "argument sets" in r.stdout and " 0 inconsistent answers" in r.stdout, r.stdout
    # the random sets reach the accepting paths too, not only early rejections
    accepted = int(r.stdout.split(" random, ")[1].split(" of them accepted")[0])
    assert accepted > 100, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
