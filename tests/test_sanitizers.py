"""AddressSanitizer and UndefinedBehaviorSanitizer builds (CPU only).

- The oracle (oracle/nf4ref.c) is built with gcc and both sanitizers and
  run over every function on small and edge-case inputs
  (tests/sanitize/oracle_run.c).
- The library's host code (every csrc/*.hip, sanitizers on the host side
  only: each -fsanitize= follows -Xarch_host, the device code is built as
  usual) is linked with tests/sanitize/host_validation.cpp, which drives
  every entry point's argument validation, the size and workspace
  functions and the code-table builder. No call reaches a HIP launch.

Any report makes the program exit non-zero (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "nf4_quantize_amd", "csrc")
INC = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return r.returncode, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_run")
    rc, out = run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
                   os.path.join(ROOT, "oracle", "nf4ref.c"), os.path.join(SAN, "oracle_run.c"),
                   "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = run([exe], env=ENV, timeout=300)
    assert rc == 0 and "ok" in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_validation_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fhip-fp32-correctly-rounded-divide-sqrt", *HOST_SAN, *INC]
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = run([HIPCC, *flags, "-c", src, "-o", obj])
        assert rc == 0, out
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "host_validation.o")
    rc, out = run([HIPCC, "--offload-host-only", "-x", "hip", "-O1", "-g", "-std=c++17", *HOST_SAN,
                   *INC, "-c", os.path.join(SAN, "host_validation.cpp"), "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "host_validation")
    rc, out = run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fsanitize=undefined", "-o", exe, *objs, drv])
    assert rc == 0, out
    rc, out = run([exe], env=ENV, timeout=300)
    assert rc == 0 and "ok" in out, out
