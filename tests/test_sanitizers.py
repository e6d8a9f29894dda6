"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds (no GPU needed).

* The fp64 oracle (oracle/ssd_oracle.c): every function on small shapes with
  exact-size buffers (tests/sanitize/oracle_main.c), OpenMP on.
* libssd's C ABI layer: every entry point's argument checks, built with the
  sanitizers on the host code only (the device code is compiled as usual);
  every call has an invalid argument, so none reaches a HIP call
  (tests/sanitize/abi_main.c).

A finding stops the program with a non-zero status and the sanitizer's report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "state_space_sequence_ssd_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
# host-only sanitizer flags for hipcc: each -fsanitize applies to the host pass alone
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-fopenmp", os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_main.c"),
         "-lm", "-o", exe])
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4"))
    assert "ok: 0 failure(s)" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_checks_under_asan_ubsan(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
             os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    run([HIPCC, *HOST_SAN, "-I", os.path.join(ROOT, "include"), "-x", "c",
         os.path.join(ROOT, "tests", "sanitize", "abi_main.c"), "-x", "none", *objs, "-o", exe])
    # the HIP runtime's own allocations at exit are not this library's
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "ok: 0 failure(s)" in r.stdout
