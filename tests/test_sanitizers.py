"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host half (csrc/api.cpp: validation, split planning, the integer
threshold, the draft cap, the indexer's host state) is built with g++ against
stand-ins for the kernel launchers (tests/sanitize/launch_stub.cpp) and driven
through every entry point with random and extreme sizes; the float64 oracle
(oracle/mla_oracle.c) is built with gcc and run on small problems, both
routes.  Any sanitizer report (the builds stop at the first one) or failed
check fails the test.  No HIP device code is involved.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("gcc/g++ not available")
    return tmp_path_factory.mktemp("san")


def test_api_host_code_is_clean(outdir):
    csrc = os.path.join(ROOT, "mla_speculative_decode_amd", "csrc")
    exe = str(outdir / "drive_api")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", csrc,
          "-I", os.path.join(ROOT, "include"),
          os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "drive_api.cpp"), "-o", exe])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"},
             timeout=300)
    assert "0 failed checks" in r.stdout


def test_oracle_is_clean(outdir):
    exe = str(outdir / "drive_oracle")
    _run(["gcc", "-std=c99", *SAN, os.path.join(ROOT, "oracle", "mla_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "drive_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"}, timeout=300)
    assert "0 disagreements" in r.stdout
