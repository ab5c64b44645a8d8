"""Build libmla.so (HIP, gfx950) in-tree with hipcc.

    python -m mla_speculative_decode_amd.build

Compiles each translation unit under csrc/ to an object in parallel, then
links the shared library next to this file.  Always rebuilds.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
BENCH_LIB = os.path.join(HERE, "libmla_bench.so")   # timing loop used by bench.py only
SOURCES = ["attn.hip", "split_absorbed.hip", "gemm.hip", "quant.hip", "indexer.hip", "noalloc.hip", "api.cpp"]
ARCH = "gfx950"
# Per-file extra flags.  The absorbed split kernel takes maxima of scores that
# are never NaN, without the canonicalising moves IEEE NaN handling adds.
EXTRA: dict = {"split_absorbed.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
            # no packed-fp32 VALU instructions in any kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *flags(), *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # bench driver: links against libmla.so, found next to it at run time
    tmp = BENCH_LIB + ".tmp"
    r = subprocess.run([cc, *flags(), "-shared", "-o", tmp, os.path.join(CSRC, "bench_driver.cpp"),
                        "-x", "hip", os.path.join(CSRC, "bench_peaks.hip"),
                        "-L", HERE, "-lmla", "-Wl,-rpath,$ORIGIN"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"bench driver build failed:\n{r.stderr}")
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
