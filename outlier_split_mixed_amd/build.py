"""Build libsqf.so (HIP for gfx950) in-tree.

    python -m outlier_split_mixed_amd.build

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 into ``_build/``
(in parallel), then linked into ``outlier_split_mixed_amd/libsqf.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsqf.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_bench(verbose)
    return LIB


BENCH_LIB = os.path.join(HERE, "libsqf_bench.so")


def build_bench(verbose: bool = False) -> str:
    """libsqf_bench.so: the matrix-unit rate micro-benchmark bench.py reports
    beside the spec peaks (measurement only; not part of the path's ABI)."""
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc_bench", "*.hip")))
    tmp = BENCH_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {srcs}:\n{r.stderr}")
    os.replace(tmp, BENCH_LIB)
    if verbose:
        print(f"built {BENCH_LIB}")
    return BENCH_LIB


SAN_LIB = os.path.join(BUILD, "libsqf_hostsan.so")
# host-side sanitizers only: each -fsanitize= follows -Xarch_host, so the
# device code is built exactly as in the product library
SAN_HOST_FLAGS = ["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address,undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_host_sanitized(verbose: bool = False) -> str:
    """libsqf with AddressSanitizer and UBSan in the C-ABI host code
    (sqf_api.hip: argument checks, workspace handling, launch set-up), linked
    with the kernels' objects of the last build(); written to _build/.  A
    process that loads it needs clang's ASan runtime preloaded."""
    api = os.path.join(CSRC, "sqf_api.hip")
    objs = sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))
    kern = [o for o in objs if os.path.basename(o) != "sqf_api.hip.o"]
    if len(kern) != len(glob.glob(os.path.join(CSRC, "*.hip"))) - 1:
        raise RuntimeError("build() first: the kernel objects are missing from _build/")
    obj = os.path.join(BUILD, "sqf_api.hostsan.o")
    cmd = [HIPCC, *FLAGS, *SAN_HOST_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", api, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {api}:\n{r.stderr}")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
           "-shared-libsan", obj, *kern, "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
