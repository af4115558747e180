"""Build libsq.so (the HIP kernels + C ABI) in-tree for gfx950, and beside
it libsq_ceiling.so, the measured-ceiling probes (measure/).

Every source under csrc/ is compiled with hipcc for gfx950 only, in parallel,
then linked into w8a8_post_quantization_channel_amd/libsq.so; the sources
under measure/ are linked into libsq_ceiling.so. Flags:
  -ffp-contract=off   no fused multiply-add: the quantization paths need one
                      IEEE rounding per fp32 operation
  -packed-fp32-ops off (device feature) keep the compiler from emitting packed
                      fp32 arithmetic
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
MEASURE = os.path.join(PKG, "measure")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsq.so")
CEILING_LIB = os.path.join(PKG, "libsq_ceiling.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def measure_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(MEASURE, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libsq.so and every measure/*.hip into
    libsq_ceiling.so; returns libsq's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs, msrcs = sources(), measure_sources()
    jobs = jobs or min(len(srcs) + len(msrcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs + msrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


def stale() -> bool:
    """True when a library is missing or older than a source or header."""
    if not os.path.exists(LIB) or not os.path.exists(CEILING_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(CEILING_LIB))
    deps = sources() + measure_sources() + glob.glob(os.path.join(CSRC, "*.h")) + \
        glob.glob(os.path.join(INCLUDE, "*.h"))
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
