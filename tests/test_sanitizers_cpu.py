"""CPU: the host code under AddressSanitizer and UndefinedBehaviorSanitizer.

- The oracle (gcc, -fsanitize=address,undefined, every report fatal) runs all
  of its pins in a child process with gcc's ASan runtime preloaded; a copy
  with a planted out-of-bounds write must abort there, which shows the
  sanitizer is active.
- libsq's host code (hipcc, sanitizer flags for the host side only; the
  device code is built as usual) runs every argument-validation test of
  test_capi_cpu.py in a child process with clang's ASan runtime preloaded.
  Those calls are rejected before anything is launched, so no GPU is needed.

Builds go to a temporary directory; nothing here touches the regular builds.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "sq_oracle.c")
CSRC = os.path.join(ROOT, "w8a8_post_quantization_channel_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}

RUN_PINS = """
import sys
sys.path.insert(0, {root!r})
from oracle import oracle as om
from tests import oracle_pins
o = om.Oracle(lib=om.load(sys.argv[1]))
for pin in oracle_pins.PINS:
    pin(o)
    print("pin ok", pin.__name__, flush=True)
"""

RUN_CAPI = """
import inspect, sys
sys.path.insert(0, {root!r})
from w8a8_post_quantization_channel_amd import capi
lib = capi.load(sys.argv[1])
from tests import test_capi_cpu as T
for name, f in sorted(vars(T).items()):
    if name.startswith("test_") and callable(f) and set(inspect.signature(f).parameters) <= {{"lib"}}:
        f(lib) if "lib" in inspect.signature(f).parameters else f()
        print("capi ok", name, flush=True)
"""


def _gcc_asan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's ASan runtime not found")
    return path


def _build_oracle(src, out):
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, cwd=os.path.dirname(src), capture_output=True)


def _run(script, lib, preload, timeout):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    return subprocess.run([sys.executable, "-c", script.format(root=ROOT), lib], env=env, capture_output=True,
                          text=True, timeout=timeout)


def test_oracle_pins_under_sanitizers(tmp_path):
    from tests import oracle_pins
    asan = _gcc_asan()
    lib = str(tmp_path / "libsq_oracle_san.so")
    _build_oracle(ORACLE_SRC, lib)
    r = _run(RUN_PINS, lib, asan, 600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.count("pin ok") == len(oracle_pins.PINS)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    """The same harness on an oracle whose absmax writes one element past the
    end of its output: the run must stop with an AddressSanitizer report."""
    asan = _gcc_asan()
    src = open(ORACLE_SRC).read()
    bad = src.replace("        absmax[j] = mx;\n    }\n}", "        absmax[j + (j == k - 1)] = mx;\n    }\n}", 1)
    assert bad != src, "the planted mistake no longer applies to the oracle source"
    shutil.copy(os.path.join(ROOT, "oracle", "sq_oracle.h"), tmp_path / "sq_oracle.h")
    (tmp_path / "sq_oracle.c").write_text(bad)
    lib = str(tmp_path / "libsq_oracle_bad.so")
    _build_oracle(str(tmp_path / "sq_oracle.c"), lib)
    r = _run(RUN_PINS, lib, asan, 600)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr


def test_capi_validation_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    runtimes = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtimes:
        pytest.skip("clang's ASan runtime not found")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", INCLUDE, "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libsq_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = _run(RUN_CAPI, lib, runtimes[-1], 600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.count("capi ok") >= 15
    assert "runtime error" not in r.stderr
