"""Sanitizer build of the C ABI's host code for the CPU tests: every translation unit of
the library compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host side
only (the device code is built as usual), linked with the host driver
tests/abi_asan_driver.cpp into one executable under _build/asan/.  Objects are rebuilt
only when their sources changed."""
from __future__ import annotations

import glob
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a16_mixed_precision_offline_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HIP_FLAGS = ["-O1", "-g", "--offload-arch=gfx950", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def available() -> bool:
    return os.path.exists(HIPCC) and os.path.exists(CLANGXX)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    deps = [src, os.path.join(CSRC, "internal.h"), os.path.join(ROOT, "include", "w4a16.h")]
    if os.path.exists(obj) and os.path.getmtime(obj) >= max(os.path.getmtime(d) for d in deps):
        return obj  # up to date
    # host code instrumented (argument validation, plans, workspace bookkeeping); each
    # -fsanitize= applies to the host pass only, the device code is built as usual
    _run([HIPCC, *HIP_FLAGS, "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-c", src, "-o", obj])
    return obj


def build() -> str:
    """Returns the path of the sanitized driver executable."""
    import concurrent.futures as cf
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    exe = os.path.join(OUT, "abi_asan")
    _run([CLANGXX, "-g", "-fsanitize=address,undefined", "-std=c++17",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_asan_driver.cpp"),
          *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe
