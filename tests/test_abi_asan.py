"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
every translation unit rebuilt with both sanitizers on its host side (tests/asan_build.py)
and driven by tests/abi_asan_driver.cpp through every query and the argument validation of
every entry point.  Any invalid access, overflow or undefined operation aborts the driver."""
import os
import subprocess

import pytest

import asan_build


@pytest.mark.skipif(not asan_build.available(), reason="hipcc / clang++ not installed")
def test_abi_host_code_is_clean_under_asan_and_ubsan():
    exe = asan_build.build()
    env = dict(os.environ)
    # leaks of the HIP runtime's own start-up are not the library's; everything else halts
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # host code only: never a device, even on a GPU machine
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-3000:], r.stderr[-3000:])


@pytest.mark.skipif(not asan_build.available(), reason="hipcc / clang++ not installed")
def test_the_sanitizer_build_catches_a_planted_overflow():
    exe = asan_build.build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe, "--planted-overflow"], capture_output=True, text=True, timeout=300,
                       env=env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout, r.stderr[-2000:])
