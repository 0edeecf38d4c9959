"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

  * the oracle (oracle/any4_oracle.c) with a driver that runs every variant on ragged,
    minimal and non-finite inputs, with and without traces, and its invalid arguments;
  * the C-ABI layer (weight_only_bit_row_amd/csrc/any4_api.cpp), built with g++ against
    host stand-ins for the kernel launchers, driven through every entry point's valid
    and invalid arguments, mixed-geometry batches with restarts, and the entry point
    that allocates nothing.

Each build is plain gcc/g++ (no GPU code); a sanitizer report aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    if r.returncode != 0 and "LeakSanitizer has encountered a fatal error" in r.stderr:
        # leak checking needs ptrace, which some sandboxes forbid; the rest still runs
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                           env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-o", exe,
                    os.path.join(ROOT, "oracle", "any4_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm"],
                   check=True, capture_output=True, text=True)
    _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "weight_only_bit_row_amd", "csrc")
    r = subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"), "-I", csrc, *SAN, "-o", exe,
                        os.path.join(csrc, "any4_api.cpp"), os.path.join(HERE, "abi_stubs.cpp"),
                        os.path.join(HERE, "abi_driver.cpp")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    _run(exe)
