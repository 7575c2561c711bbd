"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The decode library's launch-plan and workspace arithmetic (plan.h), built
   as plain host C++ into a harness that plans every supported shape against
   budgets up to the int32 limit and capacities up to 524288.
2. The C oracle, built with both sanitizers, running the whole oracle pin
   suite in a child process (the ASan runtime preloaded into the interpreter;
   leak detection off, since the interpreter itself is not instrumented).
Any sanitizer report aborts the child, which fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_long_fwht_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _gcc_file(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_plan_arithmetic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_harness")
    cmd = ["g++", "-std=c++17", "-O1", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "plan_harness.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout[-2000:], res.stderr[-4000:])
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "failures: 0" in res.stdout


def test_oracle_pins_under_sanitizers():
    asan = _gcc_file("libasan.so")
    if asan is None:
        pytest.skip("no libasan in this toolchain")
    sys.path.insert(0, ROOT)
    import oracle.build as ob
    lib = ob.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, ADAMAS_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = res.stdout[-3000:] + res.stderr[-3000:]
    print(tail)
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error:" not in res.stderr
