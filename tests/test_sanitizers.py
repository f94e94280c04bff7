"""Host code under sanitizers, on the CPU: the oracle and the layout planner under
AddressSanitizer + UndefinedBehaviorSanitizer, the offloaded host update under
the same and under ThreadSanitizer (its thread pool).  Each driver in
tests/sanitize/ is built with the host compiler and run; any sanitizer report
fails the test.  (GPU code is not built here: these are host-only builds.)"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sharded_optimizer_step_zero_amd", "csrc")
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:",
           "WARNING: ThreadSanitizer")
ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

CASES = {
    "oracle": ("gcc", ["-std=c99", "-fopenmp", "-ffp-contract=off", *ASAN_UBSAN],
               [os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "zo.c")],
               ["-lm"], "oracle check ok"),
    "planner": ("g++", ["-std=c++17", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", *ASAN_UBSAN],
                [os.path.join(SAN, "plan_check.cpp"), os.path.join(CSRC, "plan.cpp")], [],
                "plan check ok"),
    "host_step": ("g++", ["-std=c++17", "-pthread", "-ffp-contract=off", "-fno-math-errno",
                          *ASAN_UBSAN],
                  [os.path.join(SAN, "host_step_check.cpp"), os.path.join(CSRC, "host_step.cpp")],
                  [], "host step check ok"),
    "host_step_threads": ("g++", ["-std=c++17", "-pthread", "-ffp-contract=off",
                                  "-fno-math-errno", "-fsanitize=thread", "-DZS_HOST_ONE_ISA"],
                          [os.path.join(SAN, "host_step_check.cpp"),
                           os.path.join(CSRC, "host_step.cpp")], [], "host step check ok"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_under_sanitizer(name):
    cc, flags, sources, libs, ok = CASES[name]
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, name)
        cmd = [cc, "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra", *flags, *sources,
               "-o", exe, *libs]
        subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", TSAN_OPTIONS="halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert not any(s in out for s in REPORTS), out[-4000:]
    assert ok in r.stdout
