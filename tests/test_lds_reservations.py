"""The LDS reservations that cap resident workgroups per CU, checked on the host:
every table entry and every ZS_WAVES_PER_CU value fits a 64 KiB per-workgroup
limit with room for static LDS and meets its intended residency, the context's
init-time check refuses a reservation that does not fit, and the override
parser accepts exactly 0 and 3..64 (tests/native/lds_check.cpp on the library's
own header)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lds_reservations(tmp_path):
    exe = tmp_path / "lds_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror",
                    "-fsanitize=address,undefined", "-o", str(exe),
                    os.path.join(ROOT, "tests", "native", "lds_check.cpp")], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "lds check ok" in r.stdout
