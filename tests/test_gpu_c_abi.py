"""The C ABI from plain C with the HIP runtime alone (tests/c_abi/abi_check.c): no
Python binding and no torch in that process; bit-identical to the oracle, including
the allocation-free step captured into a HIP graph and replayed."""
import os
import subprocess

import pytest

from _gpu import log

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_check")


def test_plain_c_program_matches_oracle():
    log("test_plain_c_program_matches_oracle")
    assert os.path.exists(EXE), "build it with __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip() + r.stderr.strip())
    assert r.returncode == 0, r.stderr
    assert "c-abi check ok" in r.stdout
