"""Builds tests/c_abi/abi_check: plain C against include/zeroshard.h, linked with the
product library, the oracle library (test infrastructure) and the system HIP runtime."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(_HERE))
EXE = os.path.join(_HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "sharded_optimizer_step_zero_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", os.path.join(_HERE, "abi_check.c"), "-o", EXE + ".tmp",
           f"-L{pkg}", "-lzeroshard", f"-L{orc}", "-lzo", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../sharded_optimizer_step_zero_amd:$ORIGIN/../../oracle:"
           f"{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
