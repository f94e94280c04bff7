"""Compiles the product library libzeroshard.so in place (hipcc, gfx950)."""
from __future__ import annotations

import os
import subprocess
import tempfile

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libzeroshard.so")
SOURCES = [os.path.join(_HERE, "csrc", f)
           for f in ("kernels.hip", "plan.cpp", "abi.cpp", "offload.cpp", "alloc.cpp",
                     "static_step.hip")]
# host-compiled part: the offloaded update (vector clones picked at load time)
HOST_SOURCES = [os.path.join(_HERE, "csrc", "host_step.cpp")]
GXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-math-errno", "-pthread",
             "-Wall", "-Wextra"]

# -ffp-contract=off: no FMA contraction (each operation rounds once);
# correctly rounded fp32 division / sqrt; fp32 subnormals kept;
# packed-fp32 instructions disabled.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
               "-fno-gpu-flush-denormals-to-zero",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall"]


def build(verbose: bool = False, extra_flags=None) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = ["g++", *GXX_FLAGS, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        # the host objects go to the linker as they are (hipcc would read them as source)
        cmd = ["hipcc", *HIPCC_FLAGS, *(extra_flags or []), "-o", LIB + ".tmp", *SOURCES,
               *[f"-Wl,{o}" for o in objs], "-pthread"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB
