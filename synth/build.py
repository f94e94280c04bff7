"""Builds the two generator libraries in place (host: gcc + OpenMP; device: hipcc gfx950)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    host_out = os.path.join(_HERE, "libsynth_host.so")
    _run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
          "-o", host_out + ".tmp", os.path.join(_HERE, "synth_host.c")], verbose)
    os.replace(host_out + ".tmp", host_out)
    dev_out = os.path.join(_HERE, "libsynth_dev.so")
    _run(["hipcc", *HIP_FLAGS, "-o", dev_out + ".tmp", os.path.join(_HERE, "synth_dev.hip")],
         verbose)
    os.replace(dev_out + ".tmp", dev_out)
    return host_out, dev_out
