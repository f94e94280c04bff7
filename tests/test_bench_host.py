"""bench.py's host side (no GPU): the one-GPU guard, the algorithmic byte count the
roofline divides by, the kernel-source hash that keeps counter records honest, and the
committed traffic records themselves."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.workloads import workload  # noqa: E402
from oracle import layout as L  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_algorithmic_bytes(M):
    # read: M bf16 contributions + fp32 master, m, v; written: master, m, v + bf16 param;
    # the clipped step reads the contributions once more for the norm
    S = 1000
    b = bench.algorithmic_bytes(S, M, False)
    assert b["step_kernel"] == S * ((2 * M + 12) + (12 + 2)) and b["norm_pass"] == 0
    c = bench.algorithmic_bytes(S, M, True)
    assert c["norm_pass"] == S * 2 * M and c["total"] == c["step_kernel"] + S * 2 * M


def _sources():
    d = os.path.join(ROOT, "sharded_optimizer_step_zero_amd", "csrc")
    return {f: open(os.path.join(d, f), encoding="utf-8").read()
            for f in ("kernels.hip", "internal.h")}


def test_source_hash_ignores_comments_not_code():
    src = _sources()
    base = bench.kernel_source_hash(lambda f: src[f])
    assert base == bench.kernel_source_hash()
    commented = dict(src, **{"kernels.hip": "// a new comment line\n" + src["kernels.hip"]
                             .replace("\n", "   // trailing note\n", 1) + "\n\n"})
    assert bench.kernel_source_hash(lambda f: commented[f]) == base
    edited = dict(src, **{"internal.h": src["internal.h"] + "\nconstexpr int kUnused = 1;\n"})
    assert bench.kernel_source_hash(lambda f: edited[f]) != base


TRAFFIC = sorted(glob.glob(os.path.join(ROOT, "profiles", "step_kernel_traffic_*.json")))


def test_traffic_records_exist():
    assert len(TRAFFIC) >= 3


@pytest.mark.parametrize("path", TRAFFIC, ids=[os.path.basename(p) for p in TRAFFIC])
def test_traffic_record_matches_kernel_and_workload(path):
    """Each committed counter record was taken on the current step-kernel source (else
    the bench reports traffic as null), names an existing summary, and its HBM bytes per
    launch agree with the algorithmic bytes of its workload within 0.5%."""
    with open(path) as f:
        rec = json.load(f)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash(), \
        "kernel source changed since the counters were taken: re-take FETCH/WRITE_SIZE"
    assert os.path.exists(os.path.join(ROOT, rec["source"]))
    names = {workload(i).name: i for i in range(1, 6)}
    w = workload(names[rec["workload"]])
    S = L.plan(w.numel, w.decay, w.world_size, w.rank, w.bucket_cap, w.align).shard_len
    alg = bench.algorithmic_bytes(S, w.M, False)["step_kernel"]
    assert abs(rec["hbm_bytes_per_launch"] / alg - 1) < 5e-3
    assert bench.traffic_for(rec["workload"]) == rec["hbm_bytes_per_launch"]
