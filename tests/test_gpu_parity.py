"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: fp32 master, m, v within 1e-6 max relative error per step, bf16 param
within 1 ulp; the kernels are built to match the oracle bit for bit (fixed
reduction order, one rounding per operation, correctly rounded div/sqrt), so
the tests also require exact equality.  Whole-shard checks run on the small
and GPT-1.3B-shard workloads and on multi-tensor cases spanning many chunks
with ragged tails; the 6.7B, 70B-shard and stress workloads run at full size
and are checked on sampled elements (seeded windows, the first/last 64
elements of every segment, every padding element).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import scaled, workload

from _gpu import full_parity, log, sampled_parity

pytestmark = pytest.mark.gpu


def _report(name, stats):
    """Logs the parity summary of a run; with ZS_PARITY_REPORT set to a directory it
    also writes it there as <name>.json (per-field worst per-step error, the bf16
    ulp histogram over every checked element and step, and the drift of the
    free-running oracle trajectory at steps 1, 10, 100, 1000 and the last)."""
    worst = {k: max(s[k] for s in stats) for k in ("rel_master", "rel_m", "rel_v")}
    exact = sum(s["exact"] for s in stats)
    hist = {}
    for s in stats:
        for k, c in s["bf16_hist"].items():
            hist[k] = hist.get(k, 0) + c
    last = stats[-1]["step"]
    drift = {s["step"]: {k: s[k] for k in ("drift_master", "drift_m", "drift_v",
                                           "drift_bf16_ulps")}
             for s in stats if s["step"] in (1, 10, 100, 1000, last)}
    coef = [s["coef_ulps"] for s in stats if "coef_ulps" in s]
    log(f"  [{name}] steps checked {len(stats)}, exact {exact}, worst rel {worst}, "
        f"bf16 ulp histogram {hist}, coef ulps {sorted(set(coef))}, drift {drift}")
    out = os.environ.get("ZS_PARITY_REPORT")
    if out:
        os.makedirs(out, exist_ok=True)
        rec = dict(name=name, steps_checked=len(stats), elements=stats[0]["n"],
                   exact_steps=exact, worst=worst, bf16_ulp_hist=hist,
                   coef_ulps=sorted(set(coef)),
                   norm_rel_max=max((s["norm_rel"] for s in stats if "norm_rel" in s),
                                    default=None),
                   drift=drift)
        with open(os.path.join(out, f"{name}.json"), "w") as f:
            json.dump(rec, f, indent=1)


def test_tiny_flat_full():
    w = workload(1)
    log(f"test_tiny_flat_full: S={w.total_params} M={w.M} steps={w.steps}")
    _report(w.name, full_parity(w, w.steps))


def test_tiny_flat_drift_1000_steps():
    """The tiny workload run for 1000 steps, every element checked every step, and
    the drift of the device trajectory against a free-running oracle reported."""
    w = workload(1)
    log(f"test_tiny_flat_drift_1000_steps: S={w.total_params} M={w.M} steps=1000")
    _report(w.name + "-1000steps", full_parity(w, 1000))


SMALL = [
    # (numel, decay, N, rank, M, max_norm, align): many decay runs, runs starting
    # inside 256-element tiles, ragged shard ends, N up to 16, M up to 16
    ([1, 63, 64, 65, 1000, 0, 4097, 12_345, 7, 300_001, 3], None, 3, 1, 3, 0.0, 64),
    ([5000] * 7 + [1], None, 8, 7, 8, 0.05, 64),
    ([70_001, 64, 5, 2 ** 17 + 8], [1, 0, 0, 1], 1, 0, 5, 0.0, 8),
    ([33_333] * 5, [0, 1, 0, 1, 0], 2, 0, 16, 1e-4, 64),
    ([1 << 16], [1], 1, 0, 1, 0.0, 64),
    ([200_000, 17], [1, 1], 16, 5, 7, 10.0, 128),
    ([3, 9, 1, 17, 2, 40, 5, 8] * 40, [1, 0] * 160, 1, 0, 2, 0.0, 8),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_multi_tensor_full(case):
    numel, decay, N, rank, M, clip, align = SMALL[case]
    w = scaled(workload(1), numel, decay, world_size=N, rank=rank, M=M,
               name=f"small{case}")
    w.max_grad_norm = clip
    w.align = align
    log(f"test_small_multi_tensor_full[{case}]: tensors={len(numel)} N={N} r={rank} M={M} "
        f"clip={clip} align={align}")
    _report(w.name, full_parity(w, 4))


def test_gpt13b_shard_full():
    w = workload(2)
    log(f"test_gpt13b_shard_full: {w.description}, steps={w.steps}")
    _report(w.name, full_parity(w, w.steps))


def test_llama67b_unsharded_sampled():
    w = workload(3)
    log(f"test_llama67b_unsharded_sampled: {w.description}, steps={w.steps}")
    _report(w.name, sampled_parity(w, w.steps))


def test_llama70b_shard_sampled():
    w = workload(4)
    log(f"test_llama70b_shard_sampled: {w.description}, steps={w.steps}")
    _report(w.name, sampled_parity(w, w.steps))


def test_stress_clip_sampled():
    from synth.device_case import DeviceCase
    from oracle import layout as L
    w = workload(5)
    log(f"test_stress_clip_sampled: {w.description}")
    from synth.workloads import special_ranges
    lay = L.plan(w.numel, w.decay, 1, 0, w.bucket_cap, w.align)
    special = special_ranges(w, [(x.shard_off, x.length, x.tensor) for x in lay.segments])
    case = DeviceCase(w, lay.shard_len, lay.padding_ranges(), "cpu", special)
    norms = {}

    def full_norm(step0):
        gs = w.grad_step_index(step0)
        if gs not in norms:
            norms[gs] = oracle.grad_sumsq(case.host_grads(step0))
            log(f"  oracle norm {np.sqrt(norms[gs]):.6e} over S={lay.shard_len:,}")
        return norms[gs]

    from _gpu import sample_indices
    idx = np.union1d(sample_indices(lay, n_windows=1024, edge=16),
                     np.concatenate([np.arange(o, o + n) for o, n, _ in special]))
    log(f"  {idx.size:,} sampled elements")
    checks = {1, 2, 3, 10, 100, 500, 1000} | set(range(50, 1001, 50))
    _report(w.name, sampled_parity(w, w.steps, idx=idx, check_steps=checks,
                                   full_norm=full_norm))
