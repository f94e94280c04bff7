"""The seeded input generator (shared by both sides; holds no optimizer arithmetic).

* h(key, i) is the published splitmix64 sequence;
* the C generator equals the definition written out in Python integers;
* random access (at indices) equals the contiguous fill;
* value distribution and gradient-kind frequencies are as configured.
"""
import os

import numpy as np

import synth
from synth.workloads import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MASK = (1 << 64) - 1


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_splitmix64_published_sequence():
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt")) as f:
        want = [int(x) for x in f if x.strip() and not x.startswith("#")]
    assert [synth.hash_at(1234567, i) for i in range(len(want))] == want


def test_host_generator_matches_definition():
    k = synth.key(77, 3)
    assert k == _mix((77 * 0x9E3779B97F4A7C15 + 3) & MASK)
    sigma = 0.02
    scale = synth.scale_for(sigma)
    vals = synth.host_normal_f32(50, k, sigma, base=1000)
    for i in range(50):
        h = _mix((k + (1000 + i + 1) * 0x9E3779B97F4A7C15) & MASK)
        s = (h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48)
        want = np.float32(np.float32(s - 131070) * scale)
        assert vals[i].view(np.uint32) == want.view(np.uint32)
    g = synth.host_grad_bf16(50, k, 0, sigma, base=1000)
    assert np.array_equal(g, (vals.view(np.uint32) >> 16).astype(np.uint16))


def test_random_access_equals_fill():
    k, ks = synth.key(5, 1), synth.key(5, 2)
    kinds = synth.Kinds(50_000, 1_000, 10_000, 1e3)
    full = synth.host_grad_bf16(100_000, k, ks, 1e-3, kinds)
    idx = np.array([0, 1, 99_999, 12_345, 777, 50_000])
    assert np.array_equal(synth.host_grad_bf16_at(idx, k, ks, 1e-3, kinds), full[idx])
    fm = synth.host_normal_f32(100_000, k, 0.02)
    assert np.array_equal(synth.host_normal_f32_at(idx, k, 0.02), fm[idx])


def test_distribution_and_kinds():
    n = 2_000_000
    k, ks = synth.key(9, 1), synth.key(9, 0x10001)
    x = synth.host_normal_f32(n, k, 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() / 0.02 - 1) < 5e-3
    kinds = synth.Kinds(50_000, 1_000, 10_000, 1e3)
    g = synth.host_grad_bf16(n, k, ks, 1e-3, kinds)
    zero = g == 0
    sub = ((g & 0x7F80) == 0) & ((g & 0x7F) != 0)
    gf = (g.astype(np.uint32) << 16).view(np.float32)
    big = np.abs(gf) > 0.05
    assert abs(zero.mean() - 0.05) < 0.002
    assert abs(sub.mean() - 0.001) < 0.0003
    assert abs(big.mean() - 0.01 * 0.9999) < 0.002     # outliers are ~N(0, 1) here


def test_stress_workload_shapes():
    w = workload(5)
    assert len(w.numel) == 10_064
    assert sum(1 for n in w.numel if n == 4096 * 4096) == 64
    small = [n for n in w.numel if n != 4096 * 4096]
    assert min(small) >= 1 and max(small) <= 4096
    assert all((d == 1) == (n == 4096 * 4096) for n, d in zip(w.numel, w.decay))
    assert workload(5).numel == w.numel   # seeded, reproducible


def test_special_tensor_overrides_host_sampled_equals_whole():
    from oracle import layout as L
    from synth.device_case import DeviceCase
    from synth.workloads import scaled, special_ranges
    w = scaled(workload(5), [300, 4000, 70, 1000, 5], [0, 0, 0, 1, 0], M=3)
    w.special = {"zero": [0, 2], "subnormal": [1]}
    lay = L.plan(w.numel, w.decay, 1, 0, w.bucket_cap, w.align)
    sp = special_ranges(w, [(s.shard_off, s.length, s.tensor) for s in lay.segments])
    case = DeviceCase.__new__(DeviceCase)      # host twins only: no device buffers
    case.w, case.S, case.pad = w, lay.shard_len, lay.padding_ranges()
    case.zero = [(o, n) for o, n, k in sp if k == "zero"]
    sub = [(o, n) for o, n, k in sp if k == "subnormal"]
    case.sub_idx = np.concatenate([np.arange(o, o + n) for o, n in sub]).astype(np.int64)
    whole = case.host_grads(0)
    idx = np.arange(0, lay.shard_len, 7, dtype=np.int64)
    at = case.host_grads(0, idx)
    for a, b in zip(whole, at):
        assert np.array_equal(a[idx], b)
    for g in whole:
        for o, n, k in sp:
            piece = g[o:o + n]
            if k == "zero":
                assert not piece.any()
            else:
                assert ((piece & 0x7F80) == 0).all() and ((piece & 0x7F) != 0).all()
