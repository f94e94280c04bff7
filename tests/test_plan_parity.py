"""The library's layout planner against the oracle layout, exactly (integer work):
shard length, buckets, segments, tensor slices and per-stage bytes on the five
workloads (several ranks) and on random tensor lists; plus the properties the
step kernel relies on for the chunk table."""
import numpy as np
import pytest

import sharded_optimizer_step_zero_amd as zs
from oracle import layout as L
from synth.workloads import workload


def _compare(numel, decay, N, r, cap, align):
    lay = L.plan(numel, decay, N, r, cap, align)
    p = zs.zs_plan_create(numel, decay, N, r, cap, align)
    try:
        q = zs.zs_plan_query(p)
        assert q["shard_len"] == lay.shard_len
        assert q["padded_total"] == lay.padded_total
        assert q["n_buckets"] == len(lay.buckets)
        assert q["n_segments"] == len(lay.segments)
        for b, (off, ln) in enumerate(lay.buckets):
            assert zs.zs_plan_bucket(p, b) == (off, ln)
        for i, s in enumerate(lay.segments):
            assert zs.zs_plan_segment(p, i) == (s.shard_off, s.length, s.tensor, s.tensor_off,
                                                s.decay), i
        for t in range(len(numel)):
            assert zs.zs_plan_tensor_slice(p, t) == lay.tensor_slice(t), t
        for stage in range(4):
            assert zs.zs_plan_state_bytes(p, stage) == lay.state_bytes(stage)
        _check_runs(p, q, lay, align)
    finally:
        zs.zs_plan_destroy(p)


def _check_runs(p, q, lay, align):
    n = q["n_runs"]
    offs = np.empty(n, np.int64)
    lens = np.empty(n, np.int64)
    flags = np.empty(n, np.int64)
    for i in range(n):
        offs[i], lens[i], flags[i] = zs.zs_plan_run(p, i)
    if lay.shard_len == 0:
        assert n == 0
        return
    # an exact partition of [0, shard_len), in order, runs starting on align boundaries
    assert offs[0] == 0
    assert np.array_equal(offs[1:], offs[:-1] + lens[:-1])
    assert offs[-1] + lens[-1] == lay.shard_len
    assert (lens > 0).all() and (offs % align == 0).all()
    # neighbouring runs differ (maximal), and each run's flag is every tensor element's flag
    assert (flags[1:] != flags[:-1]).all()
    seg_off = np.array([x.shard_off for x in lay.segments], np.int64)
    seg_end = np.array([x.shard_off + x.length for x in lay.segments], np.int64)
    seg_flag = np.array([x.decay for x in lay.segments], np.int64)
    seg_tensor = np.array([x.tensor >= 0 for x in lay.segments], bool)
    first = np.searchsorted(seg_end, offs, side="right")
    last = np.searchsorted(seg_off, offs + lens, side="left")
    for i in range(n):
        sl = slice(first[i], last[i])
        assert (seg_flag[sl][seg_tensor[sl]] == flags[i]).all(), i


@pytest.mark.parametrize("index,ranks", [(1, [0]), (2, [0, 3, 7]), (3, [0]), (4, [0, 15]),
                                         (5, [0])])
def test_workloads(index, ranks):
    w = workload(index)
    for r in ranks:
        _compare(w.numel, w.decay, w.world_size, r, w.bucket_cap, w.align)


@pytest.mark.parametrize("seed", range(20))
def test_random_lists(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(0, 60))
    numel = [int(x) for x in rng.integers(0, 9000, T)]
    decay = [int(x) for x in rng.integers(0, 2, T)]
    N = int(rng.choice([1, 2, 3, 5, 8, 16]))
    align = int(rng.choice([8, 64, 128]))
    cap = int(rng.choice([1000, 8192, 40_000]))
    for r in {0, N - 1, int(rng.integers(0, N))}:
        _compare(numel, decay, N, r, cap, align)


@pytest.mark.parametrize("numel", [[5000, 0, 7000], [0, 0, 5000, 0, 0, 7000, 0], [300, 5000, 0, 0, 6000],
                                   [0], [0, 0], [5000, 0]])
def test_empty_tensors_leave_no_empty_bucket(numel):
    """A tensor without elements joins the open bucket: with a cap below the
    tensors, an empty tensor after an oversize one must not open a bucket that the
    next tensor closes empty."""
    decay = [1] * len(numel)
    for N, r in ((1, 0), (4, 3)):
        _compare(numel, decay, N, r, 4096, 64)
        lay = L.plan(numel, decay, N, r, 4096, 64)
        if sum(numel):
            assert all(ln > 0 for _, ln in lay.buckets), lay.buckets
        assert len(lay.buckets) == max(1, sum(1 for n in numel if n > 0)) or sum(numel) == 0
