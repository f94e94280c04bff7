"""Pins of the oracle's flat bucket / shard layout (pure integer work).

* the per-rank memory figures printed in the CS324 notes (exercise 1, §9);
* shard sizes of the GPT-1.3B / Llama-6.7B / Llama-70B parameter lists equal
  total/N (every tensor size there is a multiple of N * align, so no padding);
* structural invariants on random tensor lists: segments partition the shard,
  the ranks' slices re-concatenate to every bucket, tensors are aligned,
  buckets respect the cap.
"""
import os

import numpy as np
import pytest

from oracle import layout as L
from synth.workloads import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append(line.split())
    return rows


def test_memory_accounting_worked_examples():
    for row in _read_rows("zero_memory_accounting.txt"):
        psi, cards = int(row[0]), int(row[1])
        lay = L.plan([psi], [1], cards, 0, 25_000_000, 64)
        for stage, tok in enumerate(row[2:6]):
            decimals = len(tok.split(".")[1]) if "." in tok else 0
            gb = lay.state_bytes(stage) / 1e9
            assert round(gb, decimals) == float(tok), (psi, cards, stage, gb, tok)


@pytest.mark.parametrize("index,expect_total", [
    (2, 1_311_182_848), (3, 6_738_415_616), (4, 68_976_648_192)])
def test_model_shard_sizes(index, expect_total):
    w = workload(index)
    assert w.total_params == expect_total
    lay = L.plan(w.numel, w.decay, w.world_size, w.rank, w.bucket_cap, w.align)
    assert lay.shard_len * w.world_size == expect_total
    assert lay.padded_total == expect_total
    assert not lay.padding_ranges()


def _check_structure(numel, decay, N, cap, align):
    lays = [L.plan(numel, decay, N, r, cap, align) for r in range(N)]
    lay0 = lays[0]
    # tensors aligned, in order, inside their buckets, buckets respect the cap
    for t, n in enumerate(numel):
        b = lay0.tensor_bucket[t]
        bs, bl = lay0.buckets[b]
        off = lay0.tensor_flat_off[t]
        assert (off - bs) % align == 0 and bs <= off and off + n <= bs + bl
        if n == 0 and t > 0:  # only a tensor with elements closes a bucket
            assert b == lay0.tensor_bucket[t - 1]
    for b, (bs, bl) in enumerate(lay0.buckets):
        assert bl % (N * align) == 0
        assert bl > 0 or sum(numel) == 0          # no bucket is left empty
        ts = [t for t in range(len(numel)) if lay0.tensor_bucket[t] == b]
        assert ts == list(range(ts[0], ts[-1] + 1))
        used = lay0.tensor_flat_off[ts[-1]] + numel[ts[-1]] - bs
        # only a bucket holding a single non-empty tensor may exceed the cap
        assert used <= cap or sum(numel[t] > 0 for t in ts) == 1
        if b + 1 < len(lay0.buckets):  # closed because the next tensor did not fit
            nxt = ts[-1] + 1
            start_next = -(-used // align) * align
            assert start_next + numel[nxt] > cap
    assert lay0.buckets[0][0] == 0
    for (s0, l0), (s1, _) in zip(lay0.buckets, lay0.buckets[1:]):
        assert s1 == s0 + l0
    flat_len = lay0.padded_total
    owner = np.full(flat_len, -1, dtype=np.int64)
    tensor_of = np.full(flat_len, -1, dtype=np.int64)
    for t, n in enumerate(numel):
        tensor_of[lay0.tensor_flat_off[t]:lay0.tensor_flat_off[t] + n] = t
    for r, lay in enumerate(lays):
        assert lay.shard_len * N == flat_len
        # segments partition [0, shard_len) in order; no two padding segments adjoin
        pos = 0
        for s in lay.segments:
            assert s.shard_off == pos and s.length > 0
            pos += s.length
        assert pos == lay.shard_len
        for a, b in zip(lay.segments, lay.segments[1:]):
            assert not (a.tensor < 0 and b.tensor < 0)
        # map shard positions back to flat positions via the bucket slices
        sh = 0
        for bs, bl in lay.buckets:
            part = bl // N
            lo = bs + r * part
            assert (owner[lo:lo + part] == -1).all()
            owner[lo:lo + part] = r
            for s in lay.segments:
                a, e = max(s.shard_off, sh), min(s.shard_off + s.length, sh + part)
                if a >= e:
                    continue
                flat = np.arange(lo + a - sh, lo + e - sh)
                if s.tensor >= 0:
                    assert (tensor_of[flat] == s.tensor).all()
                    assert flat[0] - lay0.tensor_flat_off[s.tensor] == s.tensor_off + (a - s.shard_off)
                    assert s.decay == decay[s.tensor]
                else:
                    assert (tensor_of[flat] == -1).all() and s.decay == 0
            sh += part
        # tensor_slice agrees with the segments
        for t in range(len(numel)):
            _, _, ln = lay.tensor_slice(t)
            covered = sum(s.length for s in lay.segments if s.tensor == t)
            assert ln == covered
    assert (owner >= 0).all()                      # the ranks' slices cover every bucket
    # every tensor element is owned by exactly one rank
    total = sum(sum(s.length for s in lay.segments if s.tensor >= 0) for lay in lays)
    assert total == sum(numel)


@pytest.mark.parametrize("seed", range(12))
def test_layout_structure_random(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 40))
    numel = [int(x) for x in rng.integers(0, 5000, T)]
    if seed % 3 == 0:
        big = int(rng.integers(0, T))
        numel[big] = 25_000  # larger than the cap below
        if seed % 2 == 0:    # an empty tensor right after it, and leading empty tensors
            numel.insert(big + 1, 0)
            numel[0:0] = [0, 0]
    decay_n = len(numel)
    decay = [int(x) for x in rng.integers(0, 2, decay_n)]
    N = int(rng.choice([1, 2, 3, 4, 7, 8, 16]))
    align = int(rng.choice([8, 16, 64]))
    cap = int(rng.choice([4096, 10_000, 20_000]))
    _check_structure(numel, decay, N, cap, align)


@pytest.mark.parametrize("numel", [[5000, 0, 7000], [0, 0, 5000, 0, 0, 7000, 0],
                                   [300, 5000, 0, 0, 6000], [0], [0, 0], [5000, 0], [0, 5000]])
def test_empty_tensors_structure(numel):
    """Empty tensors before, between and after tensors larger than the cap."""
    for N in (1, 4):
        _check_structure(numel, [1] * len(numel), N, 4096, 64)
        lay = L.plan(numel, [1] * len(numel), N, 0, 4096, 64)
        assert len(lay.buckets) == max(1, sum(n > 0 for n in numel))


def test_bucket_closes_only_beyond_the_cap():
    """A tensor that ends exactly at the cap still joins the open bucket; one
    element more and it opens the next."""
    lay = L.plan([64, 64], [1, 1], 2, 0, 128, 64)
    assert lay.buckets == [(0, 128)] and lay.tensor_bucket == [0, 0]
    lay = L.plan([64, 65], [1, 1], 2, 0, 128, 64)
    assert lay.buckets == [(0, 128), (128, 128)] and lay.tensor_bucket == [0, 1]
    lay = L.plan([1, 64], [1, 1], 1, 0, 128, 64)  # alignment counts: 64 + 64 fits
    assert lay.tensor_flat_off == [0, 64] and len(lay.buckets) == 1
    lay = L.plan([1, 65], [1, 1], 1, 0, 128, 64)  # 64 + 65 does not
    assert lay.tensor_flat_off == [0, 64] and len(lay.buckets) == 2


def test_gpt_buckets():
    w = workload(2)
    lay = L.plan(w.numel, w.decay, 8, 0, w.bucket_cap, w.align)
    assert len(lay.buckets) == 73
    assert all(bl <= w.bucket_cap or bl == 50304 * 2048 for _, bl in lay.buckets)


@pytest.mark.parametrize("N", [1, 3, 8])
def test_canonical_mapping_partitions_the_model(N):
    """Over all ranks, the shards' tensor elements map onto the canonical order
    (tensors concatenated, unpadded) exactly once, and back."""
    numel = [1, 63, 64, 65, 1000, 0, 4097, 12_345, 7, 30_001, 3]
    decay = [i % 2 for i in range(len(numel))]
    canon_want = np.concatenate([np.full(n, t, np.int64) * 100_000 + np.arange(n)
                                 for t, n in enumerate(numel)])
    got = np.full(canon_want.size, -1, np.int64)
    seen = np.zeros(canon_want.size, np.int64)
    for r in range(N):
        lay = L.plan(numel, decay, N, r, 20_000, 64)
        shard = np.full(lay.shard_len, -7, np.int64)
        for s in lay.segments:
            if s.tensor >= 0:
                shard[s.shard_off:s.shard_off + s.length] = \
                    s.tensor * 100_000 + np.arange(s.tensor_off, s.tensor_off + s.length)
        part = np.full(canon_want.size, -1, np.int64)
        lay.to_canonical(shard, part)
        seen += part >= 0
        got[part >= 0] = part[part >= 0]
        back = np.full(lay.shard_len, -7, np.int64)
        lay.from_canonical(canon_want, back)
        assert np.array_equal(back, shard)
    assert (seen == 1).all()
    assert np.array_equal(got, canon_want)
