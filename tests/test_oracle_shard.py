"""ZeRO-sharded step = unsharded step, bit for bit (the invariant printed in the
CS324 notes §3.4: parameter difference 0.0 after 15 steps on 4 simulated cards,
and still 0.0 at 8 cards, exercise 7(a)), and padding stays inert.

Each tensor's data is generated per (tensor, element), so every layout (N = 1
or N shards, whose bucket paddings differ) sees the same values.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
SEED = 0x5EED_0006


def _tensor_values(numel, M, steps):
    """master[t], grads[step][j][t] as per-tensor arrays."""
    master = [synth.host_normal_f32(n, synth.key(SEED, 10_000 + t), 0.02)
              for t, n in enumerate(numel)]
    grads = []
    for s in range(steps):
        per_j = []
        for j in range(M):
            per_j.append([synth.host_grad_bf16(n, synth.key(SEED, 20_000 + 97 * t + 7 * j + s),
                                               0, 1e-3) for t, n in enumerate(numel)])
        grads.append(per_j)
    return master, grads


def _to_shard(lay, per_tensor, dtype):
    out = np.zeros(lay.shard_len, dtype=dtype)
    for s in lay.segments:
        if s.tensor >= 0:
            out[s.shard_off:s.shard_off + s.length] = \
                per_tensor[s.tensor][s.tensor_off:s.tensor_off + s.length]
    return out


def _from_shards(lays, shard_arrays, numel, dtype):
    out = [np.full(n, np.nan if dtype == np.float32 else 0xFFFF, dtype=dtype) for n in numel]
    for lay, arr in zip(lays, shard_arrays):
        for s in lay.segments:
            if s.tensor >= 0:
                out[s.tensor][s.tensor_off:s.tensor_off + s.length] = \
                    arr[s.shard_off:s.shard_off + s.length]
    return out


def _run(numel, decay, N, M, steps, clip, cap, align=64):
    lays = [L.plan(numel, decay, N, r, cap, align) for r in range(N)]
    master, grads = _tensor_values(numel, M, steps)
    st = []
    for lay in lays:
        st.append(dict(p=_to_shard(lay, master, np.float32),
                       m=np.zeros(lay.shard_len, np.float32),
                       v=np.zeros(lay.shard_len, np.float32),
                       b=np.zeros(lay.shard_len, np.uint16)))
    for s in range(steps):
        shard_grads = [[_to_shard(lay, grads[s][j], np.uint16) for j in range(M)] for lay in lays]
        coef = None
        if clip:
            # the global norm: what the scalar all-reduce of per-shard partials carries
            sumsq = sum(oracle.grad_sumsq(g) for g in shard_grads)
            coef = oracle.clip_coef(sumsq, clip)
        for lay, g, x in zip(lays, shard_grads, st):
            oracle.step_f32(g, x["p"], x["m"], x["v"], x["b"], lay.decay_mask(), step=s + 1,
                            coef=coef, **HP)
    out = {k: _from_shards(lays, [x[k] for x in st], numel,
                           np.uint16 if k == "b" else np.float32) for k in "pmvb"}
    return lays, st, out


CASES = [
    # odd tensor sizes, tensors bigger than the bucket cap, zero-size tensor
    ([1, 63, 64, 65, 1000, 0, 4097, 12_345, 7, 300_000, 3], 50_000),
    ([5000] * 7 + [1], 8192),
]


@pytest.mark.parametrize("N", [2, 3, 7, 8, 16])
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("clip", [0.0, 0.05])
def test_sharded_equals_unsharded(N, case, clip):
    numel, cap = CASES[case]
    decay = [i % 2 for i in range(len(numel))]
    M, steps = 3, 3
    _, _, ref = _run(numel, decay, 1, M, steps, clip, cap)
    _, _, got = _run(numel, decay, N, M, steps, clip, cap)
    for k in "pmvb":
        for t in range(len(numel)):
            a, b = ref[k][t], got[k][t]
            assert a.view(np.uint32 if a.dtype == np.float32 else np.uint16).tobytes() == \
                b.view(np.uint32 if b.dtype == np.float32 else np.uint16).tobytes(), (k, t)


def test_zero_equals_dp_worked_example():
    spec = {}
    with open(os.path.join(GOLDEN, "zero_equals_dp.txt")) as f:
        for line in f:
            if not line.startswith("#") and line.strip():
                k, *vals = line.split()
                spec[k] = vals
    steps = int(spec["steps"][0])
    numel = [2000, 64, 333, 1, 4096, 777]
    decay = [1, 0, 1, 0, 1, 1]
    for cards in (int(c) for c in spec["cards"]):
        # cards data-parallel ranks -> M = cards gradient contributions per step
        _, _, dp = _run(numel, decay, 1, cards, steps, 0.0, 100_000)
        _, _, zero = _run(numel, decay, cards, cards, steps, 0.0, 100_000)
        diff = max(float(np.max(np.abs(a - b))) for a, b in zip(dp["p"], zero["p"]))
        assert diff == float(spec["max_abs_diff"][0])


@pytest.mark.parametrize("decay_flag", [0, 1])
def test_padding_is_inert(decay_flag):
    """Zero padding in every array stays exactly +0 through many steps."""
    numel = [1, 65, 130, 3]
    lay = L.plan(numel, [decay_flag] * 4, 4, 1, 10_000, 64)
    pad = lay.padding_ranges()
    assert sum(n for _, n in pad) > 0
    _, st, _ = _run(numel, [decay_flag] * 4, 4, 2, 5, 0.5, 10_000)
    x = st[1]
    for off, n in pad:
        for k in "pmvb":
            assert not x[k][off:off + n].view(np.uint32 if k != "b" else np.uint16).any()
