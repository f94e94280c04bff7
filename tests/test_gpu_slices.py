"""Grids issued as several launches.

One dispatch carries at most 2^32 - 1 work-items, which the step grid passes
beyond 2^34 elements (one 64-lane work-group per 256 elements).  Every kernel
with a size-dependent grid (the step kernels, the norm passes, the state copy)
is issued as consecutive slices of whole work-groups, each slice's kernel
adding its first group's index.  Such shards do not fit a test, so these tests
lower the slice size with ZS_MAX_GROUPS_PER_LAUNCH (read when a context is
created) and check every path against the oracle, bit for bit: slices of 1, 3
and 7 groups cut through weight-decay runs, norm tiles and checkpoint pieces
at every possible place.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard
from synth.workloads import scaled, workload

from _gpu import full_parity, log, to_host

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
SLICES = ["1", "3", "7"]

# (numel, decay, N, rank, M, max_norm): many decay runs with runs starting
# inside tiles and a ragged end; a clipped shard with M = 16
CASES = [
    ([1, 63, 64, 65, 1000, 0, 4097, 12_345, 7, 300_001, 3], None, 3, 1, 3, 0.0),
    ([33_333] * 5, [0, 1, 0, 1, 0], 2, 0, 16, 1e-4),
    ([5000] * 7 + [1], None, 8, 7, 8, 0.05),
]


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("stage", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("groups", SLICES)
def test_sliced_bf16_step_matches_oracle(monkeypatch, groups, case, stage):
    monkeypatch.setenv("ZS_MAX_GROUPS_PER_LAUNCH", groups)
    numel, decay, N, rank, M, clip = CASES[case]
    w = scaled(workload(1), numel, decay, world_size=N, rank=rank, M=M, name=f"sliced{case}")
    w.max_grad_norm = clip
    log(f"test_sliced_bf16_step_matches_oracle groups={groups} case={case} stage={stage}")
    full_parity(w, 3, flags=zsm.ZS_STAGE_AVERAGE if stage else 0)


@pytest.mark.parametrize("stage", [False, True])
@pytest.mark.parametrize("groups", SLICES)
def test_sliced_amp_step_matches_oracle(monkeypatch, groups, stage):
    monkeypatch.setenv("ZS_MAX_GROUPS_PER_LAUNCH", groups)
    log(f"test_sliced_amp_step_matches_oracle groups={groups} stage={stage}")
    numel = [70_001, 64, 5, 13_000, 333]
    decay = [1, 0, 0, 1, 0]
    N, rank, M = 3, 1, 3
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    z = ZeroShard(numel, decay, N, rank, M, fp16=True,
                  flags=zsm.ZS_STAGE_AVERAGE if stage else 0, grad_buffers=True)
    S = z.shard_len
    pad = lay.padding_ranges()
    master = synth.host_normal_f32(S, synth.key(91, 0), 0.02)
    for o, n in pad:
        master[o:o + n] = 0
    z.master[:S].copy_(torch.from_numpy(master))
    z.amp_init(2.0 ** 12)
    sc = oracle.Scaler(scale=2.0 ** 12, growth_interval=2)
    p, m, v = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    pf = np.zeros(S, np.uint16)
    mask = lay.decay_mask()
    for s in range(5):
        scale = float(sc.scale[0])
        gs = []
        for j in range(M):
            g = synth.host_grad_f16(S, synth.key(91, 1 + j + M * s), 1e-3, scale)
            for o, n in pad:
                g[o:o + n] = 0
            gs.append(g)
        if s == 2:
            gs[2][S - 9] = 0x7C00              # an overflow near the end: every slice skips
        for j, g in enumerate(gs):
            z.grads[j][:S].copy_(torch.from_numpy(g.view(np.int16)).view(torch.float16))
        clip = 0.01 if s % 2 else 0.0
        z.step_amp(z.grads, max_grad_norm=clip, growth_interval=2, **HP)
        torch.cuda.synchronize()
        fi, _ = oracle.amp_step(gs, p, m, v, pf, mask, sc, max_grad_norm=clip, **HP)
        assert fi == (s == 2)
        got = [to_host(z.master)[:S], to_host(z.exp_avg)[:S], to_host(z.exp_avg_sq)[:S],
               z.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]]
        for a, b in zip(got, (p, m, v, pf)):
            assert np.array_equal(_bits(a), _bits(b)), s
        assert z.amp_read() == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied), s
    z.close()


@pytest.mark.parametrize("groups", SLICES)
def test_sliced_state_copy_matches_layout(monkeypatch, groups):
    monkeypatch.setenv("ZS_MAX_GROUPS_PER_LAUNCH", groups)
    log(f"test_sliced_state_copy_matches_layout groups={groups}")
    # tensors above the 65,536-element piece size, so pieces and their parts both split
    numel = [3000, 1, 64, 140_001, 5, 4096, 70_000, 0, 129]
    decay = [1, 0, 0, 1, 0, 1, 1, 0, 0]
    N, rank, M = 2, 1, 2
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    z = ZeroShard(numel, decay, N, rank, M)
    S, total = z.shard_len, sum(numel)
    shard = [synth.host_normal_f32(S, synth.key(92, k), 1.0) for k in range(3)]
    for a in shard:
        for o, n in lay.padding_ranges():
            a[o:o + n] = 0
    for t, a in zip((z.master, z.exp_avg, z.exp_avg_sq), shard):
        t[:S].copy_(torch.from_numpy(a))
    # export: this rank's elements land at their canonical offsets, the rest untouched
    fill = np.float32(-7.0)
    canon = [torch.full((total,), float(fill), device="cuda") for _ in range(3)]
    z.export_state(*canon)
    torch.cuda.synchronize()
    for a, c in zip(shard, canon):
        want = np.full(total, fill, np.float32)
        lay.to_canonical(a, want)
        assert np.array_equal(_bits(to_host(c)), _bits(want))
    # import of other values: state and the bf16 param of this rank's elements
    new = [synth.host_normal_f32(total, synth.key(93, k), 1.0) for k in range(3)]
    for t in (z.master, z.exp_avg, z.exp_avg_sq):
        t.zero_()
    z.import_state(*[torch.from_numpy(a).cuda() for a in new])
    torch.cuda.synchronize()
    for t, a in zip((z.master, z.exp_avg, z.exp_avg_sq), new):
        want = np.zeros(S, np.float32)
        lay.from_canonical(a, want)
        assert np.array_equal(_bits(to_host(t)[:S]), _bits(want))
    want_p = np.zeros(S, np.float32)
    lay.from_canonical(new[0], want_p)
    got_p = z.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]
    own = np.ones(S, bool)
    for o, n in lay.padding_ranges():
        own[o:o + n] = False
    assert np.array_equal(got_p[own], oracle.f32_to_bf16(want_p)[own])
    z.close()
