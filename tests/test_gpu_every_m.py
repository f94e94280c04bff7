"""GPU parity for every compiled contribution count M = 1..16.

The kernels are instantiated per M (the reduction is unrolled over the M
contributions), so each instantiation is checked on its own against the oracle,
bit for bit: the bf16 step with and without clipping (step_kernel<M, CLIP>,
sumsq_kernel<M, false>), the staged clip (sumsq_kernel<M, true>), and the
loss-scaled fp16 step fused and staged (sumsq_f16_kernel<M, STAGE>,
step_f16_kernel<M>).  The layout is small but spans several 256-element tiles,
several decay runs, a run starting inside a tile and a ragged shard end.
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

NUMEL = [3001, 64, 5, 9000, 130]
DECAY = [1, 0, 0, 1, 0]
N, RANK = 3, 2
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@pytest.mark.parametrize("M", range(1, 17))
@pytest.mark.parametrize("mode", ["plain", "clip", "staged_clip"])
def test_bf16_step_every_m(mode, M):
    w = scaled(workload(1), NUMEL, DECAY, world_size=N, rank=RANK, M=M, name=f"m{M}-{mode}")
    w.max_grad_norm = 0.0 if mode == "plain" else 0.005  # binding at every M
    w.align = 64
    log(f"test_bf16_step_every_m: M={M} mode={mode}")
    flags = zsm.ZS_STAGE_AVERAGE if mode == "staged_clip" else 0
    stats = full_parity(w, 3, flags=flags)
    assert all(s["exact"] for s in stats)


def _u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("M", range(1, 17))
@pytest.mark.parametrize("stage", [False, True])
def test_amp_step_every_m(stage, M):
    log(f"test_amp_step_every_m: M={M} stage={stage}")
    lay = L.plan(NUMEL, DECAY, N, RANK, 25_000_000, 64)
    z = ZeroShard(NUMEL, DECAY, N, RANK, M, fp16=True,
                  flags=zsm.ZS_STAGE_AVERAGE if stage else 0)
    S = z.shard_len
    assert S == lay.shard_len
    pad = lay.padding_ranges()
    master = synth.host_normal_f32(S, synth.key(900 + M, 0), 0.02)
    for o, n in pad:
        master[o:o + n] = 0
    z.master[:S].copy_(torch.from_numpy(master))
    z.amp_init(2.0 ** 12)
    sc = oracle.Scaler(scale=2.0 ** 12, growth_interval=2)
    p, m, v = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    pf = np.zeros(S, np.uint16)
    mask = lay.decay_mask()
    hit = [x for x in lay.segments if x.tensor >= 0][-1].shard_off + 7  # inside a tensor
    for s in range(4):
        scale = float(sc.scale[0])
        gs = []
        for j in range(M):
            g = synth.host_grad_f16(S, synth.key(900 + M, 1 + j + M * s), 1e-3, scale)
            for o, n in pad:
                g[o:o + n] = 0
            gs.append(g)
        if s == 2:
            gs[M - 1][hit] = 0x7C00  # the last contribution overflows: the step is skipped
        clip = 0.0 if s % 2 == 0 else 0.01  # binding at every M
        rc, norm = z.step_amp([_u16(g) for g in gs], max_grad_norm=clip, growth_interval=2,
                              want_norm=True, return_code=True, **HP)
        fi, onorm = oracle.amp_step(gs, p, m, v, pf, mask, sc, max_grad_norm=clip, **HP)
        assert (rc == zsm.ZS_NONFINITE) == fi == (s == 2)
        if not fi:
            assert abs(norm - onorm) <= 1e-12 * onorm
        got = [to_host(z.master)[:S], to_host(z.exp_avg)[:S], to_host(z.exp_avg_sq)[:S],
               z.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]]
        for name, a, b in zip("pmvb", got, (p, m, v, pf)):
            assert np.array_equal(_bits(a), _bits(b)), (s, name)
        assert z.amp_read() == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied)
    z.close()
