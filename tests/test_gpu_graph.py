"""The step inside a HIP graph: captured once on a side stream, replayed several
times with eager work in between, every replay checked bit for bit against an
eager twin doing the same calls.  The steps queue only kernels (no memset, no
host wait, no allocation) when no norm is read back, so they capture as they
are; the loss-scaled step keeps its step count and scale on the device, so one
captured step replays as consecutive optimizer steps."""
import numpy as np
import pytest
import torch

import sharded_optimizer_step_zero_amd as zsm
import synth
from sharded_optimizer_step_zero_amd import ZeroShard
from synth.workloads import scaled, workload

from _gpu import Shard, log, to_host

pytestmark = pytest.mark.gpu
NUMEL, DECAY = [5000, 64, 130_001, 7, 2 ** 16], [1, 0, 1, 0, 1]


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _state(z):
    return [to_host(x)[:z.shard_len].copy() for x in (z.master, z.exp_avg, z.exp_avg_sq, z.param)]


@pytest.mark.parametrize("flags", [0, zsm.ZS_SKIP_NONFINITE | zsm.ZS_STAGE_AVERAGE])
def test_bf16_step_replays_equal_eager(flags):
    log(f"test_bf16_step_replays_equal_eager flags={flags}")
    w = scaled(workload(1), NUMEL, DECAY, world_size=2, rank=1, M=3, name="graph")
    a, b = Shard(w, flags=flags), Shard(w, flags=flags)      # graph, eager
    grads_a = a.case.fill_grads(0)
    grads_b = b.case.fill_grads(0)
    hp = a.hp()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a.zs.set_stream(side.cuda_stream)
        a.zs.step(grads_a, step=7, max_grad_norm=0.5, **hp)     # warm-up outside the graph
        b.zs.step(grads_b, step=7, max_grad_norm=0.5, **hp)
        torch.cuda.synchronize()
    with torch.cuda.graph(g):
        a.zs.set_stream(torch.cuda.current_stream().cuda_stream)
        a.zs.step(grads_a, step=8, max_grad_norm=0.5, **hp)
    a.zs.set_stream(torch.cuda.current_stream().cuda_stream)
    b.zs.set_stream(torch.cuda.current_stream().cuda_stream)
    for r in range(4):
        g.replay()
        b.zs.step(grads_b, step=8, max_grad_norm=0.5, **hp)
        # eager work between replays: perturb both runs' gradients the same way
        for ga, gb in zip(grads_a, grads_b):
            ga.mul_(1.5)
            gb.mul_(1.5)
        torch.cuda.synchronize()
        for x, y in zip(_state(a.zs), _state(b.zs)):
            assert np.array_equal(_bits(x), _bits(y)), r
    a.close()
    b.close()


@pytest.mark.parametrize("flags", [0, zsm.ZS_STAGE_AVERAGE])
def test_loss_scaled_step_replays_as_consecutive_steps(flags):
    log(f"test_loss_scaled_step_replays_as_consecutive_steps flags={flags}")
    S_total = sum(NUMEL)
    za = ZeroShard(NUMEL, DECAY, 1, 0, 2, fp16=True, flags=flags)
    zb = ZeroShard(NUMEL, DECAY, 1, 0, 2, fp16=True, flags=flags)
    S = za.shard_len
    for z in (za, zb):
        synth.dev_normal_f32(z.master[:S], synth.key(9, 0), 0.02)
        z.amp_init(2.0 ** 12)
    ga = [torch.empty(S, dtype=torch.float16, device="cuda") for _ in range(2)]
    gb = [torch.empty(S, dtype=torch.float16, device="cuda") for _ in range(2)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_grad_norm=1.0,
              growth_interval=2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        za.set_stream(torch.cuda.current_stream().cuda_stream)
        za.step_amp(ga, **hp)
    za.set_stream(torch.cuda.current_stream().cuda_stream)
    zb.set_stream(torch.cuda.current_stream().cuda_stream)
    # the capture itself ran nothing: start both from the same state
    for z in (za, zb):
        synth.dev_normal_f32(z.master[:S], synth.key(9, 0), 0.02)
        z.exp_avg.zero_()
        z.exp_avg_sq.zero_()
        z.amp_init(2.0 ** 12)       # same buffer as at capture time
    for r in range(6):
        for j in range(2):       # fresh gradients, eagerly, between replays
            synth.dev_grad_f16(ga[j], synth.key(9, 10 + 2 * r + j), 1e-3, 2.0 ** 12)
            gb[j].copy_(ga[j])
        if r == 3:               # an overflow: the replay must skip and back off
            ga[1][100] = float("inf")
            gb[1][100] = float("inf")
        g.replay()
        zb.step_amp(gb, **hp)
        torch.cuda.synchronize()
        for x, y in zip(_state(za), _state(zb)):
            assert np.array_equal(_bits(x), _bits(y)), r
        assert za.amp_read() == zb.amp_read()
    scale, tracker, applied = zb.amp_read()
    assert applied == 5            # six replays, one skipped
    assert S_total <= S
    za.close()
    zb.close()
