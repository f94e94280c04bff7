"""GPU parity on seeded random layouts: tensor lists mixing empty, tiny, medium and
large tensors with random weight-decay flags, world sizes 1-16 and any rank,
M = 1..16, tensor alignment 8/64/128, bucket caps small enough to cut many buckets,
clipped and not.  Every case checks the whole shard against the oracle for two
steps, bit for bit (tests/_gpu.py: per-step error from the device's pre-step state,
the oracle's own clip coefficient, a free-running drift trajectory), and the
allocation-free step against the context step on the same layout."""
import numpy as np
import pytest
import torch

import synth
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard
from synth.workloads import scaled, workload

from _gpu import full_parity, log, to_host

pytestmark = pytest.mark.gpu
SEED, COUNT = 0x2AD0_5EED, 64


def _layouts():
    rng = np.random.default_rng(SEED)
    out = []
    for _ in range(COUNT):
        T = int(rng.integers(1, 41))
        kind = rng.integers(0, 4, T)
        sizes = np.select([kind == 0, kind == 1, kind == 2],
                          [rng.integers(0, 3, T), rng.integers(1, 300, T),
                           rng.integers(300, 20_000, T)], rng.integers(20_000, 200_000, T))
        numel = [int(x) for x in sizes]
        numel[int(rng.integers(0, T))] += 1          # never an all-empty model
        decay = [int(x) for x in rng.integers(0, 2, T)]
        N = int(rng.choice([1, 2, 3, 4, 7, 8, 16]))
        out.append(dict(numel=numel, decay=decay, N=N, rank=int(rng.integers(0, N)),
                        M=int(rng.integers(1, 17)), align=int(rng.choice([8, 64, 128])),
                        cap=int(rng.choice([25_000_000, 60_000, 9_000])),
                        clip=float(rng.choice([0.0, 0.0, 0.05, 10.0]))))
    return out


LAYOUTS = _layouts()


def _workload(i):
    c = LAYOUTS[i]
    w = scaled(workload(1), c["numel"], c["decay"], world_size=c["N"], rank=c["rank"],
               M=c["M"], name=f"random{i}")
    w.align, w.bucket_cap, w.max_grad_norm = c["align"], c["cap"], c["clip"]
    return w


def _describe(i):
    c = LAYOUTS[i]
    return (f"case {i}: tensors={len(c['numel'])} total={sum(c['numel']):,} N={c['N']} "
            f"r={c['rank']} M={c['M']} align={c['align']} cap={c['cap']:,} clip={c['clip']}")


@pytest.mark.parametrize("i", range(COUNT))
def test_random_layout_matches_oracle(i):
    log(f"test_random_layout_matches_oracle {_describe(i)}")
    full_parity(_workload(i), 2)


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("i", range(0, COUNT, 4))
def test_random_layout_static_step_equals_context_step(i):
    log(f"test_random_layout_static_step_equals_context_step {_describe(i)}")
    c = LAYOUTS[i]
    kw = dict(bucket_cap=c["cap"], align=c["align"])
    lay = L.plan(c["numel"], c["decay"], c["N"], c["rank"], c["cap"], c["align"])
    ref = ZeroShard(c["numel"], c["decay"], c["N"], c["rank"], c["M"], grad_buffers=True, **kw)
    sta = ZeroShard(c["numel"], c["decay"], c["N"], c["rank"], c["M"], **kw)
    S = ref.shard_len
    assert S == sta.shard_len == lay.shard_len
    master = synth.host_normal_f32(S, synth.key(97, i), 0.02)
    for o, n in lay.padding_ranges():
        master[o:o + n] = 0
    for z in (ref, sta):
        z.master[:S].copy_(torch.from_numpy(master))
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    for step in (1, 2):
        for j in range(c["M"]):
            g = synth.host_grad_bf16(S, synth.key(98, 100 * i + 10 * step + j),
                                     synth.key(99, 100 * i + 10 * step + j), 1e-3)
            for o, n in lay.padding_ranges():
                g[o:o + n] = 0
            ref.grads[j][:S].copy_(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        ref.step(ref.grads, step=step, max_grad_norm=c["clip"], **hp)
        zsm.zero_shard_step_static(sta.plan, c["M"], sta.param.data_ptr(), sta.master.data_ptr(),
                                   sta.exp_avg.data_ptr(), sta.exp_avg_sq.data_ptr(),
                                   [g.data_ptr() for g in ref.grads], step=step,
                                   max_grad_norm=c["clip"],
                                   stream=torch.cuda.current_stream().cuda_stream, **hp)
        torch.cuda.synchronize()
        for x, y, name in zip((sta.master, sta.exp_avg, sta.exp_avg_sq, sta.param),
                              (ref.master, ref.exp_avg, ref.exp_avg_sq, ref.param),
                              ("master", "m", "v", "param")):
            assert np.array_equal(_bits(to_host(x)[:S]), _bits(to_host(y)[:S])), (i, step, name)
    ref.close()
    sta.close()
