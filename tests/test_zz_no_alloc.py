"""The allocation-free step (zero_shard_step_static) against the context step
(zero_shard_step) through the C ABI: the same seeded inputs through both entry
points give the same bits for master, m, v and the bf16 param, on two calls in
a row (two steps each), the second with a smaller shard, clipped and not.  The
second call reuses the static scratch the first left behind."""
import numpy as np
import pytest
import torch

import synth
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard

from _gpu import log, to_host

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)

CASES = [
    # (numel, decay, N, rank, M, max_grad_norm): a larger shard with several decay
    # runs and a ragged end, clipped; then a smaller one, unclipped
    ([70_001, 64, 5, 2 ** 17 + 8, 333], [1, 0, 0, 1, 0], 2, 1, 5, 0.05),
    ([3000, 64, 7], [1, 0, 1], 1, 0, 3, 0.0),
]


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _state(z):
    S = z.shard_len
    return [to_host(z.master)[:S], to_host(z.exp_avg)[:S], to_host(z.exp_avg_sq)[:S],
            to_host(z.param)[:S]]


def test_static_step_equals_context_step():
    for case, (numel, decay, N, rank, M, clip) in enumerate(CASES):
        log(f"test_static_step_equals_context_step case {case}: tensors={len(numel)} N={N} "
            f"r={rank} M={M} clip={clip}")
        lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
        ref = ZeroShard(numel, decay, N, rank, M, grad_buffers=True)   # the context step
        sta = ZeroShard(numel, decay, N, rank, M)                      # buffers for the static one
        S = ref.shard_len
        assert S == sta.shard_len == lay.shard_len
        master = synth.host_normal_f32(S, synth.key(91, case), 0.02)
        for o, n in lay.padding_ranges():
            master[o:o + n] = 0
        for z in (ref, sta):
            z.master[:S].copy_(torch.from_numpy(master))
        for step in (1, 2):
            for j in range(M):
                g = synth.host_grad_bf16(S, synth.key(92, 100 * case + 10 * step + j),
                                         synth.key(93, 100 * case + 10 * step + j), 1e-3)
                for o, n in lay.padding_ranges():
                    g[o:o + n] = 0
                ref.grads[j][:S].copy_(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16))
            torch.cuda.synchronize()
            ptrs = [g.data_ptr() for g in ref.grads]
            ref.step(ref.grads, step=step, max_grad_norm=clip, **HP)
            zsm.zero_shard_step_static(sta.plan, M, sta.param.data_ptr(), sta.master.data_ptr(),
                                       sta.exp_avg.data_ptr(), sta.exp_avg_sq.data_ptr(), ptrs,
                                       step=step, max_grad_norm=clip,
                                       stream=torch.cuda.current_stream().cuda_stream, **HP)
            torch.cuda.synchronize()
            for a, b, name in zip(_state(sta), _state(ref), ("master", "m", "v", "param")):
                assert np.array_equal(_bits(a), _bits(b)), (case, step, name)
        log(f"  case {case}: S={S:,}, 2 steps bit-identical to zero_shard_step")
        ref.close()
        sta.close()
