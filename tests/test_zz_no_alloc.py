"""The allocation-free step (zero_shard_step_static) against the context step
(zero_shard_step) through the C ABI: the same seeded inputs through both entry
points give the same bits for master, m, v and the bf16 param, on two calls in
a row (two steps each), each shard smaller than the one before, clipped and not;
every call reuses the static scratch the one before left behind.  The same step
captured in a HIP graph and replayed, with eager work and synchronisations
between the replays, matches the eager context step after every replay; on
non-finite contributions the static step does what a flags-0 context does; and at
the largest clipped shard the scratch holds it still matches, while one tile more
is refused."""
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
    # (numel, decay, N, rank, M, max_grad_norm, align): a larger shard with several
    # decay runs and a ragged end, clipped; 320 small tensors alternating decay (321
    # runs: a run table of three kernel-argument launches, runs starting inside
    # tiles); then a smaller shard, unclipped
    ([70_001, 64, 5, 2 ** 17 + 8, 333], [1, 0, 0, 1, 0], 2, 1, 5, 0.05, 64),
    ([3, 9, 1, 17, 2, 40, 5, 8] * 40, [1, 0] * 160, 1, 0, 2, 0.3, 8),
    ([3000, 64, 7], [1, 0, 1], 1, 0, 3, 0.0, 64),
]


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _state(z):
    S = z.shard_len
    return [to_host(z.master)[:S], to_host(z.exp_avg)[:S], to_host(z.exp_avg_sq)[:S],
            to_host(z.param)[:S]]


def test_static_step_equals_context_step():
    for case, (numel, decay, N, rank, M, clip, align) in enumerate(CASES):
        log(f"test_static_step_equals_context_step case {case}: tensors={len(numel)} N={N} "
            f"r={rank} M={M} clip={clip} align={align}")
        lay = L.plan(numel, decay, N, rank, 25_000_000, align)
        ref = ZeroShard(numel, decay, N, rank, M, align=align, grad_buffers=True)  # context step
        sta = ZeroShard(numel, decay, N, rank, M, align=align)  # buffers for the static one
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


def test_static_step_replayed_from_a_graph():
    """Two static steps captured once in a HIP graph (torch's graph API on a side
    stream) and replayed four times, with eager work and a synchronisation between
    replays: after every replay master, m, v and the param equal those of a context
    that took the same two steps eagerly each time."""
    numel, decay, N, rank, M, clip = [5000, 64, 70_001, 7], [1, 0, 1, 0], 2, 1, 3, 0.4
    log("test_static_step_replayed_from_a_graph")
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    ref = ZeroShard(numel, decay, N, rank, M, grad_buffers=True)
    sta = ZeroShard(numel, decay, N, rank, M)
    S = ref.shard_len
    master = synth.host_normal_f32(S, synth.key(94, 0), 0.02)
    for o, n in lay.padding_ranges():
        master[o:o + n] = 0
    for z in (ref, sta):
        z.master[:S].copy_(torch.from_numpy(master))
    for j in range(M):
        g = synth.host_grad_bf16(S, synth.key(95, j), synth.key(96, j), 1e-3)
        for o, n in lay.padding_ranges():
            g[o:o + n] = 0
        ref.grads[j][:S].copy_(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16))
    ptrs = [g.data_ptr() for g in ref.grads]
    # the first call on a device resolves the scratch and queries the device: make it
    # outside the capture (an eager step on a throwaway shard)
    w0 = ZeroShard([256], [1], 1, 0, 1, grad_buffers=True)
    zsm.zero_shard_step_static(w0.plan, 1, w0.param.data_ptr(), w0.master.data_ptr(),
                               w0.exp_avg.data_ptr(), w0.exp_avg_sq.data_ptr(),
                               [w0.grads[0].data_ptr()], step=1, **HP)
    torch.cuda.synchronize()
    w0.close()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        s = torch.cuda.current_stream().cuda_stream
        for step in (1, 2):
            zsm.zero_shard_step_static(sta.plan, M, sta.param.data_ptr(), sta.master.data_ptr(),
                                       sta.exp_avg.data_ptr(), sta.exp_avg_sq.data_ptr(), ptrs,
                                       step=step, max_grad_norm=clip, stream=s, **HP)
    other = torch.ones(1 << 20, device="cuda")
    for replay in range(4):
        graph.replay()
        for step in (1, 2):
            ref.step(ref.grads, step=step, max_grad_norm=clip, **HP)
        other.mul_(1.5).add_(0.25)          # the program's own eager work between replays
        torch.cuda.synchronize()
        for a, b, name in zip(_state(sta), _state(ref), ("master", "m", "v", "param")):
            assert np.array_equal(_bits(a), _bits(b)), (replay, name)
    log("  4 replays, each bit-identical to the eager context steps")
    ref.close()
    sta.close()


def test_static_step_with_nonfinite_gradient_matches_flags0_context():
    """A clipped step whose contributions hold an Inf and a NaN: the static step does
    what a context made with flags 0 does (the non-finite norm is not skipped), bit
    for bit, including the non-finite results."""
    numel, decay, N, rank, M, clip = [4097, 64, 9000], [1, 0, 1], 1, 0, 2, 1.0
    log("test_static_step_with_nonfinite_gradient_matches_flags0_context")
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    ref = ZeroShard(numel, decay, N, rank, M, grad_buffers=True)
    sta = ZeroShard(numel, decay, N, rank, M)
    S = ref.shard_len
    master = synth.host_normal_f32(S, synth.key(97, 0), 0.02)
    for o, n in lay.padding_ranges():
        master[o:o + n] = 0
    for z in (ref, sta):
        z.master[:S].copy_(torch.from_numpy(master))
    for j in range(M):
        g = synth.host_grad_bf16(S, synth.key(98, j), synth.key(99, j), 1e-3)
        for o, n in lay.padding_ranges():
            g[o:o + n] = 0
        if j == 1:
            g[5] = 0x7F80                    # +Inf in the first tensor
            g[4224 + 100] = 0x7FC1           # a quiet NaN in the third (which starts at 4224)
        ref.grads[j][:S].copy_(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16))
    torch.cuda.synchronize()
    ptrs = [g.data_ptr() for g in ref.grads]
    for step in (1, 2):
        ref.step(ref.grads, step=step, max_grad_norm=clip, **HP)
        zsm.zero_shard_step_static(sta.plan, M, sta.param.data_ptr(), sta.master.data_ptr(),
                                   sta.exp_avg.data_ptr(), sta.exp_avg_sq.data_ptr(), ptrs,
                                   step=step, max_grad_norm=clip,
                                   stream=torch.cuda.current_stream().cuda_stream, **HP)
        torch.cuda.synchronize()
        st = _state(sta)
        assert not np.isfinite(st[0]).all()  # the non-finite norm reached the state
        for a, b, name in zip(st, _state(ref), ("master", "m", "v", "param")):
            assert np.array_equal(_bits(a), _bits(b)), (step, name)
    log(f"  S={S:,}: 2 clipped steps on non-finite contributions, bit-identical")
    ref.close()
    sta.close()


# The largest clipped single-run shard whose norm partials fit the static scratch:
# 2^20 - 192 tiles of 2,048 elements (one fp64 partial per tile, plus one per 8,192 of
# those, plus the 256-byte run table and 256 bytes of clip scalars: 8 MiB exactly).
S_MAX_CLIPPED = ((1 << 20) - 192) * 2048


def test_static_step_at_the_largest_clipped_shard_its_scratch_holds():
    """At 2,147,090,432 elements a clipped static step fills the 8 MiB scratch exactly
    and equals the context step bit for bit; one 2,048-element tile more is refused with
    ZS_EINVAL before anything is enqueued (the buffers passed there are large enough for
    that shard anyway)."""
    S = S_MAX_CLIPPED
    assert zsm.ZS_STATIC_SCRATCH_BYTES == 8 << 20
    log(f"test_static_step_at_the_largest_clipped_shard_its_scratch_holds: S={S:,} M=1 clip=1.0")
    ref = ZeroShard([S], [1], 1, 0, 1, grad_buffers=True)
    big = ZeroShard([S + 2048], [1], 1, 0, 1)        # the static step's buffers
    assert ref.shard_len == S and big.shard_len == S + 2048
    synth.dev_normal_f32(ref.master[:S], synth.key(101, 0), 0.02)
    synth.dev_grad_bf16(ref.grads[0][:S], synth.key(102, 0), synth.key(103, 0), 1e-3)
    big.master[:S].copy_(ref.master[:S])
    torch.cuda.synchronize()
    g = [ref.grads[0].data_ptr()]
    s = torch.cuda.current_stream().cuda_stream
    for step in (1, 2):
        ref.step(ref.grads, step=step, max_grad_norm=1.0, **HP)
        zsm.zero_shard_step_static(ref.plan, 1, big.param.data_ptr(), big.master.data_ptr(),
                                   big.exp_avg.data_ptr(), big.exp_avg_sq.data_ptr(), g,
                                   step=step, max_grad_norm=1.0, stream=s, **HP)
        torch.cuda.synchronize()
        for a, b, name in ((big.master, ref.master, "master"), (big.exp_avg, ref.exp_avg, "m"),
                           (big.exp_avg_sq, ref.exp_avg_sq, "v"), (big.param, ref.param, "param")):
            ia = a[:S].view(torch.int32 if a.element_size() == 4 else torch.int16)
            ib = b[:S].view(torch.int32 if b.element_size() == 4 else torch.int16)
            assert torch.equal(ia, ib), (step, name)
    with pytest.raises(zsm.ZeroShardError) as e:
        zsm.zero_shard_step_static(big.plan, 1, big.param.data_ptr(), big.master.data_ptr(),
                                   big.exp_avg.data_ptr(), big.exp_avg_sq.data_ptr(),
                                   [big.master.data_ptr()], step=3, max_grad_norm=1.0,
                                   stream=s, **HP)
    assert e.value.code == zsm.ZS_EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    log("  2 clipped steps bit-identical at the limit; one tile more refused")
    ref.close()
    big.close()
