"""GPU parity of the fp16 loss-scaled step (ZS_FP16, zero_shard_step_amp) with the
oracle: bit for bit per step, including skipped steps, the device-side scaler
state (scale, growth count, applied steps), every finite fp16 gradient pattern
through the widening, and the fp16 re-cast across its subnormal, tie and
overflow boundaries."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard

from _gpu import log, rel_err, to_host

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _u16(t):
    return torch.from_numpy(np.ascontiguousarray(t).view(np.int16)).cuda()


def _state(z):
    S = z.shard_len
    return [to_host(z.master)[:S], to_host(z.exp_avg)[:S], to_host(z.exp_avg_sq)[:S],
            z.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]]


def _eq(a, b):
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return np.array_equal(a, b)


@pytest.mark.parametrize("stage", [False, True])
@pytest.mark.parametrize("clip", [0.0, 2.0])
def test_amp_sequence_matches_oracle(clip, stage):
    log(f"test_amp_sequence_matches_oracle clip={clip} stage={stage}")
    numel = [70_001, 64, 5, 130_000, 333]
    decay = [1, 0, 0, 1, 0]
    N, rank, M = 3, 1, 3
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    z = ZeroShard(numel, decay, N, rank, M, fp16=True, flags=zsm.ZS_STAGE_AVERAGE if stage else 0)
    S = z.shard_len
    pad = lay.padding_ranges()
    master = synth.host_normal_f32(S, synth.key(77, 0), 0.02)
    for o, n in pad:
        master[o:o + n] = 0
    z.master[:S].copy_(torch.from_numpy(master))
    z.amp_init(2.0 ** 14)
    sc = oracle.Scaler(scale=2.0 ** 14, growth_interval=3)
    p, m, v = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    pf = np.zeros(S, np.uint16)
    mask = lay.decay_mask()
    skips = 0
    for s in range(14):
        scale = float(sc.scale[0])
        gs = []
        for j in range(M):
            g = synth.host_grad_f16(S, synth.key(77, 1 + j + M * s), 1e-3, scale)
            for o, n in pad:
                g[o:o + n] = 0
            gs.append(g)
        if s in (4, 9):
            gs[1][1234] = 0x7C00 if s == 4 else 0x7E00      # Inf, then NaN
        rc, norm = z.step_amp([_u16(g) for g in gs], max_grad_norm=clip, growth_interval=3,
                              want_norm=True, return_code=True, **HP)
        fi, onorm = oracle.amp_step(gs, p, m, v, pf, mask, sc, max_grad_norm=clip, **HP)
        skips += fi
        assert (rc == zsm.ZS_NONFINITE) == fi
        if not fi:
            assert abs(norm - onorm) <= 1e-12 * onorm
        got = _state(z)
        for a, b in zip(got, (p, m, v, pf)):
            assert _eq(a, b), (s, rel_err(a, b) if a.dtype == np.float32 else "param")
        assert z.amp_read() == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied)
    assert skips == 2
    log(f"  14 steps, 2 skipped, final scale {float(sc.scale[0])}, all bit-exact")
    z.close()


def test_fp16_widening_every_finite_pattern():
    log("test_fp16_widening_every_finite_pattern")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (pats & 0x7C00) != 0x7C00
    g = np.where(finite, pats, 0).astype(np.uint16)
    S = g.size
    z = ZeroShard([S], [1], 1, 0, 1, fp16=True)
    z.amp_init(1.0)
    hp = dict(HP, lr=0.0, weight_decay=0.0)
    z.step_amp([_u16(g)], **hp)
    sc = oracle.Scaler(scale=1.0)
    p, m, v, pf = (np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.float32),
                   np.zeros(S, np.uint16))
    oracle.amp_step([g], p, m, v, pf, None, sc, **hp)
    for a, b in zip(_state(z), (p, m, v, pf)):
        assert _eq(a, b)
    z.close()


def test_fp16_recast_boundaries():
    log("test_fp16_recast_boundaries")
    rng = np.random.default_rng(50)
    lo, hi = 0x32000000, 0x48000000             # 2^-27 .. 2^17: fp16 subnormals to overflow
    u = rng.integers(lo, hi, 1 << 20, dtype=np.int64).astype(np.uint32)
    ties = (rng.integers(lo, hi, 1 << 16, dtype=np.int64).astype(np.uint32) & ~np.uint32(0x1FFF)) \
        | np.uint32(0x1000)                      # halfway between two fp16 normals
    u = np.concatenate([u, ties, np.array([0x477FEFFF, 0x477FF000, 0x38800000, 0x387FFFFF,
                                           0x33000000, 0x33000001, 0x33C00000], np.uint32)])
    sign = rng.integers(0, 2, u.size).astype(np.uint32) << 31
    x = (u | sign).view(np.float32)
    S = (x.size + 63) // 64 * 64
    master = np.zeros(S, np.float32)
    master[:x.size] = x
    z = ZeroShard([S], [0], 1, 0, 1, fp16=True)
    z.master.copy_(torch.from_numpy(master))
    z.amp_init(1.0)
    hp = dict(HP, lr=0.0, weight_decay=0.0)
    z.step_amp([torch.zeros(S, dtype=torch.int16, device="cuda")], **hp)
    got = _state(z)
    assert _eq(got[0], master)                   # lr = 0, no decay: master unchanged
    assert np.array_equal(got[3], oracle.f32_to_f16(master))
    z.close()


def test_amp_rejects_wrong_context():
    z = ZeroShard([1000], [1], 1, 0, 1)          # bf16 context
    z.amp_state = torch.zeros(2, dtype=torch.int64, device="cuda")
    with pytest.raises(zsm.ZeroShardError) as e:
        z.step_amp([torch.zeros(1024, dtype=torch.int16, device="cuda")], **HP)
    assert e.value.code == zsm.ZS_ESTATE
    gt = torch.zeros(1024, dtype=torch.int16, device="cuda")
    g = [gt.data_ptr()]
    d = torch.zeros(2, dtype=torch.float64, device="cuda")
    for call in (lambda: zsm.zero_shard_grad_sumsq_amp(z.ctx, g, z.amp_state.data_ptr(),
                                                       d.data_ptr()),
                 lambda: zsm.zero_shard_step_amp_global_norm(
                     z.ctx, g, max_grad_norm=1.0, state_dev=z.amp_state.data_ptr(),
                     global_sumsq_dev=d.data_ptr(), **HP)):
        with pytest.raises(zsm.ZeroShardError) as e:
            call()
        assert e.value.code == zsm.ZS_ESTATE
    z.close()
    y = ZeroShard([1000], [1], 1, 0, 1, fp16=True)
    with pytest.raises(zsm.ZeroShardError) as e:
        y.step([torch.zeros(1024, dtype=torch.int16, device="cuda")], step=1, **HP)
    assert e.value.code == zsm.ZS_ESTATE
    y.amp_init(1024.0)
    st = y.amp_state.data_ptr()
    for bad in (dict(state_dev=st + 8, global_sumsq_dev=d.data_ptr()),      # state alignment
                dict(state_dev=st, global_sumsq_dev=d.data_ptr() + 4),      # sumsq alignment
                dict(state_dev=st, global_sumsq_dev=0)):                    # NULL
        with pytest.raises(zsm.ZeroShardError) as e:
            zsm.zero_shard_step_amp_global_norm(y.ctx, g, max_grad_norm=1.0, **bad, **HP)
        assert e.value.code == zsm.ZS_EINVAL
    with pytest.raises(zsm.ZeroShardError) as e:
        zsm.zero_shard_grad_sumsq_amp(y.ctx, g, st, d.data_ptr() + 4)
    assert e.value.code == zsm.ZS_EINVAL
    assert y.amp_read() == (1024.0, 0, 0)       # rejected calls changed nothing
    y.close()


@pytest.mark.parametrize("stage", [False, True])
def test_gpt13b_shard_amp_full(stage):
    """The loss-scaled step on the GPT-1.3B 1/8 shard (M = 8, the size the benchmark
    times), whole-shard against the oracle for 3 steps, the second with an Inf."""
    from synth.workloads import workload
    w = workload(2)
    log(f"test_gpt13b_shard_amp_full stage={stage}: {w.description}")
    lay = L.plan(w.numel, w.decay, w.world_size, w.rank, w.bucket_cap, w.align)
    z = ZeroShard(w.numel, w.decay, w.world_size, w.rank, w.M, bucket_cap=w.bucket_cap,
                  align=w.align, fp16=True, flags=zsm.ZS_STAGE_AVERAGE if stage else 0)
    S = z.shard_len
    assert S == lay.shard_len
    master = synth.host_normal_f32(S, w.master_key(), w.sigma_master)
    z.master[:S].copy_(torch.from_numpy(master))
    z.amp_init(2.0 ** 14)
    sc = oracle.Scaler(scale=2.0 ** 14, growth_interval=2)
    p, m, v = master, np.zeros(S, np.float32), np.zeros(S, np.float32)
    pf = np.zeros(S, np.uint16)
    mask = lay.decay_mask()
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    for s in range(3):
        scale = float(sc.scale[0])
        gs = [synth.host_grad_f16(S, k, w.sigma_grad, scale) for k, _ in w.grad_keys(s)]
        if s == 1:
            gs[5][S // 2] = 0x7C00
        dev = [_u16(g) for g in gs]
        rc, norm = z.step_amp(dev, growth_interval=2, want_norm=True, return_code=True, **hp)
        fi, onorm = oracle.amp_step(gs, p, m, v, pf, mask, sc, **hp)
        assert (rc == zsm.ZS_NONFINITE) == fi and fi == (s == 1)
        if not fi:
            assert abs(norm - onorm) <= 1e-12 * onorm
        for a, b in zip(_state(z), (p, m, v, pf)):
            assert _eq(a, b), s
        assert z.amp_read() == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied)
        del dev
        log(f"  step {s + 1}: {'skipped' if fi else 'applied'}, bit-exact over {S:,} elements")
    z.close()


def test_amp_empty_shard_keeps_the_scaler_in_step():
    """A rank whose shard is empty still advances its scaler like every other
    rank: the norm of nothing is 0 (finite), and a global value decides the
    multi-rank split."""
    log("test_amp_empty_shard_keeps_the_scaler_in_step")
    z = ZeroShard([0, 0], [1, 1], 2, 1, 2, fp16=True)
    assert z.shard_len == 0
    z.amp_init(1024.0)
    g = torch.zeros(8, dtype=torch.int16, device="cuda")
    for _ in range(2):
        assert z.step_amp([g, g], growth_interval=2, want_norm=True, **HP) == 0.0
    assert z.amp_read() == (2048.0, 0, 2)
    d = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    zsm.zero_shard_grad_sumsq_amp(z.ctx, [g.data_ptr()] * 2, z.amp_state.data_ptr(), d.data_ptr())
    assert d.item() == 0.0
    for total, want in ((4.0, (2048.0, 1, 3)), (float("inf"), (1024.0, 0, 3))):
        d.fill_(total)
        zsm.zero_shard_step_amp_global_norm(z.ctx, [g.data_ptr()] * 2, max_grad_norm=1.0,
                                            state_dev=z.amp_state.data_ptr(), growth_interval=2,
                                            global_sumsq_dev=d.data_ptr(), **HP)
        assert z.amp_read() == want
    z.close()


@pytest.mark.parametrize("start", [float(np.finfo(np.float32).max), 2.0 ** 127])
def test_amp_scale_growth_stays_finite(start):
    """Growth every step from next to the largest finite fp32 scale: a grown scale
    that would be Inf is dropped and the growth count restarts, on the device as
    in the oracle (torch's GradScaler).  Zero gradients keep the steps applied;
    one contribution that overflowed fp16 (Inf) makes a step skip and back the
    scale off."""
    log(f"test_amp_scale_growth_stays_finite start={start}")
    numel, decay = [5000, 64, 3], [1, 0, 1]
    lay = L.plan(numel, decay, 1, 0, 25_000_000, 64)
    z = ZeroShard(numel, decay, 1, 0, 2, fp16=True)
    S = z.shard_len
    master = synth.host_normal_f32(S, synth.key(78, 0), 0.02)
    for o, n in lay.padding_ranges():
        master[o:o + n] = 0
    z.master[:S].copy_(torch.from_numpy(master))
    z.amp_init(start)
    sc = oracle.Scaler(scale=start, growth_interval=1)
    p, m, v = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    pf = np.zeros(S, np.uint16)
    mask = lay.decay_mask()
    for s in range(7):
        gs = [np.zeros(S, np.uint16) for _ in range(2)]
        if s == 3:
            gs[1][17] = 0x7C00        # an overflowed (Inf) fp16 contribution
        z.step_amp([_u16(g) for g in gs], growth_interval=1, **HP)
        fi, _ = oracle.amp_step(gs, p, m, v, pf, mask, sc, **HP)
        assert fi == (s == 3)
        got = _state(z)
        for a, b in zip(got, (p, m, v, pf)):
            assert _eq(a, b), s
        scale, tracker, applied = z.amp_read()
        assert np.isfinite(scale), s
        assert (scale, tracker, applied) == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied), s
    z.close()
