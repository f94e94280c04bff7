"""The multi-rank split of the clipped and of the loss-scaled step, on one GPU.

N ranks are simulated as N contexts, each over its own shard of one model (its
own plan for rank r of N): device contexts (fused and with the staged average)
and offload contexts (the update on host cores).  Per step every rank enqueues
part 1 (its shard's sum of squares); the scalar all-reduce that a real job
would run over the ranks is a fixed-order sum of the N device doubles; every
rank then runs part 2 with that global value.  The shards, mapped back tensor
by tensor, must equal the unsharded oracle run over the whole model bit for
bit: the same clip coefficient, the same skip decision and the same scaler
state on every rank.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroOffload, ZeroShard

from _gpu import assert_within_tolerance, coef_ulps, log, to_host

pytestmark = pytest.mark.gpu

NUMEL = [70_001, 64, 5, 30_000, 333, 4096, 1]
DECAY = [1, 0, 0, 1, 0, 1, 0]
N, M, CAP = 3, 2, 40_000
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _scatter(lay, per_tensor, dtype):
    """Per-tensor arrays -> this layout's shard (padding zero)."""
    out = np.zeros(lay.shard_len, dtype)
    for s in lay.segments:
        if s.tensor >= 0:
            out[s.shard_off:s.shard_off + s.length] = \
                per_tensor[s.tensor][s.tensor_off:s.tensor_off + s.length]
    return out


def _gather(lays, shards, numel, dtype):
    """Shards of all ranks -> per-tensor arrays."""
    out = [np.zeros(n, dtype) for n in numel]
    for lay, x in zip(lays, shards):
        for s in lay.segments:
            if s.tensor >= 0:
                out[s.tensor][s.tensor_off:s.tensor_off + s.length] = \
                    x[s.shard_off:s.shard_off + s.length]
    return out


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


VARIANTS = ["device", "device_staged", "offload"]

# part 1 and part 2 of the split, by context kind
SUMSQ = {"device": zsm.zero_shard_grad_sumsq, "offload": zsm.zero_offload_grad_sumsq}
STEP = {"device": zsm.zero_shard_step_global_norm, "offload": zsm.zero_offload_step_global_norm}
SUMSQ_AMP = {"device": zsm.zero_shard_grad_sumsq_amp, "offload": zsm.zero_offload_grad_sumsq_amp}
STEP_AMP = {"device": zsm.zero_shard_step_amp_global_norm,
            "offload": zsm.zero_offload_step_amp_global_norm}


def _kind(variant):
    return "offload" if variant == "offload" else "device"


def _setup(fp16, variant):
    lays = [L.plan(NUMEL, DECAY, N, r, CAP, 64) for r in range(N)]
    one = L.plan(NUMEL, DECAY, 1, 0, CAP, 64)
    if variant == "offload":   # small chunks: the host pipeline runs many of them
        zs = [ZeroOffload(NUMEL, DECAY, N, r, M, bucket_cap=CAP, fp16=fp16, chunk_elems=8192)
              for r in range(N)]
    else:
        flags = zsm.ZS_STAGE_AVERAGE if variant == "device_staged" else 0
        zs = [ZeroShard(NUMEL, DECAY, N, r, M, bucket_cap=CAP, fp16=fp16, flags=flags)
              for r in range(N)]
    master_t = [synth.host_normal_f32(n, synth.key(31, t), 0.02) for t, n in enumerate(NUMEL)]
    for lay, z in zip(lays, zs):
        assert z.shard_len == lay.shard_len
        z.master[:lay.shard_len].copy_(torch.from_numpy(_scatter(lay, master_t, np.float32)))
    ref = dict(p=_scatter(one, master_t, np.float32), m=np.zeros(one.shard_len, np.float32),
               v=np.zeros(one.shard_len, np.float32), b=np.zeros(one.shard_len, np.uint16))
    return lays, one, zs, ref


def _check(lays, one, zs, ref, step, exact=True):
    """The shards mapped back tensor by tensor against the unsharded oracle: bit for
    bit, or (exact=False) within the stated tolerance."""
    got_all, want_all = [], []
    for key, dev, dt in (("p", "master", np.float32), ("m", "exp_avg", np.float32),
                         ("v", "exp_avg_sq", np.float32), ("b", "param", np.uint16)):
        shards = [to_host(getattr(z, dev))[:lay.shard_len] if dt == np.float32 else
                  getattr(z, dev).cpu().view(torch.int16).numpy().view(np.uint16)[:lay.shard_len]
                  for lay, z in zip(lays, zs)]
        got = _gather(lays, shards, NUMEL, dt)
        want = _gather([one], [ref[key]], NUMEL, dt)
        if exact:
            for t in range(len(NUMEL)):
                assert np.array_equal(_bits(got[t]), _bits(want[t])), (step, key, t)
        got_all.append(np.concatenate(got))
        want_all.append(np.concatenate(want))
    assert_within_tolerance(step, got_all, want_all)


@pytest.mark.parametrize("variant", VARIANTS)
def test_bf16_clip_split_over_ranks_equals_unsharded(variant):
    log(f"test_bf16_clip_split_over_ranks_equals_unsharded {variant}")
    lays, one, zs, ref = _setup(False, variant)
    kind = _kind(variant)
    part = torch.zeros(N, dtype=torch.float64, device="cuda")
    glob = torch.zeros(1, dtype=torch.float64, device="cuda")
    mask = one.decay_mask()
    same = True      # the device's coefficient has equalled the oracle's on every step so far
    for s in range(4):
        grads_t = [[synth.host_grad_bf16(n, synth.key(32, 100 * s + 10 * j + t),
                                         synth.key(33, 100 * s + 10 * j + t), 1e-3)
                    for t, n in enumerate(NUMEL)] for j in range(M)]
        dev = [[_u16(_scatter(lay, grads_t[j], np.uint16)) for j in range(M)] for lay in lays]
        for r, z in enumerate(zs):
            SUMSQ[kind](z.ctx, [g.data_ptr() for g in dev[r]], part[r:r + 1].data_ptr())
        glob.copy_(part[0:1] + part[1:2] + part[2:3])        # the scalar all-reduce
        max_norm = 0.02 if s % 2 else 1e3                    # binding, then not
        for r, z in enumerate(zs):
            STEP[kind](z.ctx, [g.data_ptr() for g in dev[r]], step=s + 1,
                       max_grad_norm=max_norm, global_sumsq_dev=glob.data_ptr(), **HP)
        torch.cuda.synchronize()
        g_one = [_scatter(one, grads_t[j], np.uint16) for j in range(M)]
        sumsq = oracle.grad_sumsq(g_one)
        want = float(np.sqrt(sumsq))
        norm = float(np.sqrt(glob.item()))
        assert abs(norm - want) <= 1e-12 * want
        coef = oracle.clip_coef(sumsq, max_norm)       # the oracle's own coefficient
        ulps = coef_ulps(oracle.coef_from_norm(norm, max_norm), coef)
        assert ulps <= 1
        same = same and ulps == 0
        assert (coef < 1) == bool(s % 2)
        oracle.step_f32(g_one, ref["p"], ref["m"], ref["v"], ref["b"], mask, step=s + 1,
                        coef=coef, **HP)
        _check(lays, one, zs, ref, s, exact=same)
    for z in zs:
        z.close()


@pytest.mark.parametrize("variant", VARIANTS)
def test_amp_split_over_ranks_equals_unsharded(variant):
    log(f"test_amp_split_over_ranks_equals_unsharded {variant}")
    lays, one, zs, ref = _setup(True, variant)
    kind = _kind(variant)
    for z in zs:
        z.amp_init(2.0 ** 12)
    sc = oracle.Scaler(scale=2.0 ** 12, growth_interval=2)
    part = torch.zeros(N, dtype=torch.float64, device="cuda")
    glob = torch.zeros(1, dtype=torch.float64, device="cuda")
    mask = one.decay_mask()
    skips = 0
    for s in range(7):
        scale = float(sc.scale[0])
        grads_t = [[synth.host_grad_f16(n, synth.key(34, 100 * s + 10 * j + t), 1e-3, scale)
                    for t, n in enumerate(NUMEL)] for j in range(M)]
        if s in (2, 5):   # an overflow in one tensor of one contribution: every rank skips
            grads_t[1][3][123] = 0x7C00 if s == 2 else 0xFE00
        dev = [[_u16(_scatter(lay, grads_t[j], np.uint16)) for j in range(M)] for lay in lays]
        for r, z in enumerate(zs):
            SUMSQ_AMP[kind](z.ctx, [g.data_ptr() for g in dev[r]], z.amp_state.data_ptr(),
                            part[r:r + 1].data_ptr())
        glob.copy_(part[0:1] + part[1:2] + part[2:3])
        clip = 0.01 if s % 2 else 0.0
        for r, z in enumerate(zs):
            STEP_AMP[kind](z.ctx, [g.data_ptr() for g in dev[r]], max_grad_norm=clip,
                           state_dev=z.amp_state.data_ptr(), growth_interval=2,
                           global_sumsq_dev=glob.data_ptr(), **HP)
        torch.cuda.synchronize()
        g_one = [_scatter(one, grads_t[j], np.uint16) for j in range(M)]
        fi, onorm = oracle.amp_step(g_one, ref["p"], ref["m"], ref["v"], ref["b"], mask, sc,
                                    max_grad_norm=clip, **HP)
        skips += fi
        assert fi == (s in (2, 5))
        total = glob.item()
        assert (not np.isfinite(total)) == fi
        if not fi:
            assert abs(np.sqrt(total) - onorm) <= 1e-12 * onorm
        _check(lays, one, zs, ref, s)
        for z in zs:
            assert z.amp_read() == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied), s
    assert skips == 2
    for z in zs:
        z.close()
