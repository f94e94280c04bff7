"""GPU edge cases through the C ABI: empty shard, non-finite gradients with and
without ZS_SKIP_NONFINITE, run-to-run determinism, the two-call global-norm
API against the single call, a non-default stream, rejected arguments."""
import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard
from synth.workloads import scaled, workload

from _gpu import Shard, log, to_host

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _state(zs):
    return [to_host(x)[:zs.shard_len].copy() for x in (zs.master, zs.exp_avg, zs.exp_avg_sq,
                                                       zs.param)]


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _small(numel=(5000, 64, 130_001, 7), decay=(1, 0, 1, 0), N=2, rank=1, M=3):
    return scaled(workload(1), list(numel), list(decay), world_size=N, rank=rank, M=M,
                  name="edge")


def test_empty_shard():
    log("test_empty_shard")
    zs = ZeroShard([0, 0, 0], [1, 0, 1], world_size=4, rank=2, M=2)
    assert zs.shard_len == 0
    g = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    assert zs.step([g, g], step=1, max_grad_norm=1.0, want_norm=True, **HP) == 0.0
    assert zs.step([g, g], step=2, **HP) is None
    zs.close()


@pytest.mark.parametrize("skip", [False, True])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("clip", [0.0, 0.5])
def test_nonfinite_gradient(skip, bad, clip):
    log(f"test_nonfinite_gradient skip={skip} bad={bad} clip={clip}")
    w = _small()
    w.max_grad_norm = clip
    sh = Shard(w, flags=zsm.ZS_SKIP_NONFINITE if skip else 0)
    S = sh.S
    # one clean step, then a step with one non-finite gradient element
    sh.step(0)
    torch.cuda.synchronize()
    grads = sh.case.fill_grads(1)
    pos = 4321
    row = torch.tensor([bad], dtype=torch.float32).to(torch.bfloat16)
    grads[1][pos] = row.to(grads[1].device)[0]
    pre = _state(sh.zs)
    rc, norm = sh.zs.step(grads, step=2, max_grad_norm=clip, want_norm=True, return_code=True,
                          **sh.hp())
    torch.cuda.synchronize()
    assert rc == zsm.ZS_NONFINITE and not np.isfinite(norm)
    got = _state(sh.zs)
    if skip:
        for a, b in zip(got, pre):
            assert np.array_equal(_bits(a), _bits(b))   # left untouched
    else:
        g = [to_host(x)[:S].copy() for x in grads]
        # the oracle's own coefficient (NaN or 0 here, as the device's)
        coef = oracle.clip_coef(oracle.grad_sumsq(g), clip) if clip > 0 else None
        p, m, v, _ = [x.copy() for x in pre]
        b = np.zeros(S, np.uint16)
        oracle.step_f32(g, p, m, v, b, sh.lay.decay_mask(), step=2, coef=coef, **sh.hp())
        for a, want in zip(got, (p, m, v, b)):
            nan_a = np.isnan(a) if a.dtype == np.float32 else ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
            nan_w = np.isnan(want) if want.dtype == np.float32 else ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
            assert np.array_equal(nan_a, nan_w)
            assert np.array_equal(_bits(a)[~nan_a], _bits(want)[~nan_w])
    sh.close()


def test_deterministic_across_runs():
    log("test_deterministic_across_runs")
    w = workload(5)
    w = scaled(w, w.numel[:600], w.decay[:600], M=4, name="stress-prefix")
    w.max_grad_norm = 1.0
    outs = []
    for _ in range(2):
        sh = Shard(w)
        norms = [sh.step(s, want_norm=True) for s in range(3)]
        torch.cuda.synchronize()
        outs.append((norms, _state(sh.zs)))
        sh.close()
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(_bits(a), _bits(b))


def test_global_norm_api_equals_single_call():
    log("test_global_norm_api_equals_single_call")
    w = _small(M=5)
    w.max_grad_norm = 0.3
    a, b = Shard(w), Shard(w)
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for s in range(3):
        na = a.step(s, want_norm=True)
        grads = b.case.fill_grads(s)
        ptrs = [g.data_ptr() for g in grads]
        zsm.zero_shard_grad_sumsq(b.zs.ctx, ptrs, sumsq.data_ptr())
        zsm.zero_shard_step_global_norm(b.zs.ctx, ptrs, step=s + 1, max_grad_norm=0.3,
                                        global_sumsq_dev=sumsq.data_ptr(), **b.hp())
        torch.cuda.synchronize()
        assert float(np.sqrt(sumsq.item())) == na
        want = oracle.grad_sumsq(b.case.host_grads(s))
        assert abs(sumsq.item() - want) <= 1e-12 * want
    for x, y in zip(_state(a.zs), _state(b.zs)):
        assert np.array_equal(_bits(x), _bits(y))
    a.close()
    b.close()


def test_non_default_stream():
    log("test_non_default_stream")
    w = _small(M=2)
    a, b = Shard(w), Shard(w)
    side = torch.cuda.Stream()
    b.zs.set_stream(side.cuda_stream)
    for s in range(2):
        a.step(s)
        grads = b.case.fill_grads(s)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            b.zs.step(grads, step=s + 1, **b.hp())
        side.synchronize()
    torch.cuda.synchronize()
    for x, y in zip(_state(a.zs), _state(b.zs)):
        assert np.array_equal(_bits(x), _bits(y))
    a.close()
    b.close()


@pytest.mark.parametrize("bad", [dict(lr=-1.0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0),
                                 dict(weight_decay=float("nan")), dict(step=0)])
def test_rejected_arguments_leave_state_untouched(bad):
    w = _small(M=2)
    sh = Shard(w)
    sh.step(0)
    torch.cuda.synchronize()
    pre = _state(sh.zs)
    args = dict(sh.hp(), step=2)
    args.update(bad)
    with pytest.raises(zsm.ZeroShardError) as e:
        sh.zs.step(sh.case.fill_grads(1), **args)
    assert e.value.code == zsm.ZS_EINVAL
    torch.cuda.synchronize()
    for x, y in zip(_state(sh.zs), pre):
        assert np.array_equal(_bits(x), _bits(y))
    sh.close()


def test_two_contexts_on_two_streams_concurrently():
    """Contexts share no library state: two shards stepping at once on two streams
    give the same bits as each stepping alone."""
    log("test_two_contexts_on_two_streams_concurrently")
    wa = _small(M=3)
    wb = _small(numel=(70_001, 3, 4096), decay=(1, 0, 1), N=1, rank=0, M=5)
    wa.max_grad_norm = 0.4
    runs = {}
    for concurrent in (False, True):
        a, b = Shard(wa), Shard(wb)
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        a.zs.set_stream(sa.cuda_stream)
        b.zs.set_stream(sb.cuda_stream)
        ga = [[g.clone() for g in a.case.fill_grads(s)] for s in range(3)]
        gb = [[g.clone() for g in b.case.fill_grads(s)] for s in range(3)]
        torch.cuda.synchronize()
        for s in range(3):
            a.zs.step(ga[s], step=s + 1, max_grad_norm=0.4, **a.hp())
            if not concurrent:
                torch.cuda.synchronize()
            b.zs.step(gb[s], step=s + 1, max_grad_norm=0.0, **b.hp())
        torch.cuda.synchronize()
        runs[concurrent] = (_state(a.zs), _state(b.zs))
        a.close()
        b.close()
    for x, y in zip(runs[False][0] + runs[False][1], runs[True][0] + runs[True][1]):
        assert np.array_equal(_bits(x), _bits(y))


@pytest.mark.parametrize("cap", ["3", "64", "0"])
def test_wave_cap_override_keeps_results(monkeypatch, cap):
    """ZS_WAVES_PER_CU at its extremes -- 3 (the largest LDS reservation any launch
    makes, 54,528 B per workgroup), 64 and 0 (no cap) -- passes the context's LDS check
    and changes only how many waves reside, never a result: clipped steps on the
    fused and the staged context stay bit-identical to the oracle."""
    monkeypatch.setenv("ZS_WAVES_PER_CU", cap)
    log(f"test_wave_cap_override_keeps_results cap={cap}")
    for flags in (0, zsm.ZS_STAGE_AVERAGE):
        w = _small(M=5)
        w.max_grad_norm = 0.3
        sh = Shard(w, flags=flags)
        S = sh.S
        mask = sh.lay.decay_mask()
        p, m, v = sh.case.host_master(), np.zeros(S, np.float32), np.zeros(S, np.float32)
        b = np.zeros(S, np.uint16)
        for s in range(2):
            sh.step(s)
            g = sh.case.host_grads(s)
            coef = oracle.clip_coef(oracle.grad_sumsq(g), w.max_grad_norm)
            oracle.step_f32(g, p, m, v, b, mask, step=s + 1, coef=coef, **sh.hp())
        torch.cuda.synchronize()
        for a, want in zip(_state(sh.zs), (p, m, v, b)):
            assert np.array_equal(_bits(a), _bits(want)), (cap, flags)
        sh.close()
