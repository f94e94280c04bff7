"""GPU + host: the offloaded step (zero_offload_step) against the oracle, bit for
bit -- host master/m/v and the bf16 params that come back to the device -- on
multi-tensor layouts with many chunks and ragged tails, with clip, with a
non-finite gradient under ZS_SKIP_NONFINITE, on the GPT-1.3B shard, and against
the all-device step on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sharded_optimizer_step_zero_amd as zsm
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroOffload, ZeroShard
from synth.device_case import DeviceCase
from synth.workloads import scaled, workload

from _gpu import assert_within_tolerance, coef_ulps, log, to_host

pytestmark = pytest.mark.gpu


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


class Off:
    def __init__(self, w, chunk, flags=0, n_threads=0):
        self.w = w
        self.lay = L.plan(w.numel, w.decay, w.world_size, w.rank, w.bucket_cap, w.align)
        self.z = ZeroOffload(w.numel, w.decay, w.world_size, w.rank, w.M, bucket_cap=w.bucket_cap,
                             align=w.align, flags=flags, chunk_elems=chunk, n_threads=n_threads)
        self.S = self.z.shard_len
        assert self.S == self.lay.shard_len
        self.case = DeviceCase(w, self.S, self.lay.padding_ranges(), self.z.device)
        self.z.master[:self.S] = torch.from_numpy(self.case.host_master())

    def hp(self):
        w = self.w
        return dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)

    def state(self):
        S = self.S
        torch.cuda.synchronize()
        return [self.z.master[:S].numpy().copy(), self.z.exp_avg[:S].numpy().copy(),
                self.z.exp_avg_sq[:S].numpy().copy(), to_host(self.z.param)[:S].copy()]


def _run_vs_oracle(w, steps, chunk, n_threads=0):
    o = Off(w, chunk, n_threads=n_threads)
    S = o.S
    p, m, v, b = o.case.host_master(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
        np.zeros(S, np.uint16)
    mask = o.lay.decay_mask()
    same = True      # the device's coefficient has equalled the oracle's on every step so far
    for s in range(steps):
        grads = o.case.fill_grads(s)
        norm = o.z.step(grads, step=s + 1, max_grad_norm=w.max_grad_norm, want_norm=True,
                        **o.hp())
        g = o.case.host_grads(s)
        sumsq = oracle.grad_sumsq(g)
        want = float(np.sqrt(sumsq))
        assert abs(norm - want) <= 1e-12 * max(want, 1e-300)
        coef = None
        if w.max_grad_norm > 0:
            coef = oracle.clip_coef(sumsq, w.max_grad_norm)    # the oracle's own
            ulps = coef_ulps(oracle.coef_from_norm(norm, w.max_grad_norm), coef)
            assert ulps <= 1
            same = same and ulps == 0
        oracle.step_f32(g, p, m, v, b, mask, step=s + 1, coef=coef, **o.hp())
        got = o.state()
        assert_within_tolerance(s, got, (p, m, v, b))
        if same:
            for x, y in zip(got, (p, m, v, b)):
                assert np.array_equal(_bits(x), _bits(y)), s
    o.z.close()


CASES = [
    # (numel, decay, N, rank, M, clip, chunk)
    ([1, 63, 64, 65, 1000, 0, 4097, 12_345, 7, 300_001, 3], None, 3, 1, 3, 0.0, 4096),
    ([5000] * 7 + [1], None, 8, 7, 8, 0.05, 64),
    ([70_001, 64, 5, 2 ** 17 + 8], [1, 0, 0, 1], 1, 0, 5, 0.0, 1 << 20),
    ([33_333] * 5, [0, 1, 0, 1, 0], 2, 0, 16, 1e-4, 12_288),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_offload_matches_oracle(case):
    numel, decay, N, rank, M, clip, chunk = CASES[case]
    w = scaled(workload(1), numel, decay, world_size=N, rank=rank, M=M, name=f"offload{case}")
    w.max_grad_norm = clip
    log(f"test_offload_matches_oracle[{case}]: tensors={len(numel)} N={N} M={M} clip={clip} "
        f"chunk={chunk}")
    _run_vs_oracle(w, 4, chunk, n_threads=[0, 1, 5, 16][case])


@pytest.mark.parametrize("groups", ["1", "5"])
@pytest.mark.parametrize("case", [0, 3])
def test_offload_sliced_norm_pass_matches_oracle(monkeypatch, case, groups):
    """The device norm pass of an offload context issued as launches of 1 or 5
    work-groups (ZS_MAX_GROUPS_PER_LAUNCH, read at init), clip and norm included."""
    monkeypatch.setenv("ZS_MAX_GROUPS_PER_LAUNCH", groups)
    numel, decay, N, rank, M, clip, chunk = CASES[case]
    w = scaled(workload(1), numel, decay, world_size=N, rank=rank, M=M, name=f"offload{case}")
    w.max_grad_norm = clip
    log(f"test_offload_sliced_norm_pass_matches_oracle[{case}] groups={groups}")
    _run_vs_oracle(w, 3, chunk)


def test_gpt13b_shard_offload():
    w = workload(2)
    log(f"test_gpt13b_shard_offload: {w.description}, 3 steps, chunk 4M")
    _run_vs_oracle(w, 3, 1 << 22)


def test_offload_equals_device_step_and_skips_nonfinite():
    log("test_offload_equals_device_step_and_skips_nonfinite")
    w = scaled(workload(1), [5000, 64, 130_001, 7], [1, 0, 1, 0], world_size=2, rank=1, M=4,
               name="offload-vs-device")
    o = Off(w, 8192, flags=zsm.ZS_SKIP_NONFINITE)
    d = ZeroShard(w.numel, w.decay, 2, 1, 4, flags=zsm.ZS_SKIP_NONFINITE)
    d.master.copy_(o.z.master.to(d.master.device))
    for s in range(4):
        grads = o.case.fill_grads(s)
        if s == 2:
            grads[3][999] = torch.tensor(float("inf"), dtype=torch.bfloat16)
        ro = o.z.step(grads, step=s + 1, max_grad_norm=0.7, want_norm=True, return_code=True,
                      **o.hp())
        rd = d.step(grads, step=s + 1, max_grad_norm=0.7, want_norm=True, return_code=True,
                    **o.hp())
        assert ro[0] == rd[0] and (ro[1] == rd[1] or (np.isnan(ro[1]) and np.isnan(rd[1])))
        if s == 2:
            assert ro[0] == zsm.ZS_NONFINITE
        got = o.state()
        S = o.S
        want = [to_host(x)[:S] for x in (d.master, d.exp_avg, d.exp_avg_sq, d.param)]
        for x, y in zip(got, want):
            assert np.array_equal(_bits(x), _bits(y)), s
    d.close()
    o.z.close()


def test_params_visible_on_the_stream():
    """Work queued on the context's stream after a step sees the new params
    without any host synchronisation."""
    log("test_params_visible_on_the_stream")
    w = scaled(workload(1), [200_000], [1], world_size=1, rank=0, M=1, name="offload-stream")
    o = Off(w, 1 << 14)
    out = torch.empty_like(o.z.param)
    for s in range(3):
        grads = o.case.fill_grads(s)
        o.z.step(grads, step=s + 1, **o.hp())
        out.copy_(o.z.param)             # queued on the current stream right away
    torch.cuda.synchronize()
    b = to_host(o.z.param)
    assert np.array_equal(to_host(out), b)
    p = o.z.master[:o.S].numpy()
    assert np.array_equal(b[:o.S], oracle.f32_to_bf16(p))
    o.z.close()


def test_offload_rejected_arguments_leave_state_untouched():
    log("test_offload_rejected_arguments_leave_state_untouched")
    w = scaled(workload(1), [5000, 64], [1, 0], world_size=1, rank=0, M=2, name="offload-args")
    o = Off(w, 1024)
    grads = o.case.fill_grads(0)
    o.z.step(grads, step=1, **o.hp())
    before = o.state()
    hp = o.hp()
    bad = [dict(step=0), dict(step=2, lr=-1.0), dict(step=2, beta1=1.0), dict(step=2, eps=0.0),
           dict(step=2, max_grad_norm=float("inf"))]
    for kw in bad:
        args = dict(hp, max_grad_norm=0.0)
        args.update(kw)
        with pytest.raises(zsm.ZeroShardError) as e:
            o.z.step(grads, **args)
        assert e.value.code == zsm.ZS_EINVAL
    with pytest.raises(zsm.ZeroShardError):     # a misaligned gradient pointer
        o.z.step([grads[0].data_ptr() + 2, grads[1].data_ptr()], step=2, **hp)
    for x, y in zip(o.state(), before):
        assert np.array_equal(_bits(x), _bits(y))
    o.z.close()


def _u16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


@pytest.mark.parametrize("clip", [0.0, 2.0])
def test_offload_amp_sequence_matches_oracle(clip):
    """The offloaded loss-scaled step: scaler decisions and step constants from the
    device, fp32 state updated on the host, fp16 param back; an Inf and a NaN
    are injected, so two steps are skipped and the scale backs off."""
    log(f"test_offload_amp_sequence_matches_oracle clip={clip}")
    numel, decay = [70_001, 64, 5, 130_000, 333], [1, 0, 0, 1, 0]
    N, rank, M = 3, 1, 3
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    z = ZeroOffload(numel, decay, N, rank, M, fp16=True, chunk_elems=1 << 14)
    S = z.shard_len
    pad = lay.padding_ranges()
    master = synth.host_normal_f32(S, synth.key(78, 0), 0.02)
    for o, n in pad:
        master[o:o + n] = 0
    z.master[:S] = torch.from_numpy(master)
    z.amp_init(2.0 ** 14)
    sc = oracle.Scaler(scale=2.0 ** 14, growth_interval=3)
    p, m, v = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    pf = np.zeros(S, np.uint16)
    mask = lay.decay_mask()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    skips = 0
    for s in range(12):
        scale = float(sc.scale[0])
        gs = []
        for j in range(M):
            g = synth.host_grad_f16(S, synth.key(78, 1 + j + M * s), 1e-3, scale)
            for o, n in pad:
                g[o:o + n] = 0
            gs.append(g)
        if s in (3, 8):
            gs[2][4321] = 0x7C00 if s == 3 else 0x7E00
        rc, norm = z.step_amp([_u16_dev(g) for g in gs], max_grad_norm=clip, growth_interval=3,
                              want_norm=True, return_code=True, **hp)
        fi, onorm = oracle.amp_step(gs, p, m, v, pf, mask, sc, max_grad_norm=clip, **hp)
        skips += fi
        assert (rc == zsm.ZS_NONFINITE) == fi
        if not fi:
            assert abs(norm - onorm) <= 1e-12 * onorm
        torch.cuda.synchronize()
        got = [z.master[:S].numpy(), z.exp_avg[:S].numpy(), z.exp_avg_sq[:S].numpy(),
               z.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]]
        for a, b in zip(got, (p, m, v, pf)):
            assert np.array_equal(_bits(a), _bits(b)), s
        assert z.amp_read() == (float(sc.scale[0]), int(sc.tracker[0]), sc.applied)
    assert skips == 2
    z.close()


def test_offload_amp_equals_device_amp():
    log("test_offload_amp_equals_device_amp")
    numel, decay = [5000, 64, 130_001, 7], [1, 0, 1, 0]
    zo = ZeroOffload(numel, decay, 2, 1, 4, fp16=True, chunk_elems=1 << 12,
                     flags=zsm.ZS_SKIP_NONFINITE)
    zd = ZeroShard(numel, decay, 2, 1, 4, fp16=True, flags=zsm.ZS_STAGE_AVERAGE)
    S = zo.shard_len
    m0 = synth.host_normal_f32(S, synth.key(79, 0), 0.02)
    zo.master[:S] = torch.from_numpy(m0)
    zd.master[:S].copy_(torch.from_numpy(m0))
    zo.amp_init(2.0 ** 10)
    zd.amp_init(2.0 ** 10)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_grad_norm=0.5,
              growth_interval=2)
    for s in range(5):
        gs = [torch.empty(S, dtype=torch.float16, device="cuda") for _ in range(4)]
        for j, g in enumerate(gs):
            synth.dev_grad_f16(g, synth.key(79, 1 + j + 4 * s), 1e-3, 2.0 ** 10)
        if s == 2:
            gs[0][10] = float("inf")
        zo.step_amp(gs, **hp)
        zd.step_amp(gs, **hp)
        torch.cuda.synchronize()
        got = [zo.master[:S].numpy(), zo.exp_avg[:S].numpy(), zo.exp_avg_sq[:S].numpy(),
               zo.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]]
        want = [to_host(x)[:S] for x in (zd.master, zd.exp_avg, zd.exp_avg_sq)] + \
               [zd.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]]
        for a, b in zip(got, want):
            assert np.array_equal(_bits(a), _bits(b)), s
        assert zo.amp_read() == zd.amp_read()
    zo.close()
    zd.close()


def test_offload_amp_empty_shard_keeps_the_scaler_in_step():
    """An offload rank with an empty shard advances its scaler like the others,
    alone and through the multi-rank split."""
    log("test_offload_amp_empty_shard_keeps_the_scaler_in_step")
    HPA = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    z = ZeroOffload([0, 0], [1, 1], 2, 1, 2, fp16=True)
    assert z.shard_len == 0
    z.amp_init(1024.0)
    g = torch.zeros(8, dtype=torch.int16, device="cuda")
    for _ in range(2):
        assert z.step_amp([g, g], growth_interval=2, want_norm=True, **HPA) == 0.0
    assert z.amp_read() == (2048.0, 0, 2)
    d = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    zsm.zero_offload_grad_sumsq_amp(z.ctx, [g.data_ptr()] * 2, z.amp_state.data_ptr(),
                                    d.data_ptr())
    assert d.item() == 0.0
    for total, want in ((4.0, (2048.0, 1, 3)), (float("inf"), (1024.0, 0, 3))):
        d.fill_(total)
        zsm.zero_offload_step_amp_global_norm(z.ctx, [g.data_ptr()] * 2, max_grad_norm=1.0,
                                              state_dev=z.amp_state.data_ptr(),
                                              growth_interval=2, global_sumsq_dev=d.data_ptr(),
                                              **HPA)
        assert z.amp_read() == want
    z.close()
