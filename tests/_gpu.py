"""GPU parity helpers: run the HIP path through the C ABI and check it against the
oracle on the same seeded inputs.

Per-step error is measured the way the tolerance is stated: before each step
the GPU's pre-step state of the checked elements is fed to the oracle, and the
oracle's result is compared with the GPU's post-step state, so earlier
rounding differences do not accumulate into the per-step figure.  A separate
free-running oracle trajectory gives the drift report.

A clipped step is checked against the oracle's own clip coefficient (from the
oracle's fp64 norm of the whole shard), never the one the device derived: the
tolerance (1e-6 relative, 1 bf16 ulp) always applies, and bit-exactness is
required on the steps where the coefficient the device's norm implies equals
the oracle's.  The free-running trajectory uses the oracle's coefficient too.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import synth
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard
from synth.device_case import DeviceCase, padding_mask_at
from synth.workloads import Workload, special_ranges

TOL_REL = 1e-6           # fp32 master, m, v: max relative error per step
TINY = 2.0 ** -126


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(a: np.ndarray, b: np.ndarray) -> float:
    """max |a - b| / max(|b|, 2^-126), b the oracle; NaN positions must agree."""
    if np.array_equal(a.view(np.uint32), b.view(np.uint32)):
        return 0.0
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan)
    if (~nan).sum() == 0:
        return 0.0
    d = np.abs(a[~nan] - b[~nan]) / np.maximum(np.abs(b[~nan]), TINY)
    d[np.isinf(a[~nan]) & (a[~nan] == b[~nan])] = 0.0
    return float(d.max()) if d.size else 0.0


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> int:
    """max distance in bf16 ulps (NaN positions must agree)."""
    if np.array_equal(a, b):
        return 0
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    an = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    bn = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(an, bn)
    if (~bn).sum() == 0:
        return 0
    return int(np.abs(ordered(a[~bn]) - ordered(b[~bn])).max())


def coef_ulps(a, b) -> int:
    """Distance of two positive fp32 coefficients in ulps."""
    return abs(int(np.float32(a).view(np.int32)) - int(np.float32(b).view(np.int32)))


def bf16_ulp_hist(a: np.ndarray, b: np.ndarray) -> dict:
    """{ulps: count} of the bf16 param against the oracle's (NaN pairs count as 0)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    d = np.abs(ordered(a) - ordered(b))
    nan = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    d[nan] = 0
    vals, counts = np.unique(np.minimum(d, 2), return_counts=True)
    return {int(v): int(c) for v, c in zip(vals, counts)}


def to_host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


class Shard:
    """A ZeroShard bound to a workload's synthetic inputs (geometry from the oracle layout)."""

    def __init__(self, w: Workload, flags=0, device="cuda", contiguous=False):
        self.w = w
        self.lay = L.plan(w.numel, w.decay, w.world_size, w.rank, w.bucket_cap, w.align)
        # the slab placement bench.py times: state, contributions and workspace in one
        # allocation, staggered
        self.zs = ZeroShard(w.numel, w.decay, w.world_size, w.rank, w.M, device=device,
                            bucket_cap=w.bucket_cap, align=w.align, flags=flags,
                            grad_buffers=True, contiguous=contiguous)
        assert self.zs.shard_len == self.lay.shard_len
        self.S = self.lay.shard_len
        special = special_ranges(w, [(x.shard_off, x.length, x.tensor) for x in self.lay.segments])
        self.case = DeviceCase(w, self.S, self.lay.padding_ranges(), self.zs.device, special,
                               grads=self.zs.grads)
        self.case.fill_master(self.zs.master)
        torch.cuda.synchronize()

    def hp(self):
        w = self.w
        return dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay)

    def step(self, step0: int, want_norm=False):
        grads = self.case.fill_grads(step0)
        return self.zs.step(grads, step=step0 + 1, max_grad_norm=self.w.max_grad_norm,
                            want_norm=want_norm, **self.hp())

    def decay_at(self, idx):
        off = np.array([s.shard_off for s in self.lay.segments], np.int64)
        flag = np.array([s.decay for s in self.lay.segments], np.uint8)
        k = np.searchsorted(off, idx, side="right") - 1
        return flag[k]

    def close(self):
        self.zs.close()
        del self.case
        torch.cuda.empty_cache()


def full_parity(w: Workload, steps: int, flags=0, exact=True, contiguous=False):
    """Whole-shard parity for `steps` steps.  Returns the per-step stats."""
    sh = Shard(w, flags, contiguous=contiguous)
    S = sh.S
    hp = sh.hp()
    mask = sh.lay.decay_mask()
    stats = []
    # free-running oracle trajectory, from the same initial state
    fr_p = sh.case.host_master()
    assert np.array_equal(fr_p.view(np.uint32), to_host(sh.zs.master)[:S].view(np.uint32)), \
        "device and host generators disagree"
    fr_m = np.zeros(S, np.float32)
    fr_v = np.zeros(S, np.float32)
    fr_b = np.zeros(S, np.uint16)
    t_last = time.time()
    for s in range(steps):
        if time.time() - t_last > 20:
            log(f"  [{w.name}] step {s + 1}/{steps}")
            t_last = time.time()
        pre = [to_host(x)[:S].copy() for x in (sh.zs.master, sh.zs.exp_avg, sh.zs.exp_avg_sq)]
        g = sh.case.host_grads(s)
        coef = None
        if w.max_grad_norm > 0:
            # the oracle's own coefficient, from its own fp64 norm of the whole shard
            sumsq = oracle.grad_sumsq(g)
            want_norm = float(np.sqrt(sumsq))
            coef = oracle.clip_coef(sumsq, w.max_grad_norm)
        norm = sh.step(s, want_norm=w.max_grad_norm > 0)
        torch.cuda.synchronize()
        p, m, v = pre
        b = np.zeros(S, np.uint16)
        oracle.step_f32(g, p, m, v, b, mask, step=s + 1, coef=coef, **hp)
        got = [to_host(x)[:S] for x in (sh.zs.master, sh.zs.exp_avg, sh.zs.exp_avg_sq, sh.zs.param)]
        st = _step_stats(s, got, (p, m, v, b))
        same_coef = True
        if coef is not None:
            st["norm_rel"] = abs(norm - want_norm) / max(want_norm, 1e-300)
            st["coef_ulps"] = coef_ulps(oracle.coef_from_norm(norm, w.max_grad_norm), coef)
            same_coef = st["coef_ulps"] == 0
            assert st["norm_rel"] <= 1e-12 and st["coef_ulps"] <= 1, st
        oracle.step_f32(g, fr_p, fr_m, fr_v, fr_b, mask, step=s + 1, coef=coef, **hp)
        st["drift_master"] = rel_err(got[0], fr_p)
        st["drift_m"] = rel_err(got[1], fr_m)
        st["drift_v"] = rel_err(got[2], fr_v)
        st["drift_bf16_ulps"] = bf16_ulps(got[3], fr_b)
        stats.append(st)
        _assert_step(st, exact and same_coef)
    sh.close()
    return stats


def _step_stats(s, got, want) -> dict:
    """Per-step figures of the device state `got` against the oracle's `want`
    (master, m, v, bf16 param)."""
    p, m, v, b = want
    return dict(step=s + 1, n=int(p.size), rel_master=rel_err(got[0], p),
                rel_m=rel_err(got[1], m), rel_v=rel_err(got[2], v),
                bf16_ulps=bf16_ulps(got[3], b), bf16_hist=bf16_ulp_hist(got[3], b),
                exact=bool(np.array_equal(got[0].view(np.uint32), p.view(np.uint32))
                           and np.array_equal(got[1].view(np.uint32), m.view(np.uint32))
                           and np.array_equal(got[2].view(np.uint32), v.view(np.uint32))
                           and np.array_equal(got[3], b)))


def assert_within_tolerance(step, got, want):
    """The stated bar on a free-running comparison: master, m, v (got[0:3]) within
    1e-6 relative of the oracle's, the bf16 param (got[3]) within 1 ulp."""
    for k in range(3):
        e = rel_err(got[k], want[k])
        assert e <= TOL_REL, (step, k, e)
    u = bf16_ulps(got[3], want[3])
    assert u <= 1, (step, u)


def _assert_step(st, exact):
    """The stated bar always; bit-exactness where asked for."""
    assert st["rel_master"] <= TOL_REL and st["rel_m"] <= TOL_REL and st["rel_v"] <= TOL_REL, st
    assert st["bf16_ulps"] <= 1, st
    if exact:
        assert st["exact"], st


class Gather:
    """Host copies of t[idx] for device tensors, with the index kept on the device."""

    def __init__(self, idx, device):
        self.idx = np.ascontiguousarray(idx, dtype=np.int64)
        self.didx = torch.from_numpy(self.idx).to(device)

    def __call__(self, t):
        if self.idx.size and int(self.idx[-1]) >= t.numel():
            raise ValueError("index outside the tensor")
        out = torch.empty(self.idx.size, dtype=t.dtype, device=t.device)
        rc = synth.dev_lib().synth_dev_gather(out.data_ptr(), t.data_ptr(), t.element_size(),
                                              self.didx.data_ptr(), self.idx.size,
                                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        return to_host(out)


def sample_indices(lay, n_windows=4096, window=1024, seed=0, edge=64):
    """Seeded windows, the first and last `edge` elements of every segment, all padding."""
    S = lay.shard_len
    rng = np.random.default_rng(seed)
    parts = []
    if S > window:
        starts = rng.integers(0, S - window, n_windows)
        parts.append((starts[:, None] + np.arange(window)[None, :]).reshape(-1))
    else:
        parts.append(np.arange(S))
    for s in lay.segments:
        if s.tensor < 0:
            parts.append(np.arange(s.shard_off, s.shard_off + s.length))
        else:
            k = min(edge, s.length)
            parts.append(np.arange(s.shard_off, s.shard_off + k))
            parts.append(np.arange(s.shard_off + s.length - k, s.shard_off + s.length))
    parts.append(np.array([0, S - 1]))
    idx = np.unique(np.concatenate(parts).astype(np.int64))
    return idx[(idx >= 0) & (idx < S)]


def sampled_parity(w: Workload, steps: int, idx=None, check_steps=None, exact=True,
                   full_norm=None):
    """Parity on sampled elements at full size; returns per-checked-step stats.

    full_norm: callable(step0) -> oracle sumsq of the whole shard (needed when clipping)."""
    t0 = time.time()
    sh = Shard(w)
    log(f"  [{w.name}] S={sh.S:,} M={w.M} allocated+filled in {time.time() - t0:.1f}s")
    if idx is None:
        idx = sample_indices(sh.lay)
    hp = sh.hp()
    gat = Gather(idx, sh.zs.device)
    dec = sh.decay_at(idx)
    pad = padding_mask_at(idx, sh.lay.padding_ranges())
    dec[pad] = 0
    st_all = []
    fr_p = sh.case.host_master(idx)
    got0 = gat(sh.zs.master)
    assert np.array_equal(fr_p.view(np.uint32), got0.view(np.uint32)), "generators disagree"
    fr_m = np.zeros(idx.size, np.float32)
    fr_v = np.zeros(idx.size, np.float32)
    fr_b = np.zeros(idx.size, np.uint16)
    cached_coef = {}
    cached_g = {}
    t_last = time.time()
    for s in range(steps):
        if time.time() - t_last > 20:
            log(f"  [{w.name}] step {s + 1}/{steps}")
            t_last = time.time()
        check = check_steps is None or (s + 1) in check_steps
        if check:
            pre = [gat(x) for x in (sh.zs.master, sh.zs.exp_avg, sh.zs.exp_avg_sq)]
        norm = sh.step(s, want_norm=w.max_grad_norm > 0)
        gs_key = w.grad_step_index(s)
        if gs_key not in cached_g:
            cached_g.clear()
            cached_g[gs_key] = sh.case.host_grads(s, idx)
        g = cached_g[gs_key]
        coef = None
        same_coef = True
        if w.max_grad_norm > 0:
            # the oracle's own coefficient, from its fp64 norm of the whole shard
            gs = w.grad_step_index(s)
            if gs not in cached_coef:
                sumsq = full_norm(s)
                cached_coef[gs] = (oracle.clip_coef(sumsq, w.max_grad_norm), float(np.sqrt(sumsq)))
            coef, want_norm = cached_coef[gs]
            ulps = coef_ulps(oracle.coef_from_norm(norm, w.max_grad_norm), coef)
            same_coef = ulps == 0
            assert abs(norm - want_norm) <= 1e-12 * want_norm, (norm, want_norm)
            assert ulps <= 1, (s, ulps)
        oracle.step_f32(g, fr_p, fr_m, fr_v, fr_b, dec, step=s + 1, coef=coef, **hp)
        if not check:
            continue
        torch.cuda.synchronize()
        p, m, v = pre
        b = np.zeros(idx.size, np.uint16)
        oracle.step_f32(g, p, m, v, b, dec, step=s + 1, coef=coef, **hp)
        got = [gat(x) for x in (sh.zs.master, sh.zs.exp_avg, sh.zs.exp_avg_sq, sh.zs.param)]
        st = _step_stats(s, got, (p, m, v, b))
        st["drift_master"] = rel_err(got[0], fr_p)
        st["drift_m"] = rel_err(got[1], fr_m)
        st["drift_v"] = rel_err(got[2], fr_v)
        st["drift_bf16_ulps"] = bf16_ulps(got[3], fr_b)
        if coef is not None:
            st["norm_rel"] = abs(norm - want_norm) / want_norm
            st["coef_ulps"] = ulps
        st_all.append(st)
        _assert_step(st, exact and same_coef)
    sh.close()
    return st_all
