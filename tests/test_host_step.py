"""The offloaded update on host cores (zs_host_adamw), on the CPU, against the
oracle: bit for bit, whatever the thread count, chunking or vector width, with
decay runs, clip coefficients, several steps, and non-finite and subnormal
gradients.  The host update takes the M-way average the device stages; the
oracle's own average (oracle.reduce_mean_f32) stands in for it here."""
import numpy as np
import pytest

import oracle
import sharded_optimizer_step_zero_amd as zs
import synth
from oracle import layout as L

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
NUMEL = [1, 63, 64, 65, 1000, 0, 4097, 12_345, 7, 100_001, 3, 33_333]
DECAY = [1, 0, 1, 0, 1, 1, 0, 1, 0, 1, 0, 0]


def _case(N=3, rank=1, M=3, seed=11):
    lay = L.plan(NUMEL, DECAY, N, rank, 25_000_000, 64)
    S = lay.shard_len
    grads = [synth.host_grad_bf16(S, synth.key(seed, 1 + j), synth.key(seed, 99 + j), 1e-3)
             for j in range(M)]
    for g in grads:
        for o, n in lay.padding_ranges():
            g[o:o + n] = 0
    master = synth.host_normal_f32(S, synth.key(seed, 0), 0.02)
    for o, n in lay.padding_ranges():
        master[o:o + n] = 0
    return lay, grads, master


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _host_step(plan, g_avg, coef, p, m, v, b, step, n_threads, chunks):
    for off, n in chunks:
        zs.zs_host_adamw(plan, off, n, g_avg[off:].ctypes.data, coef, p[off:].ctypes.data,
                         m[off:].ctypes.data, v[off:].ctypes.data, b[off:].ctypes.data,
                         step=step, n_threads=n_threads, **HP)


def _chunks(S, sizes):
    out, off, i = [], 0, 0
    while off < S:
        n = min(sizes[i % len(sizes)], S - off)
        out.append((off, n))
        off += n
        i += 1
    return out


@pytest.mark.parametrize("n_threads,chunk_sizes", [(1, [1 << 30]), (3, [1 << 30]),
                                                    (8, [1000, 77, 4096, 12_345]),
                                                    (0, [64, 65_536])])
@pytest.mark.parametrize("clip", [None, 0.05])
def test_host_update_equals_oracle(n_threads, chunk_sizes, clip):
    lay, grads, master = _case()
    S = lay.shard_len
    plan = zs.zs_plan_create(NUMEL, DECAY, 3, 1)
    try:
        assert zs.zs_plan_query(plan)["shard_len"] == S
        g_avg = oracle.reduce_mean_f32(grads)
        coef = oracle.clip_coef(oracle.grad_sumsq(grads), clip) if clip else None
        p, m, v, b = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
            np.zeros(S, np.uint16)
        op, om, ov, ob = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
            np.zeros(S, np.uint16)
        mask = lay.decay_mask()
        for t in range(1, 4):
            _host_step(plan, g_avg, float(coef) if coef is not None else 1.0, p, m, v, b, t,
                       n_threads, _chunks(S, chunk_sizes))
            oracle.step_f32(grads, op, om, ov, ob, mask, step=t, coef=coef, **HP)
            for x, y in zip((p, m, v, b), (op, om, ov, ob)):
                assert np.array_equal(_bits(x), _bits(y)), t
        for o, n in lay.padding_ranges():   # padding stays zero
            assert not p[o:o + n].any() and not b[o:o + n].any()
    finally:
        zs.zs_plan_destroy(plan)


def test_host_update_special_values():
    lay, grads, master = _case(N=1, rank=0, M=2, seed=12)
    S = lay.shard_len
    rng = np.random.default_rng(5)
    idx = rng.choice(S, 600, replace=False)
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x8001, 0x007F, 0x0000, 0x8000],
                        np.uint16)
    grads[0][idx] = specials[np.arange(idx.size) % specials.size]
    grads[1][idx[::3]] = 0x7F80
    master[idx[::5]] = np.float32(1e-40)            # subnormal masters
    plan = zs.zs_plan_create(NUMEL, DECAY, 1, 0)
    try:
        g_avg = oracle.reduce_mean_f32(grads)
        p, m, v, b = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
            np.zeros(S, np.uint16)
        op, om, ov, ob = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
            np.zeros(S, np.uint16)
        _host_step(plan, g_avg, 1.0, p, m, v, b, 1, 4, [(0, S)])
        oracle.step_f32(grads, op, om, ov, ob, lay.decay_mask(), step=1, **HP)
        for x, y in zip((p, m, v, b), (op, om, ov, ob)):
            assert np.array_equal(_bits(x), _bits(y))
        assert np.isnan(p).any() and np.isnan(m).any()
    finally:
        zs.zs_plan_destroy(plan)


def test_host_update_argument_errors():
    plan = zs.zs_plan_create([1000], [1], 1, 0)
    a = np.zeros(1024, np.float32)
    b = np.zeros(1024, np.uint16)
    p = a.ctypes.data
    try:
        for off, n in ((-1, 10), (0, 1025), (1000, 100)):
            with pytest.raises(zs.ZeroShardError) as e:
                zs.zs_host_adamw(plan, off, n, p, 1.0, p, p, p, b.ctypes.data, step=1, **HP)
            assert e.value.code == zs.ZS_EINVAL
        with pytest.raises(zs.ZeroShardError):
            zs.zs_host_adamw(plan, 0, 10, p, float("nan"), p, p, p, b.ctypes.data, step=1, **HP)
        with pytest.raises(zs.ZeroShardError):
            zs.zs_host_adamw(plan, 0, 10, p, 1.0, p, p, p, b.ctypes.data, step=0, **HP)
        zs.zs_host_adamw(plan, 5, 0, 0, 1.0, 0, 0, 0, 0, step=1, **HP)     # empty range
    finally:
        zs.zs_plan_destroy(plan)


def test_offload_init_argument_errors_before_any_device_call():
    plan = zs.zs_plan_create([1000], [1], 1, 0)
    ws = zs.zs_workspace_bytes(plan, 2, zs.ZS_STAGE_AVERAGE)
    st = zs.zs_offload_staging_bytes(1 << 16)
    assert st > 6 * (1 << 16) and zs.zs_offload_staging_bytes(100) == 0
    try:
        bad = [dict(chunk_elems=100), dict(flags=0x80), dict(n_threads=-1),
               dict(workspace_bytes=ws - 1), dict(staging_bytes=st - 1), dict(staging=272)]
        for kw in bad:
            args = dict(workspace_bytes=ws, staging=256, staging_bytes=st, chunk_elems=1 << 16,
                        n_threads=0, flags=0)
            args.update(kw)
            with pytest.raises(zs.ZeroShardError) as e:
                zs.zero_offload_init(plan, 2, 16, 16, 16, 16, 256, args["workspace_bytes"],
                                     args["staging"], args["staging_bytes"], args["chunk_elems"],
                                     args["n_threads"], 0, args["flags"])
            assert e.value.code == zs.ZS_EINVAL, kw
    finally:
        zs.zs_plan_destroy(plan)


@pytest.mark.parametrize("clip", [None, 0.05])
def test_host_update_fp16_equals_oracle(clip):
    """The loss-scaled variant's host update: the unscaled M-way average in, the
    fp16 param copy out (flags = ZS_FP16), against the oracle's fp16 step."""
    lay = L.plan(NUMEL, DECAY, 3, 1, 25_000_000, 64)
    S = lay.shard_len
    scale = 2.0 ** 13
    grads = [synth.host_grad_f16(S, synth.key(21, 1 + j), 1e-3, scale) for j in range(3)]
    for g in grads:
        for o, n in lay.padding_ranges():
            g[o:o + n] = 0
    master = synth.host_normal_f32(S, synth.key(21, 0), 0.02)
    for o, n in lay.padding_ranges():
        master[o:o + n] = 0
    inv = oracle.inv_scale(scale)
    g_avg = oracle.reduce_mean_f16(grads, inv)
    coef = oracle.clip_coef(oracle.grad_sumsq_f16(grads, inv), clip) if clip else None
    plan = zs.zs_plan_create(NUMEL, DECAY, 3, 1)
    try:
        p, m, v, b = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
            np.zeros(S, np.uint16)
        op, om, ov, ob = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), \
            np.zeros(S, np.uint16)
        for t in range(1, 4):
            zs.zs_host_adamw(plan, 0, S, g_avg.ctypes.data, float(coef) if clip else 1.0,
                             p.ctypes.data, m.ctypes.data, v.ctypes.data, b.ctypes.data, step=t,
                             n_threads=4, flags=zs.ZS_FP16, **HP)
            oracle.step_f16(grads, op, om, ov, ob, lay.decay_mask(), step=t, inv_scale=inv,
                            coef=coef, **HP)
            for x, y in zip((p, m, v, b), (op, om, ov, ob)):
                assert np.array_equal(_bits(x), _bits(y)), t
    finally:
        zs.zs_plan_destroy(plan)


def test_host_fp16_recast_matches_oracle():
    """With lr = 0 the update leaves master as it is, so the param copy is the
    fp16 conversion of master: every exponent, both signs, mantissas at and around
    each rounding boundary of the normal and subnormal ranges, and random ones."""
    rng = np.random.default_rng(7)
    exps = np.arange(256, dtype=np.uint32)
    low = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x3FFF, 0x7FFFFF,
                    0x400000, 0x3FFFFF, 0x7FF000, 0x7FEFFF], np.uint32)
    rand = rng.integers(0, 1 << 23, 600, dtype=np.uint32)
    mant = np.concatenate([low, rand])
    # subnormal-range boundaries: for exponent e the result keeps the bits above 126 - e
    for s in range(14, 25):
        half = np.uint32(1 << (s - 1))
        for q in (0, 1, 2, 3):
            base = np.uint32((q << s) & 0x7FFFFF)
            mant = np.concatenate([mant, np.array([base, base + half, base + half - 1,
                                                   base + half + 1], np.uint32) & 0x7FFFFF])
    u = (exps[:, None] << 23 | mant[None, :]).reshape(-1)
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    x = u.view(np.float32)
    n = x.size
    pad = (-n) % 8
    x = np.concatenate([x, np.zeros(pad, np.float32)])
    n = x.size
    plan = zs.zs_plan_create([n], [0], 1, 0, align=8)
    try:
        p = x.copy()
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        g = np.zeros(n, np.float32)
        b = np.zeros(n, np.uint16)
        hp = dict(HP, lr=0.0, weight_decay=0.0)
        zs.zs_host_adamw(plan, 0, n, g.ctypes.data, 1.0, p.ctypes.data, m.ctypes.data,
                         v.ctypes.data, b.ctypes.data, step=1, n_threads=4, flags=zs.ZS_FP16, **hp)
        nan = np.isnan(x)
        assert np.array_equal(p.view(np.uint32)[~nan], x.view(np.uint32)[~nan])
        want = oracle.f32_to_f16(x)
        assert np.array_equal(b[~nan], want[~nan])
        assert ((b[nan] & 0x7C00) == 0x7C00).all() and ((b[nan] & 0x3FF) != 0).all()
    finally:
        zs.zs_plan_destroy(plan)
