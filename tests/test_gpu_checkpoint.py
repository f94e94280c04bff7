"""Checkpoint / resharding on the GPU through the C ABI.

N ranks are simulated by N contexts on the one GPU.  Each rank's inputs are its
shard of per-tensor data (mapped by the oracle layout), so a canonical export
over all ranks must equal the oracle's unsharded trajectory bit for bit; after
resharding N -> N' (export, import into contexts of another plan) or a
save/load round trip through files, continuing must equal never stopping.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import layout as L
from sharded_optimizer_step_zero_amd import ZeroShard

from _gpu import log, to_host

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
NUMEL = [3000, 1, 64, 70_001, 5, 4096, 12_345, 0, 129]
DECAY = [1, 0, 0, 1, 0, 1, 1, 0, 0]
M = 2
SEED = 0xC4EC_0001


def _canon_data(steps):
    total = sum(NUMEL)
    master = synth.host_normal_f32(total, synth.key(SEED, 0), 0.02)
    grads = [[synth.host_grad_bf16(total, synth.key(SEED, 1 + j + M * s), 0, 1e-3)
              for j in range(M)] for s in range(steps)]
    mask = np.concatenate([np.full(n, d, np.uint8) for n, d in zip(NUMEL, DECAY)])
    return master, grads, mask


def _oracle_run(master, grads, mask, steps):
    p = master.copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for s in range(steps):
        oracle.step_f32(grads[s], p, m, v, None, mask, step=s + 1, **HP)
    return p, m, v


class Ranks:
    """N contexts of one plan geometry, fed from canonical host data."""

    def __init__(self, N, bucket_cap):
        self.lays = [L.plan(NUMEL, DECAY, N, r, bucket_cap, 64) for r in range(N)]
        self.zs = [ZeroShard(NUMEL, DECAY, N, r, M, bucket_cap=bucket_cap) for r in range(N)]
        for lay, z in zip(self.lays, self.zs):
            assert lay.shard_len == z.shard_len

    def load_master(self, master):
        for lay, z in zip(self.lays, self.zs):
            sh = np.zeros(z.shard_len, np.float32)
            lay.from_canonical(master, sh)
            z.master[:z.shard_len].copy_(torch.from_numpy(sh))

    def step(self, canon_grads, t):
        for lay, z in zip(self.lays, self.zs):
            gs = []
            for g in canon_grads:
                sh = np.zeros(z.shard_len, np.uint16)
                lay.from_canonical(g, sh)
                gs.append(torch.from_numpy(sh.view(np.int16)).to(z.device))
            z.step(gs, step=t, **HP)
        torch.cuda.synchronize()

    def export(self):
        total = sum(NUMEL)
        c = [torch.full((total,), float("nan"), device="cuda") for _ in range(3)]
        for z in self.zs:
            z.export_state(*c)
        torch.cuda.synchronize()
        return [x.cpu().numpy() for x in c]

    def import_(self, canon):
        d = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in canon]
        for z in self.zs:
            z.import_state(*d)
        torch.cuda.synchronize()

    def close(self):
        for z in self.zs:
            z.close()


def _same(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("N", [1, 3, 8])
def test_export_equals_unsharded_oracle(N):
    log(f"test_export_equals_unsharded_oracle N={N}")
    K = 3
    master, grads, mask = _canon_data(K)
    rk = Ranks(N, 20_000)
    rk.load_master(master)
    for s in range(K):
        rk.step(grads[s], s + 1)
    got = rk.export()
    want = _oracle_run(master, grads, mask, K)
    for g, w in zip(got, want):
        assert _same(g, w)
    rk.close()


@pytest.mark.parametrize("N,N2", [(3, 5), (8, 1), (1, 16)])
def test_reshard_then_continue(N, N2):
    log(f"test_reshard_then_continue {N}->{N2}")
    K = 2
    master, grads, mask = _canon_data(2 * K)
    a = Ranks(N, 20_000)
    a.load_master(master)
    for s in range(K):
        a.step(grads[s], s + 1)
    canon = a.export()
    a.close()
    b = Ranks(N2, 50_000)                       # another card count and bucket layout
    b.import_(canon)
    for lay, z in zip(b.lays, b.zs):            # import re-casts the bf16 params
        sh = np.zeros(z.shard_len, np.float32)
        lay.from_canonical(canon[0], sh)
        assert np.array_equal(to_host(z.param)[:z.shard_len], oracle.f32_to_bf16(sh))
    for s in range(K, 2 * K):
        b.step(grads[s], s + 1)
    got = b.export()
    want = _oracle_run(master, grads, mask, 2 * K)
    for g, w in zip(got, want):
        assert _same(g, w)
    b.close()


def test_checkpoint_file_roundtrip(tmp_path):
    log("test_checkpoint_file_roundtrip")
    K = 2
    master, grads, mask = _canon_data(2 * K)
    a = Ranks(4, 20_000)
    a.load_master(master)
    for s in range(K):
        a.step(grads[s], s + 1)
    for name, arr in zip(("master", "exp_avg", "exp_avg_sq"), a.export()):
        np.save(tmp_path / f"{name}.npy", arr)
    a.close()
    b = Ranks(4, 20_000)
    b.import_([np.load(tmp_path / f"{n}.npy") for n in ("master", "exp_avg", "exp_avg_sq")])
    for s in range(K, 2 * K):
        b.step(grads[s], s + 1)
    got = b.export()
    want = _oracle_run(master, grads, mask, 2 * K)
    for g, w in zip(got, want):
        assert _same(g, w)
    b.close()


@pytest.mark.parametrize("numel", [NUMEL, [4096, 8192, 65_536 * 2 + 256]])
def test_fp16_context_import_writes_fp16_param(numel):
    """Import into a ZS_FP16 context: master, m, v of this rank's elements and the
    fp16 param copy fp16_rne(master), padding untouched; export returns the state.
    NUMEL's sizes put most canonical offsets off 16-byte alignment (the 4-byte
    path); the second list keeps every part aligned (the 16-byte path)."""
    log(f"test_fp16_context_import_writes_fp16_param numel={numel}")
    decay = [1] * len(numel)
    N, rank = 2, 1
    lay = L.plan(numel, decay, N, rank, 25_000_000, 64)
    z = ZeroShard(numel, decay, N, rank, M, fp16=True)
    S, total = z.shard_len, sum(numel)
    new = [synth.host_normal_f32(total, synth.key(SEED, 200 + k), 3.0) for k in range(3)]
    z.import_state(*[torch.from_numpy(a).cuda() for a in new])
    torch.cuda.synchronize()
    own = np.ones(S, bool)
    for o, n in lay.padding_ranges():
        own[o:o + n] = False
    for t, a in zip((z.master, z.exp_avg, z.exp_avg_sq), new):
        want = np.zeros(S, np.float32)
        lay.from_canonical(a, want)
        assert _same(to_host(t)[:S], want)
    want_p = np.zeros(S, np.float32)
    lay.from_canonical(new[0], want_p)
    got_p = z.param.cpu().view(torch.int16).numpy().view(np.uint16)[:S]
    assert np.array_equal(got_p[own], oracle.f32_to_f16(want_p)[own])
    assert not got_p[~own].any()
    back = [torch.full((total,), -1.0, device="cuda") for _ in range(3)]
    z.export_state(*back)
    torch.cuda.synchronize()
    mine = np.zeros(total, bool)         # canonical positions this rank owns
    co = lay.canonical_offsets()
    for sg in lay.segments:
        if sg.tensor >= 0:
            c0 = co[sg.tensor] + sg.tensor_off
            mine[c0:c0 + sg.length] = True
    for c, a in zip(back, new):
        got = to_host(c)
        assert _same(got[mine], a[mine]) and (got[~mine] == -1.0).all()
    z.close()


def test_llama67b_export_import_sampled():
    """Export and import at the Llama-6.7B size (6.74G parameters: canonical
    offsets beyond 2^32), checked on samples through device gathers: seeded
    windows, the first and last elements of every tensor, and the last 4096
    elements of the model."""
    from synth.workloads import workload
    from _gpu import Gather
    w = workload(3)
    log(f"test_llama67b_export_import_sampled: {w.description}")
    torch.cuda.empty_cache()      # 94 GB of shard state and 81 GB of canonical arrays
    lay = L.plan(w.numel, w.decay, 1, 0, w.bucket_cap, w.align)
    z = ZeroShard(w.numel, w.decay, 1, 0, 1, bucket_cap=w.bucket_cap, align=w.align)
    S = z.shard_len
    synth.dev_normal_f32(z.master[:S], synth.key(SEED, 100), 0.02)
    synth.dev_normal_f32(z.exp_avg[:S], synth.key(SEED, 101), 1e-3)
    synth.dev_normal_f32(z.exp_avg_sq[:S], synth.key(SEED, 102), 1e-6)
    total = w.total_params
    assert total > (1 << 32)
    canon = [torch.empty(total, dtype=torch.float32, device="cuda") for _ in range(3)]
    z.export_state(*canon)
    torch.cuda.synchronize()
    co = lay.canonical_offsets()
    rng = np.random.default_rng(33)
    parts = [rng.integers(0, total - 64, 2048)[:, None] + np.arange(64)[None, :],
             np.arange(total - 4096, total)]
    for t, n in enumerate(w.numel):
        if n:
            parts += [np.array([co[t], co[t] + n - 1])]
    cidx = np.unique(np.concatenate([np.ravel(x) for x in parts]).astype(np.int64))
    # canonical index -> shard offset (N = 1: the tensor's flat offset + offset inside it)
    starts = np.array(co, np.int64)
    # the last tensor starting at or before each index (never an empty tensor)
    t_of = np.searchsorted(starts, cidx, side="right") - 1
    sidx = np.array(lay.tensor_flat_off, np.int64)[t_of] + (cidx - starts[t_of])
    order = np.argsort(sidx)
    gc, gs = Gather(cidx, "cuda"), Gather(sidx[order], "cuda")
    for c, s in zip(canon, (z.master, z.exp_avg, z.exp_avg_sq)):
        got = gc(c)[order]
        want = gs(s)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # import into a zeroed shard: state back, param = bf16_rne(master)
    for x in (z.master, z.exp_avg, z.exp_avg_sq, z.param):
        x.zero_()
    z.import_state(*canon)
    torch.cuda.synchronize()
    for c, s in zip(canon, (z.master, z.exp_avg, z.exp_avg_sq)):
        assert np.array_equal(gc(c)[order].view(np.uint32), gs(s).view(np.uint32))
    assert np.array_equal(gs(z.param), oracle.f32_to_bf16(gs(z.master)))
    log(f"  {cidx.size:,} sampled elements, max canonical offset {int(cidx.max()):,}")
    del canon
    z.close()
