"""Benchmark of the fused per-rank ZeRO shard step on one MI355X.

One "step" is one call of zero_shard_step over the rank's whole shard: the
M-way bf16 gradient reduce, (optional clip,) the AdamW update of the fp32
master and moments, and the bf16 re-cast -- every row of the hot path.  Inputs
are seeded synthetic values already resident in HBM when timing starts; the
gradient contributions of one batch are reused for every timed step.

Prints one JSON line.  `value` is params/s over the shard (the whole job on
one GPU); `roofline` prices the step kernel against MI355X's 8 TB/s HBM peak
using the algorithmic bytes 2M+12 read + 14 written per parameter;
`cpu_baseline` times the CPU oracle on a bounded slab of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload 1..5] [--no-cpu-baseline]
                    [--checkpoint] [--amp] [--offload] [--cold] [--no-extras]
                    [--graph] [--static-step] [--sweep-caps 8,9,...] [--ceiling]

The default workload is the largest one a single GPU holds: the unsharded
Llama-shaped 6.7B parameter list (M = 1, 108 GB of state resident).  With
--workload 2 (the GPT-1.3B 1/8 shard) the line also carries the checkpoint
export/import, the loss-scaled fp16 step (fused and staged) and the offloaded
step on host cores ("checkpoint", "amp_fp16", "amp_fp16_staged", "offload",
"offload_fp16") and the timed steps replayed from one HIP graph ("graph"), each
timed after the headline step; --no-extras leaves them out.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused reduce+AdamW shard step: params/s and HBM GB/s as % of MI355X peak"
PEAK_HBM_GBS = 8000.0


def _code_only(text: str) -> str:
    """Source text without // comments, trailing blanks and empty lines."""
    out = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            out.append(code)
    return "\n".join(out)


def kernel_source_hash(read=None) -> str:
    """Hash of the step kernel's code (comments ignored): counters taken on one
    version of the code stay valid across comment edits, not across code edits."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "internal.h"):
        path = os.path.join(ROOT, "sharded_optimizer_step_zero_amd", "csrc", f)
        if read is None:
            with open(path, encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(S: int, M: int, clip: bool) -> dict:
    step = S * (2 * M + 12 + 14)
    norm = S * 2 * M if clip else 0
    return {"step_kernel": step, "norm_pass": norm, "total": step + norm}


def traffic_for(workload_name: str):
    """HBM bytes per launch of the step kernel from the committed counter summary,
    or None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"step_kernel_traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, slab: int, min_seconds: float = 10.0) -> dict:
    """The CPU oracle, as it stands, on a slab of `slab` elements of the workload."""
    import numpy as np

    import oracle
    import synth

    threads = oracle.get_threads()
    keys = w.grad_keys(0)
    grads = [synth.host_grad_bf16(slab, k, ks, w.sigma_grad, w.kinds) for k, ks in keys]
    p = synth.host_normal_f32(slab, w.master_key(), w.sigma_master)
    m = np.zeros(slab, np.float32)
    v = np.zeros(slab, np.float32)
    b = np.zeros(slab, np.uint16)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    clip = w.max_grad_norm > 0

    def run(n: int, seconds: float):
        oracle.set_threads(n)
        steps = 0
        t0 = time.perf_counter()
        while True:
            coef = oracle.clip_coef(oracle.grad_sumsq(grads), w.max_grad_norm) if clip else None
            oracle.step_f32(grads, p, m, v, b, None, step=steps + 1, coef=coef, **hp)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return steps, el

    try:
        steps, el = run(threads, min_seconds)
        steps1, el1 = run(1, min_seconds / 4)
    finally:
        oracle.set_threads(threads)
    return {"value": slab * steps / el, "unit": "params/s", "cores": int(threads),
            "kind": "oracle",
            "one_thread_value": slab * steps1 / el1,
            "sample": f"{steps} oracle steps over a {slab:,}-element slab of the shard "
                      f"(M={w.M}{', with the norm pass' if clip else ''}), {el:.1f} s on "
                      f"{threads} threads; then {steps1} steps on one thread, {el1:.1f} s"}


def time_graph(zs, grads, w, hp, steps: int, step0: int) -> dict:
    """The same steps captured once into a HIP graph (step numbers step0.. baked in)
    and replayed: launch gaps disappear, which matters where a step is a few
    microseconds.  The step queues kernels only, so it captures as it is."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        zs.set_stream(torch.cuda.current_stream().cuda_stream)
        for s in range(steps):
            zs.step(grads, step=step0 + s, max_grad_norm=w.max_grad_norm, **hp)
    cur = torch.cuda.current_stream()
    zs.set_stream(cur.cuda_stream)
    g.replay()                                   # warm-up replay
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return {"ms_per_step": ms, "params_per_s": zs.shard_len / (ms * 1e-3), "steps": steps}


def time_checkpoint(zs, w, stream, reps: int = 10) -> dict:
    """Export and import of this rank's fp32 state to/from the canonical order:
    12 B read + 12 B written per shard parameter (import also writes the 2-byte
    bf16 param)."""
    import torch
    total = w.total_params
    canon = [torch.zeros(total, dtype=torch.float32, device=zs.device) for _ in range(3)]
    out = {}
    for name, fn, nbytes in (("export", zs.export_state, 24), ("import", zs.import_state, 26)):
        fn(*canon)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn(*canon)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": ms, "bytes_per_param": nbytes,
                     "gbs": zs.shard_len * nbytes / (ms * 1e-3) / 1e9}
    del canon
    return out


def percentiles(xs) -> dict:
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


def sweep_caps(zs, grads, w, hp, stream, caps, rounds: int, steps: int) -> dict:
    """The step kernel's wave cap swept on the same buffers: one context per cap
    (ZS_WAVES_PER_CU set while it is created; 0 = no cap), all bound to this shard's
    arrays, timed in alternating rounds so that placement does not mix into the
    comparison.  Returns GB/s per cap and round at the algorithmic bytes."""
    import torch

    import sharded_optimizer_step_zero_amd as zsm
    ctxs, keep = {}, []
    old = os.environ.get("ZS_WAVES_PER_CU")
    try:
        for c in caps:
            os.environ["ZS_WAVES_PER_CU"] = str(c)
            ws = torch.zeros(zs.ws_bytes + 256, dtype=torch.uint8, device=zs.device)
            keep.append(ws)
            ctxs[c] = zsm.zero_shard_init(zs.plan, w.M, zs.param.data_ptr(), zs.master.data_ptr(),
                                          zs.exp_avg.data_ptr(), zs.exp_avg_sq.data_ptr(),
                                          ws.data_ptr() + (-ws.data_ptr()) % 256, zs.ws_bytes,
                                          stream.cuda_stream, 0)
    finally:
        if old is None:
            os.environ.pop("ZS_WAVES_PER_CU", None)
        else:
            os.environ["ZS_WAVES_PER_CU"] = old
    ptrs = [g if isinstance(g, int) else g.data_ptr() for g in grads]
    by = zs.shard_len * (2 * w.M + 26)
    out = {c: [] for c in caps}
    try:
        for c in caps:                            # one untimed step per context
            zsm.zero_shard_step(ctxs[c], ptrs, step=1, max_grad_norm=0.0, **hp)
        for _ in range(rounds):
            for c in caps:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for s in range(steps):
                    zsm.zero_shard_step(ctxs[c], ptrs, step=2 + s, max_grad_norm=0.0, **hp)
                e1.record(stream)
                torch.cuda.synchronize()
                out[c].append(by / (e0.elapsed_time(e1) / steps * 1e-3) / 1e9)
    finally:
        for ctx in ctxs.values():
            zsm.zero_shard_destroy(ctx)
    return {"gbs_per_round": {str(c): v for c, v in out.items()}, "rounds": rounds,
            "steps_per_round": steps, "note": "same buffers, one context per cap, no clip"}


def time_static(zs, grads, w, hp, stream, steps: int, step0: int) -> dict:
    """The allocation-free entry point (zero_shard_step_static) on the same buffers:
    no context, its tables and partials in the library's static device scratch."""
    import torch

    import sharded_optimizer_step_zero_amd as zsm
    ptrs = [g if isinstance(g, int) else g.data_ptr() for g in grads]

    def one(step):
        zsm.zero_shard_step_static(zs.plan, w.M, zs.param.data_ptr(), zs.master.data_ptr(),
                                   zs.exp_avg.data_ptr(), zs.exp_avg_sq.data_ptr(), ptrs,
                                   step=step, max_grad_norm=w.max_grad_norm,
                                   stream=stream.cuda_stream, **hp)
    one(step0)                                    # the first call resolves the scratch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(steps):
        one(step0 + 1 + s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms_per_step": ms, "params_per_s": zs.shard_len / (ms * 1e-3), "steps": steps}


def time_ceiling(zs, stream, reps: int) -> dict:
    """What the library-side copies reach on the shard's own slab (same placement as
    the step): torch's device-to-device copy_ (hipMemcpyAsync) and a plain 16-byte
    copy kernel from master into exp_avg (one read and one write stream, as the
    step's mix), a fill of exp_avg_sq (writes only; again over its first S rounded
    down to a multiple of 2^20 elements) and a sum of master (reads only).
    Overwrites the optimizer state, so it runs after every other step leg."""
    import torch

    import synth
    S = zs.shard_len
    src, dst, fill = zs.master[:S], zs.exp_avg[:S], zs.exp_avg_sq[:S]
    acc = torch.empty((), dtype=torch.float32, device=zs.device)
    S20 = S >> 20 << 20
    fill20 = zs.exp_avg_sq[:S20]
    legs = {
        "memcpy_d2d": (lambda: dst.copy_(src), 8 * S),
        "copy_kernel_16B": (lambda: synth.dev_copy(dst, src, stream.cuda_stream), 8 * S),
        "fill": (lambda: fill.fill_(1.0), 4 * S),
        # torch's fill is slower at some element counts: the same array, cut down to a
        # multiple of 2^20 elements
        "fill_2pow20_multiple": (lambda: fill20.fill_(1.0), 4 * S20),
        "sum": (lambda: torch.sum(src, (0,), out=acc), 4 * S),
    }
    if S20 == 0:
        del legs["fill_2pow20_multiple"]
    out = {}
    for name, (fn, nbytes) in legs.items():
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "bytes": nbytes, "gbs": gbs, "frac": gbs / PEAK_HBM_GBS}
    return out


def time_cold(zs, grads, w, hp, stream, step0: int, reps: int) -> dict:
    """Per-step time with the 256 MB Infinity Cache evicted before each step (a
    1 GiB buffer is overwritten between steps, outside the timed events)."""
    import torch
    junk = torch.empty(1 << 28, dtype=torch.float32, device=zs.device)
    out = []
    for r in range(reps):
        junk.fill_(float(r))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        zs.step(grads, step=step0 + r, max_grad_norm=w.max_grad_norm, **hp)
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del junk
    return percentiles(out)


def time_amp(w, pad, dev, stream, steps: int, warmup: int, stage: bool = False,
             init_scale: float = 2.0 ** 14) -> dict:
    """The fp16 loss-scaled variant on the same shard: fp16 contributions
    (generated at the initial loss scale), unscale fused into the reduce, the
    norm pass that detects overflow on every step, the device-side skip and
    scaler update, and the fp16 re-cast.  Bytes per parameter: 2M (norm pass)
    + 2M + 12 read + 14 written (step kernel); staged (ZS_STAGE_AVERAGE): the
    norm pass reads 2M and writes 4, the step reads 4 + 12 and writes 14."""
    import torch

    import synth
    from sharded_optimizer_step_zero_amd import ZS_STAGE_AVERAGE, ZeroShard

    za = ZeroShard(w.numel, w.decay, w.world_size, w.rank, w.M, device=dev,
                   bucket_cap=w.bucket_cap, align=w.align, fp16=True,
                   flags=ZS_STAGE_AVERAGE if stage else 0, grad_buffers=True)
    za.set_stream(stream.cuda_stream)
    S = za.shard_len
    synth.dev_normal_f32(za.master[:S], w.master_key(), w.sigma_master)
    synth.dev_zero_ranges(za.master, pad)
    grads = za.grads
    for (k, _), g in zip(w.grad_keys(0), grads):
        synth.dev_grad_f16(g[:S], k, w.sigma_grad, init_scale)
        synth.dev_zero_ranges(g, pad)
    za.amp_init(init_scale)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm)
    for _ in range(warmup):
        za.step_amp(grads, **hp)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        za.step_amp(grads, **hp)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    scale, tracker, applied = za.amp_read()
    bpp = 2 * w.M + 34 if stage else 4 * w.M + 26
    by = S * bpp
    za.close()
    del grads
    return {"ms_per_step": ms, "params_per_s": S / (ms * 1e-3), "staged": stage,
            "bytes_per_param": bpp,
            "hbm_gbs_whole_step": by / (ms * 1e-3) / 1e9,
            "frac_of_peak_whole_step": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "applied_steps": applied, "final_scale": scale,
            "kernels": "zs::sumsq_f16_kernel, sum_blocks, amp_finalize, "
                       + ("zs::step_staged_kernel<true>" if stage else "zs::step_f16_kernel")}


def time_offload(w, pad, dev, stream, steps: int, warmup: int, chunk: int = 1 << 24,
                 fp16: bool = False) -> dict:
    """The optimizer step on host cores (zero_offload_step) on the same shard:
    device reduce + norm, the fp32 averages to pinned host memory (4 B/param),
    the AdamW update of host fp32 state (30 B/param of host memory traffic), the
    bf16 params back (2 B/param); chunks overlap.  Also times its parts: pinned
    copies each way, the host update alone, and a host STREAM-add of 3 arrays,
    so the figure can be read against the slowest of them.  fp16: the loss-scaled
    variant (zero_offload_step_amp: fp16 contributions at the initial scale, the
    scaler decided on the device, fp16 param back)."""
    import numpy as np
    import torch

    import sharded_optimizer_step_zero_amd as zsm
    from sharded_optimizer_step_zero_amd import ZeroOffload
    from synth.device_case import DeviceCase

    zo = ZeroOffload(w.numel, w.decay, w.world_size, w.rank, w.M, device=dev,
                     bucket_cap=w.bucket_cap, align=w.align, chunk_elems=chunk, fp16=fp16)
    zo.set_stream(stream.cuda_stream)
    S = zo.shard_len
    case = DeviceCase(w, S, pad, dev)
    zo.master[:S] = torch.from_numpy(case.host_master())
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm)
    if fp16:
        import synth
        grads = []
        for k, _ in w.grad_keys(0):
            g = torch.empty(max(S, 8), dtype=torch.float16, device=dev)
            synth.dev_grad_f16(g[:S], k, w.sigma_grad, 2.0 ** 14)
            synth.dev_zero_ranges(g, pad)
            grads.append(g)
        zo.amp_init(2.0 ** 14)

        def one(step):
            zo.step_amp(grads, **hp)
    else:
        grads = case.fill_grads(0)

        def one(step):
            zo.step(grads, step=step, **hp)
    for s in range(warmup):
        one(s + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one(warmup + s + 1)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps

    # the host update alone, over the whole shard
    g = np.full(S, 1e-4, np.float32)
    p = zo.master[:S].numpy().copy()
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    b = np.zeros(S, np.uint16)
    reps = 3
    for t in range(reps + 1):           # the first pass also faults the pages in, untimed
        if t == 1:
            t0 = time.perf_counter()
        zsm.zs_host_adamw(zo.plan, 0, S, g.ctypes.data, 1.0, p.ctypes.data, m.ctypes.data,
                          v.ctypes.data, b.ctypes.data, lr=w.lr, beta1=w.beta1, beta2=w.beta2,
                          eps=w.eps, weight_decay=w.weight_decay, step=t + 1,
                          flags=zsm.ZS_FP16 if fp16 else 0)
    host_s = (time.perf_counter() - t0) / reps
    del g, p, m, v, b

    # pinned copies of 1 GiB each way
    n = 1 << 28
    h = torch.empty(n, dtype=torch.float32, pin_memory=True)
    d = torch.empty(n, dtype=torch.float32, device=dev)
    bw = {}
    for name, dst, src_ in (("d2h", h, d), ("h2d", d, h)):
        dst.copy_(src_, non_blocking=True)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dst.copy_(src_, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        bw[name] = 3 * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del h, d

    # host memory reference: c = a + b over 3 x 1 GiB with the intra-op threads
    a = torch.ones(n)
    b2 = torch.ones(n)
    c = torch.empty(n)
    torch.add(a, b2, out=c)
    t0 = time.perf_counter()
    for _ in range(3):
        torch.add(a, b2, out=c)
    stream_gbs = 3 * 3 * 4 * n / (time.perf_counter() - t0) / 1e9
    del a, b2, c
    zo.close()
    del grads
    return {"ms_per_step": ms, "params_per_s": S / (ms * 1e-3), "chunk_elems": chunk,
            "param_dtype": "fp16 (loss-scaled)" if fp16 else "bf16",
            "pcie_bytes_per_param": {"d2h": 4, "h2d": 2},
            "pcie_d2h_gbs": bw["d2h"], "pcie_h2d_gbs": bw["h2d"],
            "host_update_params_per_s": S / host_s,
            "host_update_gbs": 30 * S / host_s / 1e9,
            "host_stream_add_gbs": stream_gbs,
            "host_threads": len(os.sched_getaffinity(0)),
            "stream_add_threads": torch.get_num_threads(),
            "bound_params_per_s": min(bw["d2h"] * 1e9 / 4, bw["h2d"] * 1e9 / 2, S / host_s),
            "note": "wall clock; the whole offloaded step incl. PCIe (never the headline value)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3,
                    help="1 tiny, 2 GPT-1.3B 1/8 shard, 3 Llama-6.7B unsharded (default: the "
                         "largest workload one GPU holds), 4 Llama-70B 1/16 shard, 5 stress "
                         "with clip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step: skip the checkpoint, loss-scaled and "
                         "offload legs that a run on the GPT shard (--workload 2) adds")
    ap.add_argument("--checkpoint", action="store_true",
                    help="also time the state export/import used for checkpoints and resharding")
    ap.add_argument("--amp", action="store_true",
                    help="also time the fp16 loss-scaled variant on the same shard")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps with the Infinity Cache evicted (default for the tiny "
                         "workload)")
    ap.add_argument("--offload", action="store_true",
                    help="also time the optimizer step on host cores with PCIe staging")
    ap.add_argument("--offload-chunk", type=int, default=1 << 24,
                    help="elements per staged chunk of the offloaded step (multiple of 64)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps replayed from one HIP graph (default for the tiny "
                         "workload, which is launch-bound)")
    ap.add_argument("--contiguous", action="store_true",
                    help="take the shard's slab from physically contiguous device memory "
                         "(ZeroShard(contiguous=True))")
    ap.add_argument("--static-step", action="store_true",
                    help="also time the allocation-free entry point (zero_shard_step_static) on "
                         "the same buffers (adds a 'static_step' object)")
    ap.add_argument("--sweep-caps", default="",
                    help="comma-separated step-kernel wave caps (0 = no cap) to time on the "
                         "same buffers after the headline (adds a 'cap_sweep' object)")
    ap.add_argument("--sweep-rounds", type=int, default=3)
    ap.add_argument("--ceiling", action="store_true",
                    help="last, time torch's device copy, a plain copy kernel, a fill and a "
                         "sum on the shard's own slab (adds a 'ceiling' object; overwrites "
                         "the optimizer state)")
    ap.add_argument("--cpu-slab", type=int, default=1 << 25)
    ap.add_argument("--calibrate-copy-gib", type=float, default=1.0,
                    help="size of the plain copy run once before timing (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the multi-GPU "
                                   "exchange (reduce-scatter / all-gather) is not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import synth
    from sharded_optimizer_step_zero_amd import ZeroShard
    from synth.device_case import DeviceCase
    from synth.workloads import special_ranges, workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workload(args.workload)
    t_setup = time.time()
    zs = ZeroShard(w.numel, w.decay, w.world_size, w.rank, w.M, device=dev,
                   bucket_cap=w.bucket_cap, align=w.align, grad_buffers=True,
                   contiguous=args.contiguous)
    segs = zs.segments()
    pad = [(o, n) for o, n, t, _, _ in segs if t < 0]
    special = special_ranges(w, [(o, n, t) for o, n, t, _, _ in segs])
    case = DeviceCase(w, zs.shard_len, pad, dev, special, grads=zs.grads)
    case.fill_master(zs.master)
    # checked once, then passed as plain device addresses: the timed loop measures the
    # library call, not the binding's per-call tensor checks
    grads = zs.grad_pointers(case.fill_grads(0))
    stream = torch.cuda.current_stream(dev)
    zs.set_stream(stream.cuda_stream)

    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * (1 << 30)) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        synth.dev_copy(b, a)
        del a, b
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    clip = w.max_grad_norm > 0
    for s in range(args.warmup):
        zs.step(grads, step=s + 1, max_grad_norm=w.max_grad_norm, **hp)
    torch.cuda.synchronize()

    # the timed steps, bracketed by two events (an event per step would add its own
    # host cost to every step, which a 1M-parameter step cannot hide)
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    for s in range(args.steps):
        zs.step(grads, step=args.warmup + s + 1, max_grad_norm=w.max_grad_norm, **hp)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e_start.elapsed_time(e_end)
    ms_per_step = gpu_ms / args.steps

    # the per-step spread, from a second run of up to 50 steps with an event between
    # consecutive steps
    n_spread = min(args.steps, 50)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
    evs[0].record(stream)
    for s in range(n_spread):
        zs.step(grads, step=args.warmup + args.steps + s + 1, max_grad_norm=w.max_grad_norm,
                **hp)
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    per_step = percentiles([evs[i].elapsed_time(evs[i + 1]) for i in range(n_spread)])

    cold = None
    if args.cold or w.name.startswith("tiny"):
        cold = time_cold(zs, grads, w, hp, stream, args.warmup + args.steps + n_spread + 1,
                         max(args.steps // 4, 5))

    # the step kernel alone (per-launch average): when clipping, the norm pass is
    # timed separately and removed
    step_kernel_ms = ms_per_step
    if clip:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            zs.step(grads, step=s + 1, max_grad_norm=0.0, **hp)
        e1.record(stream)
        torch.cuda.synchronize()
        step_kernel_ms = e0.elapsed_time(e1) / args.steps

    S = zs.shard_len
    by = algorithmic_bytes(S, w.M, clip)
    achieved = by["step_kernel"] / (step_kernel_ms * 1e-3) / 1e9
    traffic = traffic_for(w.name)

    out = {
        "metric": METRIC,
        "value": S / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "slab": "physically contiguous" if args.contiguous else "ordinary device memory",
            "shard_params": S,
            "M": w.M,
            "world_size": w.world_size,
            "rank": w.rank,
            "tensors": len(w.numel),
            "clip": w.max_grad_norm if clip else None,
            "bytes_per_param": 2 * w.M + 12 + 14 + (2 * w.M if clip else 0),
            "hbm_gbs_whole_step": by["total"] / (ms_per_step * 1e-3) / 1e9,
            "pct_of_peak_whole_step": 100.0 * by["total"] / (ms_per_step * 1e-3) / 1e9
                                      / PEAK_HBM_GBS,
            "per_step_ms": per_step,
            "cold_per_step_ms": cold,
            "wall_s_timed": wall,
            "setup_s": setup_s,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "zs::step_kernel<M=%d>" % w.M,
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": by["step_kernel"],
            "avg_launch_ms": step_kernel_ms,
        },
        "cpu_baseline": None,
    }
    if args.static_step:
        out["static_step"] = time_static(zs, grads, w, hp, stream, args.steps,
                                         args.warmup + args.steps + n_spread + 1)
    if args.sweep_caps:
        out["cap_sweep"] = sweep_caps(zs, grads, w, hp, stream,
                                      [int(c) for c in args.sweep_caps.split(",")],
                                      args.sweep_rounds, max(args.steps // 2, 3))
    if args.graph or w.name.startswith("tiny") or (not args.no_extras and args.workload == 2):
        out["graph"] = time_graph(zs, grads, w, hp, args.steps,
                                  args.warmup + args.steps + n_spread + 1)
    # a run on the GPT shard adds the follow-on paths' legs
    extras = not args.no_extras and args.workload == 2
    if args.checkpoint or extras:
        out["checkpoint"] = time_checkpoint(zs, w, stream)
    if args.amp or extras:
        out["amp_fp16"] = time_amp(w, pad, dev, stream, args.steps, args.warmup)
        out["amp_fp16_staged"] = time_amp(w, pad, dev, stream, args.steps, args.warmup, True)
    if args.offload or extras:
        out["offload"] = time_offload(w, pad, dev, stream, max(3, args.steps // 20), 2,
                                      args.offload_chunk)
        out["offload_fp16"] = time_offload(w, pad, dev, stream, max(3, args.steps // 20), 2,
                                           args.offload_chunk, fp16=True)
    if args.ceiling:
        out["ceiling"] = time_ceiling(zs, stream, max(args.steps, 5))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_slab, S))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
