"""Python binding of libzeroshard.so: the fused per-rank ZeRO shard step on MI355X.

Every C entry point of include/zeroshard.h is exposed under the same name; the
functions here only marshal arguments (ints for device pointers, numpy/lists
for host arrays) and turn negative return codes into ZeroShardError.  All the
work of a step runs in the HIP kernels of the library.  There is no fallback:
importing this package without the built library raises ImportError.

``ZeroShard`` is a convenience owner for tests and benchmarks: it builds a
plan, allocates the rank's buffers with torch on a device and binds a context
to them.  PyTorch supplies device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzeroshard.so")

ZS_OK = 0
ZS_NONFINITE = 1
ZS_EINVAL = -1
ZS_ENOMEM = -2
ZS_EHIP = -3
ZS_ESTATE = -4
ZS_SKIP_NONFINITE = 1
ZS_FP16 = 2
ZS_STAGE_AVERAGE = 4
ZS_MAX_M = 16
ZS_STATIC_SCRATCH_BYTES = 8 << 20

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(there is no fallback implementation)")

# A process must use one HIP runtime.  PyTorch bundles its own libamdhip64
# (same soname, libamdhip64.so.7); loading torch first makes this library bind
# to that copy instead of mapping a second runtime that then sees no device.
try:
    import torch  # noqa: F401
except ImportError:  # no torch in the process: the system ROCm runtime is used
    pass

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _u32, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_uint32, ctypes.c_float, ctypes.c_double,
                                          ctypes.c_size_t)
_P = ctypes.POINTER


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_sig("zs_plan_create", ctypes.c_int, _vp, _vp, _i64, _i32, _i32, _i64, _i32, _P(_vp))
_sig("zs_plan_query", ctypes.c_int, _vp, _P(_i64), _P(_i64), _P(_i64), _P(_i64), _P(_i64))
_sig("zs_plan_tensor_slice", ctypes.c_int, _vp, _i64, _P(_i64), _P(_i64), _P(_i64))
_sig("zs_plan_segment", ctypes.c_int, _vp, _i64, _P(_i64), _P(_i64), _P(_i64), _P(_i64),
     _P(_i32))
_sig("zs_plan_bucket", ctypes.c_int, _vp, _i64, _P(_i64), _P(_i64))
_sig("zs_plan_run", ctypes.c_int, _vp, _i64, _P(_i64), _P(_i64), _P(_i32))
_sig("zs_plan_state_bytes", ctypes.c_int, _vp, _i32, _P(_i64))
_sig("zs_plan_destroy", None, _vp)
_sig("zs_workspace_bytes", _sz, _vp, _i32, _u32)
_sig("zs_slab_layout", ctypes.c_int, _vp, _i32, _u32, _i32, _P(_sz), _P(_sz))
_sig("zero_shard_init", ctypes.c_int, _P(_vp), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
     _u32)
_sig("zero_shard_step", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _i64, _f32,
     _P(_f64))
_sig("zero_shard_grad_sumsq", ctypes.c_int, _vp, _vp, _vp)
_sig("zero_shard_step_global_norm", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _i64,
     _f32, _vp)
_sig("zero_shard_amp_state_init", ctypes.c_int, _vp, _vp, _f32)
_sig("zero_shard_step_amp", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _f32, _vp, _f32,
     _f32, _i32, _P(_f64))
_sig("zero_shard_grad_sumsq_amp", ctypes.c_int, _vp, _vp, _vp, _vp)
_sig("zero_shard_step_amp_global_norm", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _f32,
     _vp, _f32, _f32, _i32, _vp)
_sig("zero_shard_export_state", ctypes.c_int, _vp, _vp, _vp, _vp)
_sig("zero_shard_import_state", ctypes.c_int, _vp, _vp, _vp, _vp)
_sig("zero_shard_params", ctypes.c_int, _vp, _P(_vp), _P(_i64))
_sig("zero_shard_set_stream", ctypes.c_int, _vp, _vp)
_sig("zero_shard_destroy", None, _vp)
_sig("zero_shard_step_static", ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _f32, _f32, _f32,
     _f32, _f32, _i64, _f32, _vp)
_sig("zero_shard_last_error", ctypes.c_char_p)
_sig("zs_host_adamw", ctypes.c_int, _vp, _i64, _i64, _vp, _f32, _vp, _vp, _vp, _vp, _f32, _f32,
     _f32, _f32, _f32, _i64, _i32, _u32)
_sig("zs_offload_staging_bytes", _sz, _i64)
_sig("zero_offload_init", ctypes.c_int, _P(_vp), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
     _sz, _i64, _i32, _vp, _u32)
_sig("zero_offload_step", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _i64, _f32,
     _P(_f64))
_sig("zero_offload_step_amp", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _f32, _vp,
     _f32, _f32, _i32, _P(_f64))
_sig("zero_offload_grad_sumsq", ctypes.c_int, _vp, _vp, _vp)
_sig("zero_offload_step_global_norm", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32, _i64,
     _f32, _vp)
_sig("zero_offload_grad_sumsq_amp", ctypes.c_int, _vp, _vp, _vp, _vp)
_sig("zero_offload_step_amp_global_norm", ctypes.c_int, _vp, _vp, _f32, _f32, _f32, _f32, _f32,
     _f32, _vp, _f32, _f32, _i32, _vp)
_sig("zero_offload_amp_state_init", ctypes.c_int, _vp, _vp, _f32)
_sig("zero_offload_set_stream", ctypes.c_int, _vp, _vp)
_sig("zero_offload_destroy", None, _vp)
_sig("zs_device_alloc_contiguous", _vp, ctypes.c_size_t, _i32, _vp)
_sig("zs_device_free", None, _vp, ctypes.c_size_t, _i32, _vp)

EXPORTED = ["zs_plan_create", "zs_plan_query", "zs_plan_tensor_slice", "zs_plan_segment",
            "zs_plan_bucket", "zs_plan_run", "zs_plan_state_bytes", "zs_plan_destroy",
            "zs_workspace_bytes", "zs_slab_layout", "zero_shard_init", "zero_shard_step",
            "zero_shard_grad_sumsq", "zero_shard_step_global_norm", "zero_shard_amp_state_init",
            "zero_shard_step_amp", "zero_shard_grad_sumsq_amp", "zero_shard_step_amp_global_norm",
            "zero_shard_export_state", "zero_shard_import_state", "zero_shard_params",
            "zero_shard_set_stream", "zero_shard_destroy", "zero_shard_last_error",
            "zero_shard_step_static", "zs_host_adamw", "zs_offload_staging_bytes",
            "zero_offload_init", "zero_offload_step", "zero_offload_step_amp",
            "zero_offload_grad_sumsq", "zero_offload_step_global_norm",
            "zero_offload_grad_sumsq_amp", "zero_offload_step_amp_global_norm",
            "zero_offload_amp_state_init", "zero_offload_set_stream", "zero_offload_destroy",
            "zs_device_alloc_contiguous", "zs_device_free"]


class ZeroShardError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


def zero_shard_last_error() -> str:
    return _lib.zero_shard_last_error().decode()


def _check(rc):
    if rc < 0:
        raise ZeroShardError(rc, zero_shard_last_error())
    return rc


def _int64_array(xs):
    return (ctypes.c_int64 * len(xs))(*[int(x) for x in xs])


def _ptr_array(ptrs):
    return (ctypes.c_void_p * max(1, len(ptrs)))(*[int(p) for p in ptrs])


# M of every live context, by handle: the library reads exactly M gradient
# pointers, so a shorter list would make it read past the pointer array
_CTX_M = {}


def _grad_array(ctx, grads):
    M = _CTX_M.get(ctx)
    if M is not None and len(grads) != M:
        raise ValueError(f"the context takes exactly {M} gradient contributions, got {len(grads)}")
    return _ptr_array(grads)


# ------------------------------------------------------------------ plan


def zs_plan_create(numel: Sequence[int], decay: Sequence[int], world_size: int, rank: int,
                   bucket_cap: int = 25_000_000, align: int = 64) -> int:
    """Returns an opaque plan handle (int)."""
    n = len(numel)
    nb = _int64_array(numel)
    db = (ctypes.c_uint8 * max(1, n))(*[1 if d else 0 for d in decay])
    if len(decay) != n:
        raise ValueError("numel and decay differ in length")
    out = ctypes.c_void_p()
    _check(_lib.zs_plan_create(nb if n else None, db if n else None, n, world_size, rank,
                               bucket_cap, align, ctypes.byref(out)))
    return out.value


def zs_plan_query(plan: int) -> dict:
    v = [ctypes.c_int64() for _ in range(5)]
    _check(_lib.zs_plan_query(plan, *[ctypes.byref(x) for x in v]))
    keys = ["shard_len", "n_segments", "n_runs", "padded_total", "n_buckets"]
    return {k: x.value for k, x in zip(keys, v)}


def zs_plan_tensor_slice(plan: int, tensor: int):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.zs_plan_tensor_slice(plan, tensor, ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c)))
    return a.value, b.value, c.value


def zs_plan_segment(plan: int, i: int):
    a, b, c, d = (ctypes.c_int64() for _ in range(4))
    e = ctypes.c_int32()
    _check(_lib.zs_plan_segment(plan, i, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                ctypes.byref(d), ctypes.byref(e)))
    return a.value, b.value, c.value, d.value, e.value


def zs_plan_bucket(plan: int, b: int):
    x, y = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.zs_plan_bucket(plan, b, ctypes.byref(x), ctypes.byref(y)))
    return x.value, y.value


def zs_plan_run(plan: int, i: int):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(_lib.zs_plan_run(plan, i, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def zs_plan_state_bytes(plan: int, stage: int) -> int:
    x = ctypes.c_int64()
    _check(_lib.zs_plan_state_bytes(plan, stage, ctypes.byref(x)))
    return x.value


def zs_plan_destroy(plan: int) -> None:
    _lib.zs_plan_destroy(plan)


def zs_workspace_bytes(plan: int, M: int, flags: int = 0) -> int:
    return int(_lib.zs_workspace_bytes(plan, M, flags))


def zs_slab_layout(plan: int, M: int, flags: int = 0, n_grads: int = 0):
    """(offsets, slab_bytes): byte offsets of param, master, exp_avg, exp_avg_sq,
    n_grads gradient buffers and the workspace inside one slab."""
    offs = (ctypes.c_size_t * (5 + max(0, min(int(n_grads), 16))))()
    total = ctypes.c_size_t()
    _check(_lib.zs_slab_layout(plan, M, flags, n_grads, offs, ctypes.byref(total)))
    return [int(x) for x in offs], int(total.value)


# ------------------------------------------------------------------ step


def zero_shard_init(plan: int, M: int, param_bf16: int, master: int, exp_avg: int,
                    exp_avg_sq: int, workspace: int, workspace_bytes: int, stream: int = 0,
                    flags: int = 0) -> int:
    """Returns an opaque context handle (int).  Pointers are device addresses."""
    out = ctypes.c_void_p()
    _check(_lib.zero_shard_init(ctypes.byref(out), plan, M, param_bf16, master, exp_avg,
                                exp_avg_sq, workspace, workspace_bytes, stream or None, flags))
    _CTX_M[out.value] = int(M)
    return out.value


def zero_shard_step(ctx: int, grads: Sequence[int], lr: float, beta1: float, beta2: float,
                    eps: float, weight_decay: float, step: int, max_grad_norm: float = 0.0,
                    want_norm: bool = False, return_code: bool = False):
    """Enqueues one step.  Returns the fp64 grad norm when want_norm (the call then
    waits), else None; with return_code, returns (code, norm) -- code is ZS_OK or
    the warning ZS_NONFINITE.  Negative codes raise ZeroShardError."""
    arr = _grad_array(ctx, grads)
    nrm = ctypes.c_double()
    rc = _check(_lib.zero_shard_step(ctx, arr, lr, beta1, beta2, eps, weight_decay, step,
                                     max_grad_norm, ctypes.byref(nrm) if want_norm else None))
    norm = nrm.value if want_norm else None
    return (rc, norm) if return_code else norm


def zero_shard_grad_sumsq(ctx: int, grads: Sequence[int], sumsq_dev: int) -> None:
    _check(_lib.zero_shard_grad_sumsq(ctx, _grad_array(ctx, grads), sumsq_dev))


def zero_shard_step_global_norm(ctx: int, grads: Sequence[int], lr: float, beta1: float,
                                beta2: float, eps: float, weight_decay: float, step: int,
                                max_grad_norm: float, global_sumsq_dev: int) -> None:
    _check(_lib.zero_shard_step_global_norm(ctx, _grad_array(ctx, grads), lr, beta1, beta2, eps,
                                            weight_decay, step, max_grad_norm,
                                            global_sumsq_dev))


def zero_shard_amp_state_init(ctx: int, state_dev: int, init_scale: float) -> None:
    _check(_lib.zero_shard_amp_state_init(ctx, state_dev, init_scale))


def zero_shard_step_amp(ctx: int, grads: Sequence[int], lr: float, beta1: float, beta2: float,
                        eps: float, weight_decay: float, max_grad_norm: float, state_dev: int,
                        growth_factor: float = 2.0, backoff_factor: float = 0.5,
                        growth_interval: int = 2000, want_norm: bool = False,
                        return_code: bool = False):
    """Enqueues one loss-scaled fp16 step (see zeroshard.h).  Returns the unscaled
    norm when want_norm (waits), else None; with return_code, (code, norm)."""
    nrm = ctypes.c_double()
    rc = _check(_lib.zero_shard_step_amp(ctx, _grad_array(ctx, grads), lr, beta1, beta2, eps,
                                         weight_decay, max_grad_norm, state_dev, growth_factor,
                                         backoff_factor, growth_interval,
                                         ctypes.byref(nrm) if want_norm else None))
    norm = nrm.value if want_norm else None
    return (rc, norm) if return_code else norm


def zero_shard_grad_sumsq_amp(ctx: int, grads: Sequence[int], state_dev: int,
                              sumsq_dev: int) -> None:
    """Multi-rank loss-scaled step, part 1: this shard's sum of squares of the
    unscaled average into the device double at sumsq_dev."""
    _check(_lib.zero_shard_grad_sumsq_amp(ctx, _grad_array(ctx, grads), state_dev, sumsq_dev))


def zero_shard_step_amp_global_norm(ctx: int, grads: Sequence[int], lr: float, beta1: float,
                                    beta2: float, eps: float, weight_decay: float,
                                    max_grad_norm: float, state_dev: int,
                                    growth_factor: float = 2.0, backoff_factor: float = 0.5,
                                    growth_interval: int = 2000,
                                    global_sumsq_dev: int = 0) -> None:
    """Part 2: the loss-scaled step decided by the global sum of squares."""
    _check(_lib.zero_shard_step_amp_global_norm(ctx, _grad_array(ctx, grads), lr, beta1, beta2,
                                                eps, weight_decay, max_grad_norm, state_dev,
                                                growth_factor, backoff_factor, growth_interval,
                                                global_sumsq_dev))


def zero_shard_export_state(ctx: int, canon_master: int, canon_exp_avg: int,
                            canon_exp_avg_sq: int) -> None:
    _check(_lib.zero_shard_export_state(ctx, canon_master or None, canon_exp_avg or None,
                                        canon_exp_avg_sq or None))


def zero_shard_import_state(ctx: int, canon_master: int, canon_exp_avg: int,
                            canon_exp_avg_sq: int) -> None:
    _check(_lib.zero_shard_import_state(ctx, canon_master or None, canon_exp_avg or None,
                                        canon_exp_avg_sq or None))


def zero_shard_params(ctx: int):
    p, n = ctypes.c_void_p(), ctypes.c_int64()
    _check(_lib.zero_shard_params(ctx, ctypes.byref(p), ctypes.byref(n)))
    return p.value or 0, n.value


def zero_shard_set_stream(ctx: int, stream: int) -> None:
    _check(_lib.zero_shard_set_stream(ctx, stream or None))


def zero_shard_destroy(ctx: int) -> None:
    _CTX_M.pop(ctx, None)
    _lib.zero_shard_destroy(ctx)


def zero_shard_step_static(plan: int, M: int, param_bf16: int, master: int, exp_avg: int,
                           exp_avg_sq: int, grads: Sequence[int], lr: float, beta1: float,
                           beta2: float, eps: float, weight_decay: float, step: int,
                           max_grad_norm: float = 0.0, stream: int = 0) -> None:
    """Enqueues one bf16 step without a context or workspace: the library's static
    device scratch holds the tables and partials (see zeroshard.h).  Pointers are
    device addresses."""
    if len(grads) != M:
        raise ValueError(f"expected {M} gradient contributions, got {len(grads)}")
    _check(_lib.zero_shard_step_static(plan, M, param_bf16, master, exp_avg, exp_avg_sq,
                                       _ptr_array(grads), lr, beta1, beta2, eps, weight_decay,
                                       step, max_grad_norm, stream or None))


# ------------------------------------------------- the step on host cores


def zs_host_adamw(plan: int, shard_off: int, n: int, grad_avg: int, coef: float, master: int,
                  exp_avg: int, exp_avg_sq: int, param: int, lr: float, beta1: float,
                  beta2: float, eps: float, weight_decay: float, step: int,
                  n_threads: int = 0, flags: int = 0) -> None:
    """The update alone on host arrays (addresses of n-element host arrays); param
    receives bf16, or fp16 with flags=ZS_FP16."""
    _check(_lib.zs_host_adamw(plan, shard_off, n, grad_avg or None, coef, master or None,
                              exp_avg or None, exp_avg_sq or None, param or None, lr,
                              beta1, beta2, eps, weight_decay, step, n_threads, flags))


def zs_offload_staging_bytes(chunk_elems: int) -> int:
    return int(_lib.zs_offload_staging_bytes(chunk_elems))


def zero_offload_init(plan: int, M: int, param_bf16: int, master: int, exp_avg: int,
                      exp_avg_sq: int, workspace: int, workspace_bytes: int, staging: int,
                      staging_bytes: int, chunk_elems: int, n_threads: int = 0, stream: int = 0,
                      flags: int = 0) -> int:
    out = ctypes.c_void_p()
    _check(_lib.zero_offload_init(ctypes.byref(out), plan, M, param_bf16, master, exp_avg,
                                  exp_avg_sq, workspace, workspace_bytes, staging, staging_bytes,
                                  chunk_elems, n_threads, stream or None, flags))
    _CTX_M[out.value] = int(M)
    return out.value


def zero_offload_step(ctx: int, grads: Sequence[int], lr: float, beta1: float, beta2: float,
                      eps: float, weight_decay: float, step: int, max_grad_norm: float = 0.0,
                      want_norm: bool = False, return_code: bool = False):
    """One offloaded step (returns once the host state is updated); results as
    zero_shard_step's."""
    nrm = ctypes.c_double()
    rc = _check(_lib.zero_offload_step(ctx, _grad_array(ctx, grads), lr, beta1, beta2, eps,
                                       weight_decay, step, max_grad_norm,
                                       ctypes.byref(nrm) if want_norm else None))
    norm = nrm.value if want_norm else None
    return (rc, norm) if return_code else norm


def zero_offload_step_amp(ctx: int, grads: Sequence[int], lr: float, beta1: float, beta2: float,
                          eps: float, weight_decay: float, max_grad_norm: float, state_dev: int,
                          growth_factor: float = 2.0, backoff_factor: float = 0.5,
                          growth_interval: int = 2000, want_norm: bool = False,
                          return_code: bool = False):
    """One offloaded loss-scaled step (see zeroshard.h); results as zero_shard_step_amp's."""
    nrm = ctypes.c_double()
    rc = _check(_lib.zero_offload_step_amp(ctx, _grad_array(ctx, grads), lr, beta1, beta2, eps,
                                           weight_decay, max_grad_norm, state_dev, growth_factor,
                                           backoff_factor, growth_interval,
                                           ctypes.byref(nrm) if want_norm else None))
    norm = nrm.value if want_norm else None
    return (rc, norm) if return_code else norm


def zero_offload_grad_sumsq(ctx: int, grads: Sequence[int], sumsq_dev: int) -> None:
    _check(_lib.zero_offload_grad_sumsq(ctx, _grad_array(ctx, grads), sumsq_dev))


def zero_offload_step_global_norm(ctx: int, grads: Sequence[int], lr: float, beta1: float,
                                  beta2: float, eps: float, weight_decay: float, step: int,
                                  max_grad_norm: float, global_sumsq_dev: int) -> None:
    _check(_lib.zero_offload_step_global_norm(ctx, _grad_array(ctx, grads), lr, beta1, beta2,
                                              eps, weight_decay, step, max_grad_norm,
                                              global_sumsq_dev))


def zero_offload_grad_sumsq_amp(ctx: int, grads: Sequence[int], state_dev: int,
                                sumsq_dev: int) -> None:
    _check(_lib.zero_offload_grad_sumsq_amp(ctx, _grad_array(ctx, grads), state_dev, sumsq_dev))


def zero_offload_step_amp_global_norm(ctx: int, grads: Sequence[int], lr: float, beta1: float,
                                      beta2: float, eps: float, weight_decay: float,
                                      max_grad_norm: float, state_dev: int,
                                      growth_factor: float = 2.0, backoff_factor: float = 0.5,
                                      growth_interval: int = 2000,
                                      global_sumsq_dev: int = 0) -> None:
    _check(_lib.zero_offload_step_amp_global_norm(ctx, _grad_array(ctx, grads), lr, beta1, beta2,
                                                  eps, weight_decay, max_grad_norm, state_dev,
                                                  growth_factor, backoff_factor,
                                                  growth_interval, global_sumsq_dev))


def zero_offload_amp_state_init(ctx: int, state_dev: int, init_scale: float) -> None:
    _check(_lib.zero_offload_amp_state_init(ctx, state_dev, init_scale))


def zero_offload_set_stream(ctx: int, stream: int) -> None:
    _check(_lib.zero_offload_set_stream(ctx, stream or None))


def zero_offload_destroy(ctx: int) -> None:
    _CTX_M.pop(ctx, None)
    _lib.zero_offload_destroy(ctx)


# ----------------------------------------------------- convenience owner


def zs_device_alloc_contiguous(nbytes: int, device: int = 0) -> int:
    """Device memory, physically contiguous when available; 0 when none is left."""
    return _lib.zs_device_alloc_contiguous(nbytes, device, None) or 0


def zs_device_free(ptr: int, nbytes: int = 0, device: int = 0) -> None:
    _lib.zs_device_free(ptr, nbytes, device, None)


_CONTIG = None


def _resolve_device(device):
    import torch
    d = torch.device(device if device is not None else "cuda")
    if d.type == "cuda" and d.index is None:
        d = torch.device("cuda", torch.cuda.current_device())
    return d


def _check_tensors(ts, n, dtypes, device, what):
    """Tensors the library will stream over: right dtype and device, contiguous,
    at least n elements.  A plain int is a raw device address the caller vouches
    for and is passed through unchecked."""
    for i, t in enumerate(ts):
        if isinstance(t, int):
            continue
        if t.dtype not in dtypes:
            raise ValueError(f"{what}[{i}]: dtype {t.dtype}, expected one of {dtypes}")
        if t.device != device:
            raise ValueError(f"{what}[{i}]: on {t.device}, the context is on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{what}[{i}]: not contiguous")
        if t.numel() < n:
            raise ValueError(f"{what}[{i}]: {t.numel()} elements, the call reads {n}")


def _contiguous_allocator():
    """The torch pluggable allocator over zs_device_alloc_contiguous / zs_device_free."""
    global _CONTIG
    if _CONTIG is None:
        from torch.cuda.memory import CUDAPluggableAllocator
        _CONTIG = CUDAPluggableAllocator(LIB_PATH, "zs_device_alloc_contiguous", "zs_device_free")
    return _CONTIG


class ZeroShard:
    """One rank's shard: plan + torch-allocated device buffers + bound context.

    The param, master, exp_avg, exp_avg_sq arrays and the workspace are views
    into one device slab placed by zs_slab_layout (array starts staggered by
    4 KiB past 2 MiB boundaries).  With grad_buffers=True the slab also holds the
    M gradient contribution buffers, exposed as `grads` (16-bit, shard_len each;
    the caller fills them before each step).  With contiguous=True the slab comes
    from physically contiguous memory (zs_device_alloc_contiguous, through a
    private torch memory pool released by close())."""

    _PERIOD = 1 << 21

    def __init__(self, numel, decay, world_size=1, rank=0, M=1, device=None, bucket_cap=25_000_000,
                 align=64, flags=0, stream=None, fp16=False, grad_buffers=False, contiguous=False):
        import torch
        self.device = _resolve_device(device)
        self.M = M
        self.total_params = int(sum(int(x) for x in numel))
        self.plan = zs_plan_create(numel, decay, world_size, rank, bucket_cap, align)
        q = zs_plan_query(self.plan)
        self.shard_len = q["shard_len"]
        self.n_runs = q["n_runs"]
        self.fp16 = fp16
        if fp16:
            flags |= ZS_FP16
        half = torch.float16 if fp16 else torch.bfloat16
        n_grads = M if grad_buffers else 0
        offs, total = zs_slab_layout(self.plan, M, flags, n_grads)
        self.ws_bytes = zs_workspace_bytes(self.plan, M, flags)
        # over-allocate one period so the slab can start on a 2 MiB boundary
        self.contiguous = bool(contiguous)
        self._pool = None
        if self.contiguous:
            # a private torch memory pool served by zs_device_alloc_contiguous; it is
            # dropped in close(), which returns the memory
            self._pool = torch.cuda.MemPool(_contiguous_allocator().allocator())
            idx = self.device.index if self.device.index is not None else torch.cuda.current_device()
            with torch.cuda.use_mem_pool(self._pool, idx):
                self.slab = torch.zeros(total + self._PERIOD, dtype=torch.uint8, device=self.device)
        else:
            self.slab = torch.zeros(total + self._PERIOD, dtype=torch.uint8, device=self.device)
        base = (-self.slab.data_ptr()) % self._PERIOD
        S = self.shard_len

        def view(off, nbytes, dtype):
            # an empty shard still gets a few elements: torch gives empty tensors no address
            nbytes = max(nbytes, 8 * torch.empty(0, dtype=dtype).element_size())
            return self.slab[base + off:base + off + nbytes].view(dtype)

        self.param = view(offs[0], 2 * S, half)
        self.master = view(offs[1], 4 * S, torch.float32)
        self.exp_avg = view(offs[2], 4 * S, torch.float32)
        self.exp_avg_sq = view(offs[3], 4 * S, torch.float32)
        self.grads = [view(offs[4 + j], 2 * S, half) for j in range(n_grads)]
        self.workspace = view(offs[4 + n_grads], self.ws_bytes, torch.uint8)
        self.amp_state = None
        self._stream = stream
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        self.ctx = zero_shard_init(self.plan, M, self.param.data_ptr(), self.master.data_ptr(),
                                   self.exp_avg.data_ptr(), self.exp_avg_sq.data_ptr(),
                                   self.workspace.data_ptr(), self.ws_bytes, s, flags)

    def set_stream(self, stream: int):
        zero_shard_set_stream(self.ctx, stream)
        self._stream = stream

    def _grad_ptrs(self, grads):
        import torch
        if len(grads) != self.M:
            raise ValueError(f"expected {self.M} gradient contributions, got {len(grads)}")
        # 16-bit patterns: the context's float type, or an integer view of them
        half = torch.float16 if self.fp16 else torch.bfloat16
        _check_tensors(grads, self.shard_len, (half, torch.int16, torch.uint16), self.device,
                       "grads")
        return [g if isinstance(g, int) else g.data_ptr() for g in grads]

    def grad_pointers(self, grads):
        """The contributions' device addresses after the same checks a step makes; a
        loop that steps many times on the same buffers can pass these plain ints and
        skip the per-call Python checks (as a C caller does)."""
        return self._grad_ptrs(grads)

    def _canon_ptrs(self, ts):
        import torch
        _check_tensors(ts, self.total_params, (torch.float32,), self.device, "canonical state")
        return [t if isinstance(t, int) else t.data_ptr() for t in ts]

    def step(self, grads, *, lr, beta1, beta2, eps, weight_decay, step, max_grad_norm=0.0,
             want_norm=False, return_code=False):
        ptrs = self._grad_ptrs(grads)
        return zero_shard_step(self.ctx, ptrs, lr, beta1, beta2, eps, weight_decay, step,
                               max_grad_norm, want_norm, return_code)

    def _amp_buffer(self):
        """The 16-byte scaler state, allocated once (it keeps its address, so graphs
        captured with it stay valid).  Allocated without a fill: the initialiser
        writes all 16 bytes on the context's stream, where a fill kernel on torch's
        current stream could land after it.  torch's current stream is drained once,
        so no earlier work there still touches the recycled block."""
        import torch
        if self.amp_state is None:
            self.amp_state = torch.empty(2, dtype=torch.int64, device=self.device)
            torch.cuda.current_stream(self.device).synchronize()
        return self.amp_state

    def amp_init(self, init_scale=65536.0):
        """(Re)initialise the device loss-scaler state to {scale, 0, 0}, enqueued on
        the context's stream (zero_shard_amp_state_init)."""
        zero_shard_amp_state_init(self.ctx, self._amp_buffer().data_ptr(), init_scale)

    def amp_read(self):
        """(scale, growth_tracker, applied_steps) from the device state (waits for the
        device)."""
        import numpy as np
        import torch
        torch.cuda.synchronize(self.device)
        raw = self.amp_state.cpu().numpy()
        head = raw[:1].view(np.float32)
        return float(head[0]), int(raw[:1].view(np.int32)[1]), int(raw[1])

    def step_amp(self, grads, *, lr, beta1, beta2, eps, weight_decay, max_grad_norm=0.0,
                 growth_factor=2.0, backoff_factor=0.5, growth_interval=2000, want_norm=False,
                 return_code=False):
        ptrs = self._grad_ptrs(grads)
        return zero_shard_step_amp(self.ctx, ptrs, lr, beta1, beta2, eps, weight_decay,
                                   max_grad_norm, self.amp_state.data_ptr(), growth_factor,
                                   backoff_factor, growth_interval, want_norm, return_code)

    def export_state(self, canon_master, canon_exp_avg, canon_exp_avg_sq):
        """Copy this rank's state into canonical device tensors (sum(numel) floats each)."""
        zero_shard_export_state(self.ctx, *self._canon_ptrs(
            [canon_master, canon_exp_avg, canon_exp_avg_sq]))

    def import_state(self, canon_master, canon_exp_avg, canon_exp_avg_sq):
        zero_shard_import_state(self.ctx, *self._canon_ptrs(
            [canon_master, canon_exp_avg, canon_exp_avg_sq]))

    def segments(self):
        n = zs_plan_query(self.plan)["n_segments"]
        return [zs_plan_segment(self.plan, i) for i in range(n)]

    def close(self):
        if getattr(self, "ctx", None):
            zero_shard_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "plan", None):
            zs_plan_destroy(self.plan)
            self.plan = None
        if getattr(self, "_pool", None) is not None:
            # a contiguous slab: wait for queued work, drop this object's views and the
            # private pool; the memory returns once no tensor uses it
            import torch
            torch.cuda.synchronize(self.device)
            self.param = self.master = self.exp_avg = self.exp_avg_sq = None
            self.grads, self.workspace, self.slab = [], None, None
            self._pool = None
            torch.cuda.empty_cache()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ZeroOffload:
    """One rank's shard with the optimizer state in host memory: plan, device
    param and workspace, host master/m/v and pinned staging (all torch-allocated),
    and the bound offload context."""

    def __init__(self, numel, decay, world_size=1, rank=0, M=1, device=None, bucket_cap=25_000_000,
                 align=64, flags=0, stream=None, chunk_elems=1 << 24, n_threads=0, fp16=False):
        import torch
        self.device = _resolve_device(device)
        self.M = M
        self.plan = zs_plan_create(numel, decay, world_size, rank, bucket_cap, align)
        q = zs_plan_query(self.plan)
        self.shard_len = S = q["shard_len"]
        n = max(S, 8)
        self.fp16 = fp16
        if fp16:
            flags |= ZS_FP16
        self.amp_state = None
        self.param = torch.zeros(n, dtype=torch.float16 if fp16 else torch.bfloat16,
                                 device=self.device)
        self.master = torch.zeros(n, dtype=torch.float32)
        self.exp_avg = torch.zeros(n, dtype=torch.float32)
        self.exp_avg_sq = torch.zeros(n, dtype=torch.float32)
        self.ws_bytes = zs_workspace_bytes(self.plan, M, ZS_STAGE_AVERAGE)
        self.workspace = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.chunk = chunk_elems
        self.staging_bytes = zs_offload_staging_bytes(chunk_elems)
        self.staging = torch.empty(max(self.staging_bytes, 256), dtype=torch.uint8, pin_memory=True)
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        self.ctx = zero_offload_init(self.plan, M, self.param.data_ptr(), self.master.data_ptr(),
                                     self.exp_avg.data_ptr(), self.exp_avg_sq.data_ptr(),
                                     self.workspace.data_ptr(), self.ws_bytes,
                                     self.staging.data_ptr(), self.staging_bytes, chunk_elems,
                                     n_threads, s, flags)

    def set_stream(self, stream: int):
        zero_offload_set_stream(self.ctx, stream)

    _grad_ptrs = ZeroShard._grad_ptrs
    _amp_buffer = ZeroShard._amp_buffer
    amp_read = ZeroShard.amp_read

    def step(self, grads, *, lr, beta1, beta2, eps, weight_decay, step, max_grad_norm=0.0,
             want_norm=False, return_code=False):
        ptrs = self._grad_ptrs(grads)
        return zero_offload_step(self.ctx, ptrs, lr, beta1, beta2, eps, weight_decay, step,
                                 max_grad_norm, want_norm, return_code)

    def amp_init(self, init_scale=65536.0):
        """(Re)initialise the device loss-scaler state to {scale, 0, 0} (a stable
        16-byte buffer), enqueued on the context's device stream
        (zero_offload_amp_state_init)."""
        zero_offload_amp_state_init(self.ctx, self._amp_buffer().data_ptr(), init_scale)

    def step_amp(self, grads, *, lr, beta1, beta2, eps, weight_decay, max_grad_norm=0.0,
                 growth_factor=2.0, backoff_factor=0.5, growth_interval=2000, want_norm=False,
                 return_code=False):
        ptrs = self._grad_ptrs(grads)
        return zero_offload_step_amp(self.ctx, ptrs, lr, beta1, beta2, eps, weight_decay,
                                     max_grad_norm, self.amp_state.data_ptr(), growth_factor,
                                     backoff_factor, growth_interval, want_norm, return_code)

    def segments(self):
        n = zs_plan_query(self.plan)["n_segments"]
        return [zs_plan_segment(self.plan, i) for i in range(n)]

    def close(self):
        if getattr(self, "ctx", None):
            zero_offload_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "plan", None):
            zs_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
