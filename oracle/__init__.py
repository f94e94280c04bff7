"""CPU oracle for the per-rank ZeRO shard step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition the GPU path is checked against: ``zo.c`` (the step, the M-way
reduce, the fp64 norm, bf16 conversion) and ``layout.py`` (the flat bucket /
shard layout).  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import it.  The product library never
imports, links or calls anything here, and nothing here imports the product.

Every function here is pinned by tests under ``tests/`` against closed forms,
invariants, library routines (torch AdamW, clip_grad_norm_, torch bf16
conversion) and the pages' worked numbers; see the test modules named
``test_oracle_*``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import layout  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libzo.so")
SOURCES = [os.path.join(_HERE, "zo.c")]
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile zo.c into libzo.so with gcc (no FMA contraction, no fast-math)."""
    import subprocess
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", *SOURCES, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        _lib = _load(LIB)
    return _lib


def use_library(path: str = None) -> None:
    """Point every function here at another build of zo.c (the mutation tests use
    deliberately broken builds); None returns to libzo.so."""
    global _lib
    _lib = _load(path) if path else None


def _load(path: str):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    vp, i64, i32, f32, f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                              ctypes.c_float, ctypes.c_double)
    L.zo_bf16_to_f32_array.argtypes = [i64, vp, vp]
    L.zo_bf16_to_f32_array.restype = None
    L.zo_f32_to_bf16_array.argtypes = [i64, vp, vp]
    L.zo_f32_to_bf16_array.restype = None
    L.zo_set_threads.argtypes = [i32]
    L.zo_set_threads.restype = None
    L.zo_get_threads.argtypes = []
    L.zo_get_threads.restype = i32
    L.zo_scalars_f32_get.argtypes = [f32, f32, f32, f32, f32, i64, vp]
    L.zo_scalars_f32_get.restype = None
    L.zo_reduce_mean_f32.argtypes = [i64, i32, vp, vp]
    L.zo_reduce_mean_f32.restype = None
    L.zo_grad_sumsq.argtypes = [i64, i32, vp]
    L.zo_grad_sumsq.restype = f64
    L.zo_clip_coef.argtypes = [f64, f32]
    L.zo_clip_coef.restype = f32
    L.zo_coef_from_norm.argtypes = [f64, f32]
    L.zo_coef_from_norm.restype = f32
    L.zo_step_f32.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, f32, f32, f32, f32, f32,
                              i64, i32, f32]
    L.zo_step_f32.restype = i32
    L.zo_step_f64.argtypes = [i64, i32, vp, vp, vp, vp, vp, f64, f64, f64, f64, f64, i64,
                              i32, f64]
    L.zo_step_f64.restype = i32
    L.zo_f16_to_f32_array.argtypes = [i64, vp, vp]
    L.zo_f16_to_f32_array.restype = None
    L.zo_f32_to_f16_array.argtypes = [i64, vp, vp]
    L.zo_f32_to_f16_array.restype = None
    L.zo_pow_int.argtypes = [f64, i64]
    L.zo_pow_int.restype = f64
    L.zo_inv_scale.argtypes = [f32]
    L.zo_inv_scale.restype = f32
    L.zo_reduce_mean_f16.argtypes = [i64, i32, vp, f32, vp]
    L.zo_reduce_mean_f16.restype = None
    L.zo_grad_sumsq_f16.argtypes = [i64, i32, vp, f32]
    L.zo_grad_sumsq_f16.restype = f64
    L.zo_step_f16.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, f32, f32, f32, f32, f32, i64,
                              f32, i32, f32]
    L.zo_step_f16.restype = i32
    L.zo_scaler_update.argtypes = [vp, vp, i32, f32, f32, i32]
    L.zo_scaler_update.restype = None
    L.zo_amp_step.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, f32, f32, f32, f32, f32, f32,
                              vp, vp, vp, f32, f32, i32, vp]
    L.zo_amp_step.restype = i32
    return L


def set_threads(n: int) -> None:
    lib().zo_set_threads(int(n))


def get_threads() -> int:
    return int(lib().zo_get_threads())


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def _grads_u16(grads):
    gs = [np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    n = gs[0].size
    if any(g.size != n for g in gs):
        raise ValueError("gradient contributions differ in length")
    return gs, n


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.size, dtype=np.float32)
    lib().zo_bf16_to_f32_array(h.size, h.ctypes.data, out.ctypes.data)
    return out.reshape(h.shape)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().zo_f32_to_bf16_array(x.size, x.ctypes.data, out.ctypes.data)
    return out.reshape(x.shape)


def step_scalars_f32(lr, beta1, beta2, eps, wd, t) -> dict:
    out = np.empty(8, dtype=np.float32)
    lib().zo_scalars_f32_get(lr, beta1, beta2, eps, wd, int(t), out.ctypes.data)
    names = ["beta1", "beta2", "c1", "c2", "alpha", "bhat", "eps", "decay_mul"]
    return dict(zip(names, out.tolist()))


def pow_int(b: float, t: int) -> float:
    return float(lib().zo_pow_int(float(b), int(t)))


def reduce_mean_f32(grads) -> np.ndarray:
    gs, n = _grads_u16(grads)
    out = np.empty(n, dtype=np.float32)
    lib().zo_reduce_mean_f32(n, len(gs), _ptr_array(gs), out.ctypes.data)
    return out


def grad_sumsq(grads) -> float:
    gs, n = _grads_u16(grads)
    return float(lib().zo_grad_sumsq(n, len(gs), _ptr_array(gs)))


def clip_coef(sumsq: float, max_norm: float) -> np.float32:
    return np.float32(lib().zo_clip_coef(float(sumsq), float(max_norm)))


def coef_from_norm(norm: float, max_norm: float) -> np.float32:
    return np.float32(lib().zo_coef_from_norm(float(norm), float(max_norm)))


def step_f32(grads, master, m, v, param=None, decay=None, *, lr, beta1, beta2, eps,
             weight_decay, step, coef=None):
    """One fp32 oracle step, in place on master/m/v (float32 arrays); writes param
    (uint16 bf16 patterns) when given.  coef: clip coefficient applied to g."""
    gs, n = _grads_u16(grads)
    for a in (master, m, v):
        if a.dtype != np.float32 or not a.flags.c_contiguous or a.size != n:
            raise ValueError("master/m/v must be contiguous float32 of the shard length")
    if param is not None and (param.dtype != np.uint16 or param.size != n
                              or not param.flags.c_contiguous):
        raise ValueError("param must be contiguous uint16 of the shard length")
    if decay is not None:
        decay = np.ascontiguousarray(decay, dtype=np.uint8)
        if decay.size != n:
            raise ValueError("decay mask length")
    rc = lib().zo_step_f32(n, len(gs), _ptr_array(gs), master.ctypes.data, m.ctypes.data,
                           v.ctypes.data, None if param is None else param.ctypes.data,
                           None if decay is None else decay.ctypes.data, lr, beta1, beta2, eps,
                           weight_decay, int(step), 0 if coef is None else 1,
                           0.0 if coef is None else float(coef))
    if rc != 0:
        raise ValueError("zo_step_f32 rejected its arguments")


def step_f64(grads, master, m, v, decay=None, *, lr, beta1, beta2, eps, weight_decay, step,
             coef=None):
    """The same formula in fp64 (grads: list of float64 arrays), in place."""
    gs = [np.ascontiguousarray(g, dtype=np.float64) for g in grads]
    n = gs[0].size
    for a in (master, m, v):
        if a.dtype != np.float64 or not a.flags.c_contiguous or a.size != n:
            raise ValueError("master/m/v must be contiguous float64")
    if decay is not None:
        decay = np.ascontiguousarray(decay, dtype=np.uint8)
    rc = lib().zo_step_f64(n, len(gs), _ptr_array(gs), master.ctypes.data, m.ctypes.data,
                           v.ctypes.data, None if decay is None else decay.ctypes.data, lr,
                           beta1, beta2, eps, weight_decay, int(step),
                           0 if coef is None else 1, 0.0 if coef is None else float(coef))
    if rc != 0:
        raise ValueError("zo_step_f64 rejected its arguments")


# ------------------------------------------- fp16 with dynamic loss scaling


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.size, dtype=np.float32)
    lib().zo_f16_to_f32_array(h.size, h.ctypes.data, out.ctypes.data)
    return out.reshape(h.shape)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().zo_f32_to_f16_array(x.size, x.ctypes.data, out.ctypes.data)
    return out.reshape(x.shape)


def inv_scale(scale: float) -> np.float32:
    return np.float32(lib().zo_inv_scale(float(scale)))


def reduce_mean_f16(grads, inv: float) -> np.ndarray:
    gs, n = _grads_u16(grads)
    out = np.empty(n, dtype=np.float32)
    lib().zo_reduce_mean_f16(n, len(gs), _ptr_array(gs), float(inv), out.ctypes.data)
    return out


def grad_sumsq_f16(grads, inv: float) -> float:
    gs, n = _grads_u16(grads)
    return float(lib().zo_grad_sumsq_f16(n, len(gs), _ptr_array(gs), float(inv)))


def step_f16(grads, master, m, v, param=None, decay=None, *, lr, beta1, beta2, eps,
             weight_decay, step, inv_scale, coef=None):
    """One fp32 step on fp16 contributions (uint16 fp16 patterns), unscaled by
    inv_scale; writes the fp16 param copy when given."""
    gs, n = _grads_u16(grads)
    for a in (master, m, v):
        if a.dtype != np.float32 or not a.flags.c_contiguous or a.size != n:
            raise ValueError("master/m/v must be contiguous float32 of the shard length")
    if decay is not None:
        decay = np.ascontiguousarray(decay, dtype=np.uint8)
    rc = lib().zo_step_f16(n, len(gs), _ptr_array(gs), master.ctypes.data, m.ctypes.data,
                           v.ctypes.data, None if param is None else param.ctypes.data,
                           None if decay is None else decay.ctypes.data, lr, beta1, beta2, eps,
                           weight_decay, int(step), float(inv_scale), 0 if coef is None else 1,
                           0.0 if coef is None else float(coef))
    if rc != 0:
        raise ValueError("zo_step_f16 rejected its arguments")


class Scaler:
    """Dynamic loss-scale state: fp32 scale, int32 growth count, and the number of
    optimizer steps actually applied (skipped steps do not count, so the bias
    correction of the next applied step uses t = applied + 1)."""

    def __init__(self, scale=65536.0, growth_factor=2.0, backoff_factor=0.5, growth_interval=2000):
        self.scale = np.array([scale], np.float32)
        self.tracker = np.array([0], np.int32)
        self._applied = np.array([0], np.int64)
        self.growth_factor = growth_factor
        self.backoff_factor = backoff_factor
        self.growth_interval = growth_interval

    @property
    def applied(self) -> int:
        return int(self._applied[0])

    def update(self, found_inf: bool) -> None:
        lib().zo_scaler_update(self.scale.ctypes.data, self.tracker.ctypes.data,
                               1 if found_inf else 0, self.growth_factor, self.backoff_factor,
                               self.growth_interval)


def amp_step(grads, master, m, v, param, decay, scaler: Scaler, *, lr, beta1, beta2, eps,
             weight_decay, max_grad_norm=0.0):
    """The whole fp16 step (zo_amp_step): unscale, found-inf (a non-finite sum of
    squares of the unscaled average), optional clip on the unscaled norm, the
    update (at t = applied + 1) unless found-inf, then the scale update.
    Returns (found_inf, norm); norm is NaN when found-inf."""
    gs, n = _grads_u16(grads)
    for a in (master, m, v):
        if a.dtype != np.float32 or not a.flags.c_contiguous or a.size != n:
            raise ValueError("master/m/v must be contiguous float32 of the shard length")
    if decay is not None:
        decay = np.ascontiguousarray(decay, dtype=np.uint8)
    norm = np.zeros(1, np.float64)
    rc = lib().zo_amp_step(n, len(gs), _ptr_array(gs), master.ctypes.data, m.ctypes.data,
                           v.ctypes.data, None if param is None else param.ctypes.data,
                           None if decay is None else decay.ctypes.data, lr, beta1, beta2, eps,
                           weight_decay, float(max_grad_norm), scaler.scale.ctypes.data,
                           scaler.tracker.ctypes.data, scaler._applied.ctypes.data,
                           scaler.growth_factor, scaler.backoff_factor, scaler.growth_interval,
                           norm.ctypes.data)
    if rc < 0:
        raise ValueError("zo_amp_step rejected its arguments")
    found_inf = rc == 1
    return found_inf, float("nan") if found_inf else float(norm[0])
