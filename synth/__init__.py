"""Seeded synthetic inputs for the ZeRO shard step (test/benchmark infrastructure).

This package makes inputs only; it holds none of the optimizer's arithmetic.
Both the product path's tests/benchmark and the CPU oracle's tests draw from it,
so the two sides see the same bits.  The generator is defined in
``synth_host.c`` (host, OpenMP) and ``synth_dev.hip`` (device); they are
bit-identical for every index, so a multi-GB input can be made in HBM while
any sampled element can be regenerated on the host.

Values are addressed by (seed, stream, index):
  * stream 0             -- fp32 master weights, ~N(0, sigma_master)
  * stream 1 + j + M*s   -- bf16 gradient contribution j of step s (0-based)
  * stream 0x10000 + ... -- the matching "kind" selector stream (zero /
                            subnormal / outlier), used by the stress workload
The index is the element's offset in the rank's flat shard.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Standard deviation of the sum of four independent uniforms on 0..65535.
IH_STD = math.sqrt((65536.0 ** 2 - 1.0) / 3.0)
SEL_STREAM = 0x10000


def scale_for(sigma: float) -> np.float32:
    """fp32 multiplier turning the centred Irwin-Hall integer into ~N(0, sigma)."""
    return np.float32(sigma / IH_STD)


_host = None
_dev = None


def _u64(x: int) -> ctypes.c_uint64:
    return ctypes.c_uint64(x & 0xFFFFFFFFFFFFFFFF)


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_hash.restype = ctypes.c_uint64
        lib.synth_hash.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                         ctypes.c_int64, ctypes.c_float]
        lib.synth_normal_f32_at.restype = None
        lib.synth_normal_f32_at.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_uint64, ctypes.c_float]
        lib.synth_grad_bf16.restype = None
        lib.synth_grad_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_uint64, ctypes.c_int64, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_uint32]
        lib.synth_grad_bf16_at.restype = None
        lib.synth_grad_bf16_at.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_uint32, ctypes.c_uint32,
                                           ctypes.c_uint32]
        lib.synth_grad_f16.restype = None
        lib.synth_grad_f16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_int64, ctypes.c_float, ctypes.c_float]
        lib.synth_grad_f16_at.restype = None
        lib.synth_grad_f16_at.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_uint64, ctypes.c_float, ctypes.c_float]
        _host = lib
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (share torch's HIP runtime; see the product binding)
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        vp, i64, u64, f32, u32, i32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_float, ctypes.c_uint32, ctypes.c_int32)
        lib.synth_dev_normal_f32.argtypes = [vp, i64, u64, i64, f32, vp]
        lib.synth_dev_grad_bf16.argtypes = [vp, i64, u64, u64, i64, f32, f32, u32, u32, u32, vp]
        lib.synth_dev_zero_ranges.argtypes = [vp, i32, vp, i64, vp]
        lib.synth_dev_gather.argtypes = [vp, vp, i32, vp, i64, vp]
        lib.synth_dev_scatter.argtypes = [vp, vp, i32, vp, i64, vp]
        lib.synth_dev_copy16.argtypes = [vp, vp, i64, vp]
        lib.synth_dev_grad_f16.argtypes = [vp, i64, u64, i64, f32, f32, vp]
        for f in (lib.synth_dev_normal_f32, lib.synth_dev_grad_bf16, lib.synth_dev_zero_ranges,
                  lib.synth_dev_gather, lib.synth_dev_scatter, lib.synth_dev_copy16,
                  lib.synth_dev_grad_f16):
            f.restype = ctypes.c_int
        _dev = lib
    return _dev


# ----------------------------------------------------------------- keys


def key(seed: int, stream: int) -> int:
    return int(host_lib().synth_key(_u64(seed), _u64(stream)))


def hash_at(k: int, i: int) -> int:
    return int(host_lib().synth_hash(_u64(k), _u64(i)))


def grad_stream(j: int, step: int, M: int) -> int:
    """Stream of contribution j at 0-based step `step`."""
    return 1 + j + M * step


class Kinds:
    """Counts per million of exact zeros, bf16 subnormals and outliers."""

    def __init__(self, zero_ppm=0, subnormal_ppm=0, outlier_ppm=0, outlier_factor=1.0):
        self.zero_ppm = int(zero_ppm)
        self.subnormal_ppm = int(subnormal_ppm)
        self.outlier_ppm = int(outlier_ppm)
        self.outlier_factor = float(outlier_factor)

    def args(self, sigma):
        return (scale_for(sigma * self.outlier_factor), self.zero_ppm, self.subnormal_ppm,
                self.outlier_ppm)


NO_KINDS = Kinds()


# ------------------------------------------------------------ host side


def host_normal_f32(n: int, k: int, sigma: float, base: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    host_lib().synth_normal_f32(out.ctypes.data, n, _u64(k), base, scale_for(sigma))
    return out


def host_normal_f32_at(idx: np.ndarray, k: int, sigma: float) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    host_lib().synth_normal_f32_at(out.ctypes.data, idx.ctypes.data, idx.size, _u64(k),
                                   scale_for(sigma))
    return out


def host_grad_bf16(n: int, k: int, ksel: int, sigma: float, kinds: Kinds = NO_KINDS,
                   base: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16)."""
    out = np.empty(n, dtype=np.uint16)
    osc, z, s, o = kinds.args(sigma)
    host_lib().synth_grad_bf16(out.ctypes.data, n, _u64(k), _u64(ksel), base, scale_for(sigma),
                               osc, z, s, o)
    return out


def host_grad_bf16_at(idx: np.ndarray, k: int, ksel: int, sigma: float,
                      kinds: Kinds = NO_KINDS) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    osc, z, s, o = kinds.args(sigma)
    host_lib().synth_grad_bf16_at(out.ctypes.data, idx.ctypes.data, idx.size, _u64(k),
                                  _u64(ksel), scale_for(sigma), osc, z, s, o)
    return out


def host_grad_f16(n: int, k: int, sigma: float, loss_scale: float, base: int = 0) -> np.ndarray:
    """fp16 bit patterns (uint16) of ~N(0, sigma) * loss_scale, narrowed by truncation."""
    out = np.empty(n, dtype=np.uint16)
    host_lib().synth_grad_f16(out.ctypes.data, n, _u64(k), base, scale_for(sigma),
                              np.float32(loss_scale))
    return out


def host_grad_f16_at(idx: np.ndarray, k: int, sigma: float, loss_scale: float) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    host_lib().synth_grad_f16_at(out.ctypes.data, idx.ctypes.data, idx.size, _u64(k),
                                 scale_for(sigma), np.float32(loss_scale))
    return out


# ---------------------------------------------------------- device side


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def dev_normal_f32(t, k: int, sigma: float, base: int = 0, stream=None):
    """Fill fp32 device tensor `t` (contiguous) with ~N(0, sigma) values."""
    import torch
    assert t.dtype == torch.float32 and t.is_contiguous() and t.is_cuda
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(dev_lib().synth_dev_normal_f32(t.data_ptr(), t.numel(), _u64(k), base,
                                          scale_for(sigma), s), "synth_dev_normal_f32")


def dev_grad_bf16(t, k: int, ksel: int, sigma: float, kinds: Kinds = NO_KINDS, base: int = 0,
                  stream=None):
    """Fill a 2-byte device tensor (bf16 or int16 view) with gradient bit patterns."""
    import torch
    assert t.element_size() == 2 and t.is_contiguous() and t.is_cuda
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    osc, z, sb, o = kinds.args(sigma)
    _check(dev_lib().synth_dev_grad_bf16(t.data_ptr(), t.numel(), _u64(k), _u64(ksel), base,
                                         scale_for(sigma), osc, z, sb, o, s),
           "synth_dev_grad_bf16")


def dev_grad_f16(t, k: int, sigma: float, loss_scale: float, base: int = 0, stream=None):
    """Fill a 2-byte device tensor with fp16 patterns of ~N(0, sigma) * loss_scale."""
    import torch
    assert t.element_size() == 2 and t.is_contiguous() and t.is_cuda
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(dev_lib().synth_dev_grad_f16(t.data_ptr(), t.numel(), _u64(k), base, scale_for(sigma),
                                        np.float32(loss_scale), s), "synth_dev_grad_f16")


def dev_zero_ranges(t, ranges, stream=None):
    """Zero the (offset, length) element ranges of device tensor `t`."""
    import torch
    if len(ranges) == 0:
        return
    r = np.asarray(ranges, dtype=np.int64).reshape(-1, 2)
    if (r[:, 0] < 0).any() or (r[:, 1] < 0).any() or (r[:, 0] + r[:, 1] > t.numel()).any():
        raise ValueError("range outside the tensor")
    rd = torch.from_numpy(r.reshape(-1)).to(t.device)
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(dev_lib().synth_dev_zero_ranges(t.data_ptr(), t.element_size(), rd.data_ptr(),
                                           r.shape[0], s), "synth_dev_zero_ranges")
    torch.cuda.current_stream().synchronize()


def dev_gather(t, idx: np.ndarray) -> np.ndarray:
    """Host copy of t[idx] for a 2- or 4-byte device tensor."""
    import torch
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= t.numel()):
        raise ValueError("index outside the tensor")
    out = torch.empty(idx.size, dtype=t.dtype, device=t.device)
    di = torch.from_numpy(idx).to(t.device)
    s = torch.cuda.current_stream().cuda_stream
    _check(dev_lib().synth_dev_gather(out.data_ptr(), t.data_ptr(), t.element_size(),
                                      di.data_ptr(), idx.size, s), "synth_dev_gather")
    torch.cuda.current_stream().synchronize()
    return out.cpu().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy().view(
        np.uint16 if t.element_size() == 2 else np.float32)


def dev_scatter(t, idx: np.ndarray, values: np.ndarray):
    """t[idx] = values for a 2- or 4-byte device tensor (values: uint16 or float32)."""
    import torch
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= t.numel()):
        raise ValueError("index outside the tensor")
    vals = np.ascontiguousarray(values)
    assert vals.itemsize == t.element_size() and vals.size == idx.size
    src = torch.from_numpy(vals.view(np.int16 if vals.itemsize == 2 else np.int32)).to(t.device)
    di = torch.from_numpy(idx).to(t.device)
    s = torch.cuda.current_stream().cuda_stream
    _check(dev_lib().synth_dev_scatter(t.data_ptr(), src.data_ptr(), t.element_size(),
                                       di.data_ptr(), idx.size, s), "synth_dev_scatter")
    torch.cuda.current_stream().synchronize()


def dev_copy(dst, src, stream=None):
    """Plain 16-byte-wide copy of a whole tensor (counter calibration)."""
    import torch
    nbytes = src.numel() * src.element_size()
    assert nbytes % 16 == 0 and dst.numel() * dst.element_size() >= nbytes
    assert dst.data_ptr() % 16 == 0 and src.data_ptr() % 16 == 0
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(dev_lib().synth_dev_copy16(dst.data_ptr(), src.data_ptr(), nbytes // 16, s),
           "synth_dev_copy16")
