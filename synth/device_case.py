"""Fills a rank's device buffers with a workload's seeded synthetic inputs.

Input plumbing for the tests and the benchmark.  Values are addressed by shard
offset (see synth/__init__.py); padding ranges -- given by the caller as
(offset, length) pairs -- are zeroed in every array, as the layout requires.
"""
from __future__ import annotations

import numpy as np

from . import Kinds, dev_grad_bf16, dev_normal_f32, dev_scatter, dev_zero_ranges, \
    host_grad_bf16, host_grad_bf16_at, host_normal_f32, host_normal_f32_at, key
from .workloads import Workload


def padding_mask_at(idx: np.ndarray, padding_ranges) -> np.ndarray:
    """True where a sampled index falls in padding."""
    if not padding_ranges:
        return np.zeros(idx.size, bool)
    r = np.asarray(padding_ranges, dtype=np.int64).reshape(-1, 2)
    starts = r[:, 0]
    ends = r[:, 0] + r[:, 1]
    order = np.argsort(starts)
    starts, ends = starts[order], ends[order]
    k = np.searchsorted(starts, idx, side="right") - 1
    ok = k >= 0
    out = np.zeros(idx.size, bool)
    out[ok] = idx[ok] < ends[k[ok]]
    return out


ALL_SUBNORMAL = Kinds(subnormal_ppm=1_000_000)


class DeviceCase:
    """Device inputs of workload `w` for a shard of `shard_len` elements.

    special: (offset, length, kind) ranges whose gradient contributions are
    overridden in every contribution ("zero": +0.0; "subnormal": bf16
    subnormals from their own hash stream).  grads: M preallocated bf16 device
    tensors of at least shard_len elements to fill (default: allocate them)."""

    def __init__(self, w: Workload, shard_len: int, padding_ranges, device, special=(),
                 grads=None):
        import torch
        self.w = w
        self.S = shard_len
        self.pad = [(int(o), int(n)) for o, n in padding_ranges if n > 0]
        self.zero = [(o, n) for o, n, k in special if k == "zero"]
        sub = [(o, n) for o, n, k in special if k == "subnormal"]
        self.sub_idx = (np.concatenate([np.arange(o, o + n) for o, n in sub]).astype(np.int64)
                        if sub else np.zeros(0, np.int64))
        self.device = device
        if grads is not None:
            if len(grads) != w.M or any(g.numel() < shard_len or g.dtype != torch.bfloat16
                                        for g in grads):
                raise ValueError("grads: expected M bf16 tensors of at least shard_len elements")
            self.grads = list(grads)
        else:
            n = max(shard_len, 8)
            self.grads = [torch.empty(n, dtype=torch.bfloat16, device=device) for _ in range(w.M)]
        self._grads_step = None

    # -------------------------------------------------------- device fills

    def fill_master(self, master):
        dev_normal_f32(master[:self.S], self.w.master_key(), self.w.sigma_master)
        dev_zero_ranges(master, self.pad)

    def fill_grads(self, step0: int):
        """Generate the M contributions of 0-based step `step0` (cached for fixed grads)."""
        s = self.w.grad_step_index(step0)
        if self._grads_step == s:
            return self.grads
        for j, (g, (k, ks)) in enumerate(zip(self.grads, self.w.grad_keys(step0))):
            dev_grad_bf16(g[:self.S], k, ks, self.w.sigma_grad, self.w.kinds)
            dev_zero_ranges(g, self.pad + self.zero)
            if self.sub_idx.size:
                dev_scatter(g, self.sub_idx, self._subnormals(j, step0, self.sub_idx))
        self._grads_step = s
        return self.grads

    def _subnormals(self, j, step0, idx):
        st = 0x30000 + j + self.w.M * self.w.grad_step_index(step0)
        return host_grad_bf16_at(idx, key(self.w.seed, st), key(self.w.seed, st + 0x8000), 1.0,
                                 ALL_SUBNORMAL)

    def _override(self, g, j, step0, idx=None):
        """Apply the special ranges to a host array (whole shard, or sampled at idx)."""
        if idx is None:
            for o, n in self.zero:
                g[o:o + n] = 0
            if self.sub_idx.size:
                g[self.sub_idx] = self._subnormals(j, step0, self.sub_idx)
            return g
        if self.zero:
            g[padding_mask_at(idx, self.zero)] = 0
        if self.sub_idx.size:
            hit = np.isin(idx, self.sub_idx)
            if hit.any():
                g[hit] = self._subnormals(j, step0, idx[hit])
        return g

    # ---------------------------------------------------------- host twins

    def host_master(self, idx=None) -> np.ndarray:
        if idx is None:
            x = host_normal_f32(self.S, self.w.master_key(), self.w.sigma_master)
            for o, n in self.pad:
                x[o:o + n] = 0
            return x
        x = host_normal_f32_at(idx, self.w.master_key(), self.w.sigma_master)
        x[padding_mask_at(idx, self.pad)] = 0
        return x

    def host_grads(self, step0: int, idx=None):
        out = []
        for j, (k, ks) in enumerate(self.w.grad_keys(step0)):
            if idx is None:
                g = host_grad_bf16(self.S, k, ks, self.w.sigma_grad, self.w.kinds)
                for o, n in self.pad:
                    g[o:o + n] = 0
            else:
                g = host_grad_bf16_at(idx, k, ks, self.w.sigma_grad, self.w.kinds)
                g[padding_mask_at(idx, self.pad)] = 0
            out.append(self._override(g, j, step0, idx))
        return out
