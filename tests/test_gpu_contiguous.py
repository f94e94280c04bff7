"""Slabs in physically contiguous device memory (zs_device_alloc_contiguous behind a
torch memory pool): the helpers themselves, the step on such a slab against the
oracle bit for bit, and the memory returned when the shard is closed."""
import pytest
import torch

import sharded_optimizer_step_zero_amd as zsm
from sharded_optimizer_step_zero_amd import ZeroShard
from synth.workloads import scaled, workload

from _gpu import full_parity, log

pytestmark = pytest.mark.gpu


def test_alloc_helpers_roundtrip():
    log("test_alloc_helpers_roundtrip")
    dev = torch.cuda.current_device()
    p = zsm.zs_device_alloc_contiguous(64 << 20, dev)
    assert p and p % 256 == 0
    zsm.zs_device_free(p, 64 << 20, dev)
    zsm.zs_device_free(0)  # NULL is ignored


@pytest.mark.parametrize("flags", [0, zsm.ZS_STAGE_AVERAGE])
def test_step_on_contiguous_slab_matches_oracle(flags):
    log(f"test_step_on_contiguous_slab_matches_oracle flags={flags}")
    w = scaled(workload(1), [5000] * 7 + [1], None, world_size=8, rank=7, M=8, name="contig")
    w.max_grad_norm = 0.05
    full_parity(w, 3, flags=flags, contiguous=True)


def test_contiguous_slab_is_returned_on_close():
    log("test_contiguous_slab_is_returned_on_close")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    before = torch.cuda.memory_reserved()
    numel = [1 << 28]  # 268M elements: a 4.3 GB slab with M = 2
    for _ in range(2):
        z = ZeroShard(numel, [1], 1, 0, 2, grad_buffers=True, contiguous=True)
        assert z.contiguous
        assert torch.cuda.memory_reserved() - before >= z.shard_len * 18
        z.step(z.grads, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
        z.close()
        torch.cuda.synchronize()
        assert torch.cuda.memory_reserved() - before < (64 << 20)
