"""The five synthetic workloads the shard step is checked and measured on.

Each workload is a parameter-tensor list (element counts in forward order and a
weight-decay flag per tensor), the ZeRO geometry (N shards, this rank), the
number M of gradient contributions reduced per step, the step count, the value
distributions and the AdamW hyper-parameters.  Shapes only: no weights, no
data set.  The model shapes are the GPT-style 1.3B and Llama-style 6.7B / 70B
parameter lists (public architecture shapes); the values are seeded synthetic.

Readings where the workload text is silent (recorded with the design notes):
  * hyper-parameters of workloads 2-5 equal workload 1's;
  * workloads 1-4 decay every tensor; workload 5 decays only its 64 matrices;
  * workload 5 uses M = 4, N = 1, one fixed gradient set reused every step,
    and a global-norm clip at 1.0;
  * "N(0, s)" means standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

from . import Kinds, NO_KINDS, hash_at, key

BUCKET_CAP = 25_000_000
ALIGN = 64


@dataclass
class Workload:
    name: str
    numel: List[int]
    decay: List[int]
    world_size: int
    rank: int
    M: int
    steps: int
    sigma_grad: float
    sigma_master: float = 0.02
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    max_grad_norm: float = 0.0  # <= 0: no clipping
    fixed_grads: bool = False
    kinds: Kinds = field(default_factory=lambda: NO_KINDS)
    bucket_cap: int = BUCKET_CAP
    align: int = ALIGN
    index: int = 0
    description: str = ""
    # tensors whose gradient contributions are overridden in every step and
    # every contribution: "zero" -> exact +0.0, "subnormal" -> bf16 subnormals
    special: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return ((0x5A5E0000 + self.index) << 16) | self.rank

    @property
    def total_params(self) -> int:
        return sum(self.numel)

    def grad_step_index(self, step: int) -> int:
        """0-based step whose gradient streams feed 0-based step `step`."""
        return 0 if self.fixed_grads else step

    def grad_keys(self, step: int):
        """(value key, kind-selector key) of each contribution at 0-based step."""
        s = self.grad_step_index(step)
        out = []
        for j in range(self.M):
            stream = 1 + j + self.M * s
            out.append((key(self.seed, stream), key(self.seed, 0x10000 + stream)))
        return out

    def master_key(self) -> int:
        return key(self.seed, 0)


def _gpt_13b():
    h, ffn, layers, vocab = 2048, 8192, 24, 50304
    numel = [vocab * h]
    for _ in range(layers):
        numel += [h, h, h * 3 * h, h * h, h, h, h * ffn, ffn * h]
    numel += [h, h]
    return numel


def _llama(h, ffn, layers, vocab, kv_dim):
    numel = [vocab * h]
    for _ in range(layers):
        numel += [h, h * h, h * kv_dim, h * kv_dim, h * h, h, h * ffn, h * ffn, ffn * h]
    numel += [h, h * vocab]
    return numel


def _stress_tensors(seed: int):
    """10,000 sizes uniform on 1..4096 plus 64 matrices of 4096x4096, shuffled."""
    ks = key(seed, 0x20000)
    small = [1 + hash_at(ks, i) % 4096 for i in range(10_000)]
    sizes = [(n, 0) for n in small] + [(4096 * 4096, 1)] * 64
    kp = key(seed, 0x20001)
    for i in range(len(sizes) - 1, 0, -1):  # Fisher-Yates with the counter hash
        j = hash_at(kp, i) % (i + 1)
        sizes[i], sizes[j] = sizes[j], sizes[i]
    return [n for n, _ in sizes], [d for _, d in sizes]


def workload(index: int, rank: Optional[int] = None) -> Workload:
    """Workload 1..5 (1-based, in the order they are listed)."""
    if index == 1:
        w = Workload("tiny-flat-1M", [1 << 20], [1], 1, 0, M=4, steps=10, sigma_grad=1e-3,
                     description="one flat tensor of 1,048,576 params, N=1, M=4")
    elif index == 2:
        n = _gpt_13b()
        w = Workload("gpt1.3b-zero1-shard1of8", n, [1] * len(n), 8, 0, M=8, steps=20,
                     sigma_grad=1e-3,
                     description="GPT-style 1.3B (h=2048, 24 layers, vocab 50304) in 25M-param "
                                 "buckets, 1/8 shard (rank 0), M=8")
    elif index == 3:
        n = _llama(4096, 11008, 32, 32000, 4096)
        w = Workload("llama6.7b-unsharded", n, [1] * len(n), 1, 0, M=1, steps=5,
                     sigma_grad=5e-4,
                     description="Llama-style 6.7B (h=4096, ffn 11008, 32 layers, vocab 32000), "
                                 "N=1, M=1")
    elif index == 4:
        n = _llama(8192, 28672, 80, 32000, 1024)
        w = Workload("llama70b-zero-shard1of16", n, [1] * len(n), 16, 0, M=8, steps=3,
                     sigma_grad=5e-4,
                     description="Llama-style 70B (h=8192, ffn 28672, 80 layers, GQA kv 1024, "
                                 "vocab 32000), 1/16 shard (rank 0), M=8")
    elif index == 5:
        seed = ((0x5A5E0000 + 5) << 16)
        n, d = _stress_tensors(seed)
        w = Workload("stress-10k-mixed-clip", n, d, 1, 0, M=4, steps=1000, sigma_grad=1e-3,
                     max_grad_norm=1.0, fixed_grads=True,
                     kinds=Kinds(zero_ppm=50_000, subnormal_ppm=1_000, outlier_ppm=10_000,
                                 outlier_factor=1e3),
                     description="10,000 tensors of 1..4096 + 64 x 4096x4096, shuffled; decay on "
                                 "matrices only; 1% x1e3 outliers, 5% zeros, 0.1% subnormals; "
                                 "fixed grads, global-norm clip 1.0, 1000 steps")
        small = [t for t, d in enumerate(d) if d == 0]
        w.special = {"zero": small[:16], "subnormal": small[16:32]}
    else:
        raise ValueError(f"no workload {index}")
    w.index = index
    if rank is not None:
        if not 0 <= rank < w.world_size:
            raise ValueError("rank out of range")
        w.rank = rank
    return w


def special_ranges(w: Workload, segments):
    """(shard offset, length, kind) of the overridden tensors' pieces in a shard.

    segments: iterable of (shard_off, length, tensor) in shard order."""
    kind_of = {}
    for kind, ts in w.special.items():
        for t in ts:
            kind_of[t] = kind
    out = []
    for off, ln, t in segments:
        if t in kind_of and ln > 0:
            out.append((int(off), int(ln), kind_of[t]))
    return out


def scaled(w: Workload, numel: List[int], decay: Optional[List[int]] = None,
           world_size: Optional[int] = None, rank: int = 0, M: Optional[int] = None,
           name: Optional[str] = None) -> Workload:
    """A small variant of workload w with another tensor list (parity-size cases)."""
    import copy
    v = copy.copy(w)
    v.numel = list(numel)
    v.decay = list(decay) if decay is not None else [1] * len(numel)
    if world_size is not None:
        v.world_size = world_size
    v.rank = rank
    if M is not None:
        v.M = M
    v.name = name or (w.name + "-small")
    return v
