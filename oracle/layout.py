"""Oracle for the flat bucket / shard layout (integer work).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The layout, written out plainly:

1. Tensors are flattened in forward order into buckets.  Inside a bucket each
   tensor starts at the next multiple of `align` elements.  A bucket is closed
   when the next tensor would end beyond `bucket_cap` elements; a tensor larger
   than the cap sits alone in its bucket.  Only a bucket that holds elements is
   closed, and only by a tensor that has elements (reading: a bucket holds
   elements; otherwise leading empty tensors, or an empty tensor after an
   oversize one, would leave a bucket with nothing in it).  (Gradient buckets: 大模型基础设施工程
   06, §6.1 on DDP buckets and §11.3 on reduce_bucket_size /
   contiguous_gradients; flattening into one contiguous buffer before cutting:
   Lecture04 notes, ZeRO-3 / FSDP section on the flattened parameter.)
2. Each bucket is padded to a multiple of world_size * align elements, so it
   cuts into world_size equal, aligned slices ("padded to shard boundary").
3. Rank r owns slice r of every bucket: after the reduce-scatter it holds the
   reduced gradient of exactly that slice and updates only it (Lecture04
   notes, "ZeRO-1"; CS324 notes §3.4; CS336 第七讲 summary, Q2).  Its flat
   shard is the concatenation of its slices in bucket order.  Cutting flat
   buffers without regard to tensor boundaries is legal because AdamW is
   elementwise (CS324 notes §3.4).
4. Segments are the maximal runs of one tensor (or of padding) inside the
   shard; each carries the tensor's weight-decay flag (padding: 0).

Memory accounting per rank (16 bytes per parameter: bf16 param 2 + bf16 grad 2
+ fp32 master, m, v 12 -- CS324 notes §2.1; CS336 第七讲 summary, Q3; the
per-stage formulas of Lecture04 notes, ZeRO-1 and ZeRO-2 sections):
   stage 0 (plain DP)  16*Psi
   stage 1             4*Psi + 12*S
   stage 2             2*Psi + 14*S
   stage 3             16*S
with Psi the model's parameter count and S this rank's (padded) shard length.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np


def _align_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


@dataclass
class Segment:
    shard_off: int
    length: int
    tensor: int       # -1 for padding
    tensor_off: int   # element offset inside the tensor (0 for padding)
    decay: int


@dataclass
class Layout:
    world_size: int
    rank: int
    align: int
    bucket_cap: int
    tensor_flat_off: List[int]
    tensor_bucket: List[int]
    buckets: List[Tuple[int, int]]   # (flat start, padded length)
    shard_len: int
    padded_total: int
    segments: List[Segment]
    total_params: int
    numel: List[int] = None

    def decay_mask(self) -> np.ndarray:
        mask = np.zeros(self.shard_len, dtype=np.uint8)
        for s in self.segments:
            if s.decay:
                mask[s.shard_off:s.shard_off + s.length] = 1
        return mask

    def padding_ranges(self) -> List[Tuple[int, int]]:
        return [(s.shard_off, s.length) for s in self.segments if s.tensor < 0]

    def canonical_offsets(self) -> List[int]:
        """Offset of each tensor in the canonical order: tensors concatenated in
        forward order without padding (the layout-independent checkpoint format)."""
        out, acc = [], 0
        for n in self.numel:
            out.append(acc)
            acc += n
        return out

    def to_canonical(self, shard: np.ndarray, canon: np.ndarray) -> None:
        """Write this rank's tensor elements of a shard array into a canonical array."""
        co = self.canonical_offsets()
        for s in self.segments:
            if s.tensor >= 0:
                c = co[s.tensor] + s.tensor_off
                canon[c:c + s.length] = shard[s.shard_off:s.shard_off + s.length]

    def from_canonical(self, canon: np.ndarray, shard: np.ndarray) -> None:
        """The reverse of to_canonical; padding is left as it is."""
        co = self.canonical_offsets()
        for s in self.segments:
            if s.tensor >= 0:
                c = co[s.tensor] + s.tensor_off
                shard[s.shard_off:s.shard_off + s.length] = canon[c:c + s.length]

    def tensor_slice(self, t: int) -> Tuple[int, int, int]:
        """(shard offset, offset inside tensor, length) of tensor t on this rank."""
        for s in self.segments:
            if s.tensor == t:
                return s.shard_off, s.tensor_off, s.length
        return 0, 0, 0

    def state_bytes(self, stage: int) -> int:
        psi, S = self.total_params, self.shard_len
        if stage == 0:
            return 16 * psi
        if stage == 1:
            return 4 * psi + 12 * S
        if stage == 2:
            return 2 * psi + 14 * S
        if stage == 3:
            return 16 * S
        raise ValueError("stage must be 0..3")


def plan(numel, decay, world_size: int, rank: int, bucket_cap: int = 25_000_000,
         align: int = 64) -> Layout:
    numel = [int(n) for n in numel]
    decay = [1 if d else 0 for d in decay]
    if len(decay) != len(numel):
        raise ValueError("numel and decay differ in length")
    if world_size < 1 or not 0 <= rank < world_size or align < 1 or bucket_cap < 1:
        raise ValueError("bad geometry")
    if any(n < 0 for n in numel):
        raise ValueError("negative tensor size")

    # 1. buckets
    buckets: List[Tuple[int, int]] = []
    members: List[List[int]] = []
    flat_off = [0] * len(numel)
    which = [0] * len(numel)
    start, fill, cur = 0, 0, []
    for t, n in enumerate(numel):
        pos = _align_up(fill, align)
        if cur and fill > 0 and n > 0 and pos + n > bucket_cap:
            length = _align_up(fill, world_size * align)
            buckets.append((start, length))
            members.append(cur)
            start, fill, cur, pos = start + length, 0, [], 0
        flat_off[t] = start + pos
        which[t] = len(buckets)
        fill = pos + n
        cur.append(t)
    if cur:
        # 2. the last bucket is padded like the others
        length = _align_up(fill, world_size * align)
        buckets.append((start, length))
        members.append(cur)

    # 3./4. this rank's slice of every bucket, cut into segments
    segments: List[Segment] = []
    shard_off = 0
    for (b_start, b_len), ts in zip(buckets, members):
        part = b_len // world_size
        lo = b_start + rank * part
        hi = lo + part
        cursor = lo
        for t in ts:
            t_lo, t_hi = flat_off[t], flat_off[t] + numel[t]
            a, b = max(t_lo, lo), min(t_hi, hi)
            if a >= b:
                continue
            if a > cursor:
                segments.append(Segment(shard_off + cursor - lo, a - cursor, -1, 0, 0))
            segments.append(Segment(shard_off + a - lo, b - a, t, a - t_lo, decay[t]))
            cursor = b
        if hi > cursor:
            segments.append(Segment(shard_off + cursor - lo, hi - cursor, -1, 0, 0))
        shard_off += part

    # merge neighbouring padding segments (a bucket boundary can split them)
    merged: List[Segment] = []
    for s in segments:
        if merged and s.tensor < 0 and merged[-1].tensor < 0:
            merged[-1].length += s.length
        else:
            merged.append(s)

    padded_total = buckets[-1][0] + buckets[-1][1] if buckets else 0
    return Layout(world_size, rank, align, bucket_cap, flat_off, which, buckets, shard_off,
                  padded_total, merged, sum(numel), list(numel))
