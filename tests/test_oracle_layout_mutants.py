"""The layout oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/layout.py (a wrong padding
multiple, a missing alignment, an off-by-one at the cap, reversed rank slices,
an offset taken from the wrong origin, a wrong memory formula, a dropped rule),
loads the copy as a module of its own, and runs the layout pins of
test_oracle_layout and test_oracle_shard with that copy in place of the
oracle's: at least one must fail.  The unmodified source, loaded the same way,
must pass all of them.
"""
import os
import sys
import types

import pytest

import test_oracle_layout as LA
import test_oracle_shard as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "layout.py")

# the pin checks, cheapest first
PINS = [
    lambda: LA.test_bucket_closes_only_beyond_the_cap(),
    lambda: LA.test_memory_accounting_worked_examples(),
    *[(lambda n=n: LA.test_empty_tensors_structure(n))
      for n in ([5000, 0, 7000], [0, 0, 5000, 0, 0, 7000, 0], [300, 5000, 0, 0, 6000], [0, 5000])],
    *[(lambda s=s: LA.test_layout_structure_random(s)) for s in range(12)],
    *[(lambda n=n: LA.test_canonical_mapping_partitions_the_model(n)) for n in (1, 3, 8)],
    lambda: LA.test_gpt_buckets(),
    lambda: LA.test_model_shard_sizes(2, 1_311_182_848),
    lambda: Z.test_padding_is_inert(1),
    lambda: Z.test_sharded_equals_unsharded(3, 0, 0.05),
    lambda: Z.test_zero_equals_dp_worked_example(),
]

MUTANTS = [
    ("bucket-padded-to-align-only",
     "length = _align_up(fill, world_size * align)", "length = _align_up(fill, align)"),
    ("last-bucket-unpadded",
     "# 2. the last bucket is padded like the others\n        length = _align_up(fill, world_size * align)",
     "# 2. the last bucket is padded like the others\n        length = fill"),
    ("no-tensor-alignment", "pos = _align_up(fill, align)", "pos = fill"),
    ("closes-at-the-cap", "pos + n > bucket_cap", "pos + n >= bucket_cap"),
    ("empty-tensor-closes", "if cur and fill > 0 and n > 0 and pos + n > bucket_cap:",
     "if cur and pos + n > bucket_cap:"),
    ("empty-bucket-closes", "if cur and fill > 0 and n > 0 and", "if cur and n > 0 and"),
    ("empty-tensor-opens", "if cur and fill > 0 and n > 0 and", "if cur and fill > 0 and"),
    ("rank-slices-reversed", "lo = b_start + rank * part",
     "lo = b_start + (world_size - 1 - rank) * part"),
    ("tensor-off-from-slice", "b - a, t, a - t_lo, decay[t]", "b - a, t, a - lo, decay[t]"),
    ("decay-of-next-tensor", "b - a, t, a - t_lo, decay[t]",
     "b - a, t, a - t_lo, decay[min(t + 1, len(decay) - 1)]"),
    ("padding-decays", "segments.append(Segment(shard_off + cursor - lo, hi - cursor, -1, 0, 0))",
     "segments.append(Segment(shard_off + cursor - lo, hi - cursor, -1, 0, 1))"),
    ("padding-not-merged", "if merged and s.tensor < 0 and merged[-1].tensor < 0:",
     "if False:"),
    ("canonical-keeps-alignment", "            out.append(acc)\n            acc += n",
     "            out.append(acc)\n            acc += _align_up(n, 64)"),
    ("stage2-omits-grad-shard", "return 2 * psi + 14 * S", "return 2 * psi + 12 * S"),
    ("stage1-keeps-full-grads", "return 4 * psi + 12 * S", "return 2 * psi + 12 * S"),
]


def _load(src, name):
    mod = types.ModuleType(name)
    mod.__file__ = SOURCE
    sys.modules[name] = mod  # dataclasses look the defining module up by name
    try:
        exec(compile(src, SOURCE, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


@pytest.fixture
def swap_layout(monkeypatch):
    def swap(mod):
        monkeypatch.setattr(LA, "L", mod)
        monkeypatch.setattr(Z, "L", mod)
    return swap


def _failures():
    bad = []
    for i, pin in enumerate(PINS):
        try:
            pin()
        except Exception as e:  # an assertion, or an error the mistake provokes
            bad.append((i, type(e).__name__))
    return bad


def test_unmodified_copy_passes_every_pin(swap_layout):
    with open(SOURCE) as f:
        swap_layout(_load(f.read(), "_layout_copy"))
    assert _failures() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(swap_layout, name, old, new):
    with open(SOURCE) as f:
        src = f.read()
    assert old in src, name
    swap_layout(_load(src.replace(old, new), "_layout_" + name.replace("-", "_")))
    assert _failures(), f"no pin caught {name}"
