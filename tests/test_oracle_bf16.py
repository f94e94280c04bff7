"""Pins of the oracle's bf16 conversions against torch's (library routines).

bf16 -> fp32 is exact (the pattern is the upper half of an fp32 pattern);
fp32 -> bf16 is round to nearest, ties to even.  Both are checked
exhaustively: all 65,536 bf16 patterns, and all 2^32 fp32 patterns in chunks.
"""
import numpy as np
import torch

import oracle


def test_bf16_to_f32_exhaustive():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(pats).view(np.uint32)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    nan = np.isnan(ours.view(np.float32))
    assert np.array_equal(nan, np.isnan(ref.view(np.float32)))
    assert np.array_equal(ours[~nan], ref[~nan])
    # widening is a 16-bit shift, NaN payloads included
    assert np.array_equal(ours, pats.astype(np.uint32) << 16)


def test_f32_to_bf16_exhaustive():
    chunk = 1 << 24
    base = np.arange(chunk, dtype=np.uint32)
    u = np.empty(chunk, dtype=np.uint32)
    ref_t = torch.empty(chunk, dtype=torch.bfloat16)
    for start in range(0, 1 << 32, chunk):
        np.add(base, np.uint32(start), out=u)
        x = u.view(np.float32)
        ours = oracle.f32_to_bf16(x)
        ref_t.copy_(torch.from_numpy(x))
        ref = ref_t.view(torch.int16).numpy().view(np.uint16)
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        if not nan.any():
            assert np.array_equal(ours, ref), hex(start)
            continue
        assert np.array_equal(ours[~nan], ref[~nan]), hex(start)
        # NaN stays NaN: exponent all ones, mantissa nonzero, sign kept
        on = ours[nan]
        assert np.all((on & 0x7F80) == 0x7F80) and np.all((on & 0x007F) != 0)
        assert np.array_equal(on >> 15, (u[nan] >> 31).astype(np.uint16))


def test_f32_to_bf16_special_cases():
    def b(x):
        return int(oracle.f32_to_bf16(np.array([x], dtype=np.float32))[0])

    def f(bits):
        return np.array([bits], dtype=np.uint32).view(np.float32)[0]

    assert b(1.0) == 0x3F80
    # halfway between 1.0 (0x3F80) and the next bf16 (0x3F81): ties to even -> 0x3F80
    assert b(f(0x3F808000)) == 0x3F80
    # halfway between 0x3F81 and 0x3F82: ties to even -> 0x3F82
    assert b(f(0x3F818000)) == 0x3F82
    # just above half rounds up
    assert b(f(0x3F808001)) == 0x3F81
    assert b(np.inf) == 0x7F80 and b(-np.inf) == 0xFF80
    # the largest finite fp32 overflows to +inf (no saturation)
    assert b(f(0x7F7FFFFF)) == 0x7F80
    # fp32 subnormals round into bf16 subnormals, the smallest one up from a tie
    assert b(f(0x00008000)) == 0x0000 and b(f(0x00018000)) == 0x0002
    assert b(-0.0) == 0x8000
