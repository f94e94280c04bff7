"""Pins of the oracle's M-way reduce (the accumulation / reduce-scatter half).

* mean of M micro-batch gradients = one large-batch gradient (least squares,
  fp64 and exactly representable bf16 cases);
* the ring all-reduce worked example printed in the CS324 notes §3.2.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import _exact as E

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lsq_grad(X, w, y):
    """Gradient of the mean squared loss 0.5*mean((Xw - y)^2) w.r.t. w."""
    return X.T @ (X @ w - y) / X.shape[0]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_accumulated_mean_equals_big_batch_gradient_f64(M):
    """(1/M) sum_j grad of micro-batch j = grad of the whole batch, for equal
    micro-batches (the accumulation identity)."""
    rng = np.random.default_rng(10 + M)
    b, d = 16, 257
    X = rng.normal(size=(M * b, d))
    y = rng.normal(size=M * b)
    w = rng.normal(size=d)
    micro = [_lsq_grad(X[j * b:(j + 1) * b], w, y[j * b:(j + 1) * b]) for j in range(M)]
    big = _lsq_grad(X, w, y)
    # the oracle's fp64 build averages the contributions inside the step; with
    # zero moments at t=1 and wd=0 its m' = (1-beta1)*g exposes g
    hp = dict(lr=1e-3, beta1=0.5, beta2=0.5, eps=1e-8, weight_decay=0.0)
    outs = []
    for grads in (micro, [big]):
        p, m, v = np.zeros(d), np.zeros(d), np.zeros(d)
        oracle.step_f64(grads, p, m, v, None, step=1, **hp)
        outs.append(m / 0.5)
    np.testing.assert_allclose(outs[0], big, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
def test_accumulated_mean_equals_big_batch_gradient_bf16_exact(M):
    """Small-integer data: every micro-batch gradient is exact in bf16 and every
    partial sum exact in fp32, so the fp32 mean is the correctly rounded
    large-batch gradient (exactly equal when M is a power of two)."""
    rng = np.random.default_rng(20 + M)
    b, d = 2, 64
    X = rng.integers(-3, 4, size=(M * b, d)).astype(np.int64)
    y = rng.integers(-3, 4, size=M * b).astype(np.int64)
    w = rng.integers(-2, 3, size=d).astype(np.int64)
    micro = [X[j * b:(j + 1) * b].T @ (X[j * b:(j + 1) * b] @ w - y[j * b:(j + 1) * b])
             for j in range(M)]                       # = b * gradient, integers
    big_num = X.T @ (X @ w - y)                       # = M*b * big-batch gradient
    grads = [oracle.f32_to_bf16((mj / b).astype(np.float32)) for mj in micro]
    for mj, gj in zip(micro, grads):                  # the contributions are exact
        assert np.array_equal(oracle.bf16_to_f32(gj), (mj / b).astype(np.float32))
    got = oracle.reduce_mean_f32(grads)
    for i in range(d):
        want = E.rne_f32(Fraction(int(big_num[i]), M * b))
        assert got[i] == want, (i, got[i], want)


def test_ring_allreduce_worked_example():
    """4 cards, card r holds (r+1)*[0..7]; the reduced vector is 10*[0..7]."""
    spec = {}
    with open(os.path.join(GOLDEN, "ring_allreduce_demo.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *vals = line.split()
            spec[k] = vals
    cards, length = int(spec["cards"][0]), int(spec["length"][0])
    want_sum = np.array([float(x) for x in spec["sum"]], dtype=np.float32)
    base = np.arange(length, dtype=np.float32)
    contribs = [oracle.f32_to_bf16((r + 1) * base) for r in range(cards)]
    mean = oracle.reduce_mean_f32(contribs)
    assert np.array_equal(mean * np.float32(cards), want_sum)
    assert np.array_equal(mean, want_sum / np.float32(cards))
    # the ring's step count and traffic per card: 2(p-1) steps of one
    # length/p block each, i.e. 2(p-1)/p * length numbers
    assert 2 * (cards - 1) == int(spec["steps"][0])
    assert 2 * (cards - 1) * (length // cards) == int(spec["sent_numbers_per_card"][0])
