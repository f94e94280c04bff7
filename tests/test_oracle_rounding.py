"""Brute-force pins of the oracle's fp32 rounding model on tiny inputs.

Every intermediate value is carried as an exact rational and rounded to fp32
(nearest, ties to even) after each operation (tests/_exact.py).  The oracle's
fp32 step must reproduce those bits exactly: this fails if an operation is
contracted into an FMA, evaluated in higher precision, reordered, or if
division/sqrt are not correctly rounded -- the properties the GPU kernel is
then held to bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import _exact as E


def _bf16_values(rng, n, scale):
    x = (rng.normal(0, scale, n)).astype(np.float32)
    return oracle.f32_to_bf16(x)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 16])
def test_reduce_is_sequential_single_rounded(M):
    rng = np.random.default_rng(100 + M)
    n = 300
    gs = [_bf16_values(rng, n, 10.0 ** rng.integers(-6, 3)) for _ in range(M)]
    # include subnormal and mixed-magnitude contributions
    gs[0][:5] = [0x0001, 0x8001, 0x007F, 0x0080, 0x3F80]
    if M > 1:
        gs[1][:5] = [0x0001, 0x0001, 0x8080, 0x0080, 0xBF80]
    got = oracle.reduce_mean_f32(gs)
    for i in range(n):
        s = oracle.bf16_to_f32(np.array([gs[0][i]], np.uint16))[0]
        for j in range(1, M):
            s = E.add(s, oracle.bf16_to_f32(np.array([gs[j][i]], np.uint16))[0])
        want = E.div(s, np.float32(M))
        assert got[i].view(np.uint32) == want.view(np.uint32), (i, got[i], want)


def _step_exact(g, p, m, v, k, decay):
    """One element, the definition with an exact rounding after every operation."""
    mN = E.mul(k["beta1"], m)
    mG = E.mul(k["c1"], g)
    m1 = E.add(mN, mG)
    gg = E.mul(g, g)
    vN = E.mul(k["beta2"], v)
    vG = E.mul(k["c2"], gg)
    v1 = E.add(vN, vG)
    r = E.sqrt(v1)
    q = E.div(r, k["bhat"])
    den = E.add(q, k["eps"])
    p1 = E.mul(p, k["decay_mul"] if decay else np.float32(1.0))
    u = E.div(m1, den)
    w = E.mul(k["alpha"], u)
    return E.sub(p1, w), m1, v1


def _scalars_exact(lr, b1, b2, eps, wd, t):
    """fp64 evaluation of the step constants, rounded once to fp32."""
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    bc1 = 1.0 - b1 ** t
    bc2 = 1.0 - b2 ** t
    return dict(beta1=np.float32(b1), beta2=np.float32(b2), c1=np.float32(1.0 - b1),
                c2=np.float32(1.0 - b2), alpha=np.float32(lr / bc1),
                bhat=np.float32(bc2 ** 0.5), eps=np.float32(eps),
                decay_mul=np.float32(1.0 - lr * wd))


@pytest.mark.parametrize("t", [1, 2, 7, 1000])
def test_step_is_single_rounded_per_operation(t):
    rng = np.random.default_rng(200 + t)
    n, M = 200, 3
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    k = oracle.step_scalars_f32(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                hp["weight_decay"], t)
    kx = _scalars_exact(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], t)
    for name in kx:  # host constants agree with an independent fp64 evaluation
        assert np.float32(k[name]) == kx[name], name
    gs = [_bf16_values(rng, n, 1e-3) for _ in range(M)]
    p = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-4, n).astype(np.float32)
    v = np.abs(rng.normal(0, 1e-7, n)).astype(np.float32)
    p[:3] = 0.0
    m[3:6] = 0.0
    v[3:6] = 0.0
    decay = (np.arange(n) % 3 != 0).astype(np.uint8)
    pb = np.zeros(n, np.uint16)
    p0, m0, v0 = p.copy(), m.copy(), v.copy()
    oracle.step_f32(gs, p, m, v, pb, decay, step=t, **hp)
    g = oracle.reduce_mean_f32(gs)
    for i in range(n):
        wp, wm, wv = _step_exact(g[i], p0[i], m0[i], v0[i], kx, decay[i])
        assert p[i].view(np.uint32) == wp.view(np.uint32), (i, p[i], wp)
        assert m[i].view(np.uint32) == wm.view(np.uint32), (i, m[i], wm)
        assert v[i].view(np.uint32) == wv.view(np.uint32), (i, v[i], wv)
        # the bf16 param is the round-to-nearest-even of the new master
        u = int(wp.view(np.uint32))
        lo, rem = u >> 16, u & 0xFFFF
        if rem > 0x8000 or (rem == 0x8000 and lo & 1):
            lo += 1
        assert int(pb[i]) == lo, i


def test_exact_helpers_against_known_values():
    # the brute-force helpers themselves: RNE ties and a known sqrt
    assert E.rne_f32(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)
    assert E.rne_f32(Fraction(1) + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2.0 ** -22)
    assert E.sqrt(np.float32(4.0)) == np.float32(2.0)
    assert E.sqrt(np.float32(2.0)).view(np.uint32) == np.uint32(0x3FB504F3)
    assert E.rne_f32(Fraction(1, 2 ** 150)) == np.float32(0.0)      # tie to even (zero)
    assert E.rne_f32(Fraction(3, 2 ** 150)).view(np.uint32) == np.uint32(2)  # 1.5 ulp -> 2


def test_pow_int_against_exact_rationals():
    """beta^t by fp64 binary powering stays within 1e-13 of the exact power, so the
    fp32 step constants equal the exactly rounded constants of the exact values."""
    for beta in (0.9, 0.95, 0.99, 0.999):
        b32 = float(np.float32(beta))
        exact = Fraction(1)
        for t in range(1, 1201):
            exact *= Fraction(b32)
            if t % 7 and t > 40:
                continue
            p = oracle.pow_int(b32, t)
            assert abs(Fraction(p) - exact) <= Fraction(1, 10 ** 13) * exact, (beta, t)


@pytest.mark.parametrize("t", [1, 2, 3, 10, 100, 1000])
def test_step_constants_exactly_rounded(t):
    lr, b1, b2 = np.float32(3e-4), np.float32(0.9), np.float32(0.95)
    k = oracle.step_scalars_f32(float(lr), float(b1), float(b2), 1e-8, 0.1, t)
    bc1 = 1 - Fraction(float(b1)) ** t
    bc2 = 1 - Fraction(float(b2)) ** t
    assert np.float32(k["alpha"]) == E.rne_f32(Fraction(float(lr)) / bc1)
    assert np.float32(k["bhat"]) == E.sqrt_rne_f32(bc2)
    assert np.float32(k["c1"]) == E.rne_f32(1 - Fraction(float(b1)))
    assert np.float32(k["decay_mul"]) == E.rne_f32(1 - Fraction(float(lr)) * Fraction(float(np.float32(0.1))))
