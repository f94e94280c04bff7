"""Pins of the oracle's AdamW update.

* the fp64 build against torch.optim.AdamW in fp64 (library routine), several
  steps, per-group weight decay, M contributions averaged;
* the fp32 build against torch.optim.AdamW in fp32 (torch uses lerp/addcmul,
  so agreement is to a few ulps, not bits);
* closed forms: the first step from zero moments, pure decay at zero gradient,
  and the constant-gradient trajectory over 1000 steps;
* invariants: scale invariance at eps = 0, wd = 0 reduces to torch Adam.
"""
import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _torch_adamw(p0, grads_per_step, decay, dtype, steps, adam=False, **hp):
    """Run torch AdamW (single-tensor path) on two param groups split by decay."""
    idx_d = np.nonzero(decay)[0]
    idx_n = np.nonzero(decay == 0)[0]
    pd = torch.nn.Parameter(torch.tensor(p0[idx_d], dtype=dtype))
    pn = torch.nn.Parameter(torch.tensor(p0[idx_n], dtype=dtype))
    groups = [{"params": [pd], "weight_decay": hp["weight_decay"]},
              {"params": [pn], "weight_decay": 0.0}]
    cls = torch.optim.Adam if adam else torch.optim.AdamW
    opt = cls(groups, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
              foreach=False, fused=False)
    for s in range(steps):
        g = grads_per_step[s]
        pd.grad = torch.tensor(g[idx_d], dtype=dtype)
        pn.grad = torch.tensor(g[idx_n], dtype=dtype)
        opt.step()
    out_p = np.empty_like(p0)
    out_p[idx_d] = pd.detach().numpy()
    out_p[idx_n] = pn.detach().numpy()
    st_d, st_n = opt.state[pd], opt.state[pn]
    m = np.empty_like(p0)
    v = np.empty_like(p0)
    m[idx_d], m[idx_n] = st_d["exp_avg"].numpy(), st_n["exp_avg"].numpy()
    v[idx_d], v[idx_n] = st_d["exp_avg_sq"].numpy(), st_n["exp_avg_sq"].numpy()
    return out_p, m, v


def test_f64_matches_torch_adamw_f64():
    rng = np.random.default_rng(1)
    n, M, steps = 4096, 3, 7
    p0 = rng.normal(0, 0.02, n)
    decay = (rng.random(n) < 0.7).astype(np.uint8)
    contribs = [[rng.normal(0, 1e-3, n) for _ in range(M)] for _ in range(steps)]
    means = [(c[0] + c[1] + c[2]) / 3.0 for c in contribs]

    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for s in range(steps):
        oracle.step_f64(contribs[s], p, m, v, decay, step=s + 1, **HP)
    tp, tm, tv = _torch_adamw(p0, means, decay, torch.float64, steps, **HP)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(p, tp, rtol=1e-12, atol=1e-15)


def test_f64_wd0_matches_torch_adam():
    rng = np.random.default_rng(2)
    n, steps = 1000, 5
    p0 = rng.normal(0, 1, n)
    gs = [rng.normal(0, 1, n) for _ in range(steps)]
    hp = dict(HP, weight_decay=0.0)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for s in range(steps):
        oracle.step_f64([gs[s]], p, m, v, None, step=s + 1, **hp)
    tp, _, _ = _torch_adamw(p0, gs, np.ones(n, np.uint8), torch.float64, steps, adam=True, **hp)
    np.testing.assert_allclose(p, tp, rtol=1e-12, atol=1e-15)


def test_f32_matches_torch_adamw_f32():
    rng = np.random.default_rng(3)
    n, M, steps = 8192, 4, 6
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    decay = (rng.random(n) < 0.5).astype(np.uint8)
    # bf16 contributions, and their exact fp32 average as torch's grad
    contribs, means = [], []
    for _ in range(steps):
        cs = [oracle.f32_to_bf16(rng.normal(0, 1e-3, n).astype(np.float32)) for _ in range(M)]
        contribs.append(cs)
        means.append(oracle.reduce_mean_f32(cs))
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for s in range(steps):
        oracle.step_f32(contribs[s], p, m, v, None, decay, step=s + 1, **HP)
    tp, tm, tv = _torch_adamw(p0, means, decay, torch.float32, steps, **HP)
    # torch rounds the moment updates differently (lerp, addcmul), so where
    # beta1*m and (1-beta1)*g cancel, the elementwise relative gap can be large;
    # the bound is a few fp32 ulps of the array's scale.
    np.testing.assert_allclose(m, tm, rtol=2e-6, atol=1e-6 * np.abs(tm).max())
    np.testing.assert_allclose(v, tv, rtol=2e-6, atol=1e-6 * np.abs(tv).max())
    np.testing.assert_allclose(p, tp, rtol=1e-6, atol=1e-9)


def test_first_step_closed_form():
    """From m = v = 0 at t = 1 the bias-corrected moments are g and g^2, so
    p' = p*(1 - lr*wd) - lr*g/(|g| + eps)."""
    rng = np.random.default_rng(4)
    n = 5000
    p0 = rng.normal(0, 0.02, n)
    g = rng.normal(0, 1e-3, n)
    g[:10] = 0.0
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    oracle.step_f64([g], p, m, v, None, step=1, **HP)
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    want = p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    np.testing.assert_allclose(p, want, rtol=1e-12, atol=1e-17)
    np.testing.assert_allclose(m, (1 - HP["beta1"]) * g, rtol=1e-14, atol=0)
    np.testing.assert_allclose(v, (1 - HP["beta2"]) * g * g, rtol=1e-14, atol=0)

    # the same in fp32: within 1e-6 of the fp64 closed form, relative to the
    # operands' scale |p| + lr (p' itself can cancel to near zero)
    p32, m32, v32 = p0.astype(np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g16 = oracle.f32_to_bf16(g.astype(np.float32))
    gq = oracle.bf16_to_f32(g16).astype(np.float64)
    oracle.step_f32([g16], p32, m32, v32, step=1, **HP)
    want32 = p0.astype(np.float32).astype(np.float64) * (1 - lr * wd) - lr * gq / (np.abs(gq) + eps)
    rel = np.abs(p32 - want32) / (np.abs(p0) + lr)
    assert rel.max() <= 1e-6


def test_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(5)
    n = 3000
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    decay = (np.arange(n) % 2).astype(np.uint8)
    zeros = np.zeros(n, np.uint16)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.step_f32([zeros, zeros], p, m, v, None, decay, step=1, **HP)
    d = np.float32(1.0 - np.float64(np.float32(HP["lr"])) * np.float64(np.float32(0.1)))
    assert np.array_equal(p[decay == 1], p0[decay == 1] * d)
    assert np.array_equal(p[decay == 0], p0[decay == 0])
    assert not m.any() and not v.any()


def test_scale_invariance_at_zero_eps():
    """With eps = 0 Adam's update does not depend on the gradient's scale."""
    rng = np.random.default_rng(6)
    n, steps = 2000, 20
    p0 = rng.normal(0, 1, n)
    gs = [rng.normal(0, 1, n) for _ in range(steps)]
    hp = dict(HP, eps=0.0)
    res = []
    for c in (1.0, 1024.0, 2.0 ** -20):
        p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
        for s in range(steps):
            oracle.step_f64([gs[s] * c], p, m, v, None, step=s + 1, **hp)
        res.append(p)
    np.testing.assert_allclose(res[1], res[0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(res[2], res[0], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_constant_gradient_closed_form_1000_steps(wd):
    """Constant g from zero moments: m_hat = g and v_hat = g^2 at every t, so
    theta_t = a^t theta_0 - c (1 - a^t)/(1 - a), a = 1 - lr*wd, c = lr*g/(|g|+eps)
    (theta_0 - t*c when wd = 0)."""
    rng = np.random.default_rng(7)
    n, T = 512, 1000
    hp = dict(HP, weight_decay=wd)
    lr, eps = hp["lr"], hp["eps"]
    p0 = rng.normal(0, 0.02, n)
    g16 = oracle.f32_to_bf16(rng.normal(0, 1e-3, n).astype(np.float32))
    g = oracle.bf16_to_f32(g16).astype(np.float64)
    a = 1.0 - lr * wd
    c = lr * g / (np.abs(g) + eps)

    def closed(t):
        if wd == 0:
            return p0 - t * c
        return a ** t * p0 - c * (1 - a ** t) / (1 - a)

    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    p32 = p0.astype(np.float32)
    m32, v32 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    p0_32 = p0.astype(np.float32).astype(np.float64)
    for t in range(1, T + 1):
        oracle.step_f64([g], p, m, v, None, step=t, **hp)
        oracle.step_f32([g16], p32, m32, v32, step=t, **hp)
        if t == 1:
            w32 = (a * p0_32 - c) if wd else (p0_32 - c)
            rel = np.abs(p32 - w32) / (np.abs(p0_32) + lr)
            assert rel.max() <= 1e-6
    want = closed(T)
    np.testing.assert_allclose(p, want, rtol=1e-11, atol=1e-14)
    # fp32 drift after 1000 steps: at most about one fp32 ulp of |p| per step
    w32 = (a ** T * p0_32 - c * (1 - a ** T) / (1 - a)) if wd else (p0_32 - T * c)
    assert np.all(np.abs(p32 - w32) <= T * 2.0 ** -23 * np.maximum(np.abs(w32), lr))
