"""Pins of the oracle's global-norm clip: torch.nn.utils.clip_grad_norm_ (a
library routine) in fp64, a closed form, and independence of the thread count."""
import numpy as np
import torch

import oracle


def test_norm_and_coef_match_torch_clip_grad_norm():
    rng = np.random.default_rng(30)
    M, n = 4, 300_001
    gs = [oracle.f32_to_bf16(rng.normal(0, 1e-2, n).astype(np.float32)) for _ in range(M)]
    g = oracle.reduce_mean_f32(gs).astype(np.float64)
    # split into "tensors" as torch would see them
    parts = np.split(g, [1000, 70_000, 200_000])
    for max_norm in (0.1, 1.0, 1e3):
        ts = [torch.tensor(p.copy()) for p in parts]
        for t in ts:
            t.grad = t.clone()
        total = float(torch.nn.utils.clip_grad_norm_(ts, max_norm))
        sumsq = oracle.grad_sumsq(gs)
        assert abs(np.sqrt(sumsq) - total) <= 1e-12 * total
        want = min(1.0, max_norm / (total + 1e-6))
        coef = oracle.clip_coef(sumsq, max_norm)
        assert abs(float(coef) - want) <= 2.0 ** -24 * want
        # the clipped gradient torch writes equals g * coef to fp32 rounding
        clipped = np.concatenate([t.grad.numpy() for t in ts])
        np.testing.assert_allclose(clipped, g * float(coef), rtol=1e-7, atol=0)


def test_norm_of_constant_gradient_closed_form():
    """All-equal g = c over S elements: ||g|| = |c| * sqrt(S)."""
    S = 1 << 20
    c = np.float32(-0.0078125)        # 2^-7: every partial sum is exact
    gs = [oracle.f32_to_bf16(np.full(S, c, np.float32))] * 3
    sumsq = oracle.grad_sumsq(gs)
    assert sumsq == float(c) ** 2 * S
    assert np.sqrt(sumsq) == abs(float(c)) * np.sqrt(S)
    assert oracle.clip_coef(sumsq, 1e9) == np.float32(1.0)


def test_results_do_not_depend_on_thread_count():
    rng = np.random.default_rng(31)
    M, n = 3, 500_000
    gs = [oracle.f32_to_bf16(rng.normal(0, 1, n).astype(np.float32)) for _ in range(M)]
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    before = oracle.get_threads()
    outs = []
    try:
        for th in (1, 3, 8):
            oracle.set_threads(th)
            s = oracle.grad_sumsq(gs)
            p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
            oracle.step_f32(gs, p, m, v, step=1, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                            weight_decay=0.1, coef=oracle.clip_coef(s, 1.0))
            outs.append((s, p))
    finally:
        oracle.set_threads(before)
    for s, p in outs[1:]:
        assert s == outs[0][0]
        assert np.array_equal(p.view(np.uint32), outs[0][1].view(np.uint32))
