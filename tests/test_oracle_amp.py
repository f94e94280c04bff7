"""Pins of the oracle's fp16 variant with dynamic loss scaling.

* fp16 -> fp32 over all 65,536 patterns against numpy's, and fp32 -> fp16 over
  all 2^32 patterns against torch's (library routines, round to nearest even);
* the scale update against torch._amp_update_scale_ and the unscale + found-inf
  test against torch._amp_foreach_non_finite_check_and_unscale_ (library
  routines, CPU);
* the whole sequence (skips, backoff, growth, applied-step count) against
  torch.optim.AdamW driven the way torch's GradScaler drives it, and a
  clipped sequence against torch's own GradScaler (unscale_, clip_grad_norm_,
  step, update) with the clip binding on alternate steps;
* the loss-scaled sum of squares against torch.nn.utils.clip_grad_norm_ in
  fp64 on the unscaled average (library routine) and against the closed form
  of a constant gradient, ||g|| = |c| sqrt(S);
* growth that would overflow the scale keeps it (torch._amp_update_scale_,
  started next to the largest finite fp32 with growth every step).

Clipping is part of the AdamW recipe of Lecture 9 分布式训练 (CS324 notes),
§7.4; the loss scaler that must keep up with fp16 overflow is CS324 notes §13
and 大模型基础设施工程 06, §12.4 pitfall 7.
"""
import numpy as np
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def test_f16_to_f32_exhaustive():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(pats)
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_exhaustive():
    chunk = 1 << 24
    base = np.arange(chunk, dtype=np.uint32)
    u = np.empty(chunk, dtype=np.uint32)
    ref_t = torch.empty(chunk, dtype=torch.float16)
    for start in range(0, 1 << 32, chunk):
        np.add(base, np.uint32(start), out=u)
        x = u.view(np.float32)
        ours = oracle.f32_to_f16(x)
        ref_t.copy_(torch.from_numpy(x))          # torch's RNE conversion (library routine)
        ref = ref_t.view(torch.int16).numpy().view(np.uint16)
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        if not nan.any():
            assert np.array_equal(ours, ref), hex(start)
            continue
        assert np.array_equal(ours[~nan], ref[~nan]), hex(start)
        on = ours[nan]
        assert np.all((on & 0x7C00) == 0x7C00) and np.all((on & 0x3FF) != 0)


def test_scale_update_matches_torch():
    rng = np.random.default_rng(40)
    sc = oracle.Scaler(scale=2.0 ** 16, growth_factor=2.0, backoff_factor=0.5, growth_interval=7)
    ts = torch.tensor([2.0 ** 16])
    tg = torch.zeros(1, dtype=torch.int32)
    for _ in range(3000):
        fi = bool(rng.random() < 0.1)
        sc.update(fi)
        torch._amp_update_scale_(ts, tg, torch.tensor([1.0 if fi else 0.0]), 2.0, 0.5, 7)
        assert sc.scale[0] == np.float32(ts.item()) and sc.tracker[0] == tg.item()


def test_unscale_and_found_inf_match_torch():
    rng = np.random.default_rng(41)
    M, n = 3, 40_000
    for scale in (2.0 ** 16, 3.0, 2.0 ** 24):
        inv = oracle.inv_scale(scale)
        assert inv == np.float32(torch.tensor([scale], dtype=torch.float64).reciprocal().item())
        gs = [oracle.f32_to_f16((rng.normal(0, 1e-3, n) * scale).astype(np.float32))
              for _ in range(M)]
        for poison in (None, np.inf, np.nan):
            if poison is not None:
                gs[1][777] = oracle.f32_to_f16(np.array([poison], np.float32))[0]
            s = oracle.f16_to_f32(gs[0])
            for g in gs[1:]:
                s = s + oracle.f16_to_f32(g)
            scaled_mean = torch.from_numpy(s / np.float32(M))
            fi = torch.zeros(1)
            torch._amp_foreach_non_finite_check_and_unscale_([scaled_mean], fi,
                                                              torch.tensor([float(inv)]))
            ours = oracle.reduce_mean_f16(gs, inv)
            ref = scaled_mean.numpy()
            both_nan = np.isnan(ours) & np.isnan(ref)
            assert np.array_equal(ours.view(np.uint32)[~both_nan], ref.view(np.uint32)[~both_nan])
            found = not np.isfinite(oracle.grad_sumsq_f16(gs, inv))
            assert found == bool(fi.item())


def test_amp_sequence_matches_torch_adamw_and_gradscaler():
    """Skipped steps leave the state alone and do not advance the step count."""
    rng = np.random.default_rng(42)
    n, M, steps = 6000, 2, 40
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    sc = oracle.Scaler(scale=2.0 ** 15, growth_interval=5)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    pf = np.zeros(n, np.uint16)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False, fused=False)
    ts, tg = torch.tensor([2.0 ** 15]), torch.zeros(1, dtype=torch.int32)
    skipped = 0
    for s in range(steps):
        scale = float(sc.scale[0])
        assert scale == ts.item()
        gs = [oracle.f32_to_f16((rng.normal(0, 1e-3, n) * scale).astype(np.float32))
              for _ in range(M)]
        if s % 9 == 4:   # overflow in one contribution
            gs[0][123] = 0x7C00
        fi, _ = oracle.amp_step(gs, p, m, v, pf, None, sc, **HP)
        # torch: average the scaled contributions in fp32, unscale, step unless found-inf
        acc = oracle.f16_to_f32(gs[0])
        for g in gs[1:]:
            acc = acc + oracle.f16_to_f32(g)
        grad = torch.from_numpy(acc / np.float32(M))
        tfi = torch.zeros(1)
        torch._amp_foreach_non_finite_check_and_unscale_([grad], tfi,
                                                          ts.double().reciprocal().float())
        assert fi == bool(tfi.item())
        if not fi:
            tp.grad = grad
            opt.step()
        else:
            skipped += 1
        torch._amp_update_scale_(ts, tg, tfi, 2.0, 0.5, 5)
    assert skipped == sum(1 for s in range(steps) if s % 9 == 4)
    assert sc.applied == steps - skipped
    assert opt.state[tp]["step"].item() == sc.applied
    # torch rounds the moments differently (lerp/addcmul): a few fp32 ulps per step,
    # accumulated over the applied steps, are expected; a wrong step count, a
    # missed skip or a wrong scale would be off by orders of magnitude more
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-6, atol=5e-8)
    assert np.array_equal(pf, oracle.f32_to_f16(p))


def test_f32_to_f16_special_cases():
    def h(x):
        return int(oracle.f32_to_f16(np.array([x], dtype=np.float32))[0])

    def f(bits):
        return np.array([bits], dtype=np.uint32).view(np.float32)[0]

    assert h(1.0) == 0x3C00 and h(-2.0) == 0xC000
    assert h(65504.0) == 0x7BFF and h(65519.0) == 0x7BFF and h(65520.0) == 0x7C00
    assert h(f(0x3F801000)) == 0x3C00          # tie between 1.0 and 1+2^-10: even
    assert h(f(0x3F803000)) == 0x3C02          # tie between 1+2^-10 and 1+2^-9: even
    assert h(2.0 ** -24) == 0x0001 and h(2.0 ** -25) == 0 and h(3 * 2.0 ** -25) == 0x0002
    assert h(5 * 2.0 ** -25) == 0x0002 and h(7 * 2.0 ** -25) == 0x0004   # subnormal ties: even
    assert h(2.0 ** -14) == 0x0400 and h(2.0 ** -14 - 2.0 ** -25) == 0x0400
    assert h(-0.0) == 0x8000 and h(np.inf) == 0x7C00 and h(-np.inf) == 0xFC00


def _f16_contributions(rng, n, M, scale, sigma=1e-3):
    return [oracle.f32_to_f16((rng.normal(0, sigma, n) * scale).astype(np.float32))
            for _ in range(M)]


def _torch_unscaled_average(gs, scale):
    """The unscaled fp32 average with numpy's fp16 widening and torch's unscale
    routine (inv_scale = fp32(1/scale) taken in fp64, as GradScaler does)."""
    acc = gs[0].view(np.float16).astype(np.float32)
    for g in gs[1:]:
        acc = acc + g.view(np.float16).astype(np.float32)
    avg = torch.from_numpy(acc / np.float32(len(gs)))
    fi = torch.zeros(1)
    inv = torch.tensor([scale], dtype=torch.float64).reciprocal().float()
    torch._amp_foreach_non_finite_check_and_unscale_([avg], fi, inv)
    return avg, bool(fi.item())


def test_f16_sumsq_matches_clip_grad_norm_f64():
    """sqrt(grad_sumsq_f16) is the L2 norm of the unscaled average: torch's
    clip_grad_norm_ over an fp64 copy of that average, split over several
    tensors as a model's parameters would be."""
    rng = np.random.default_rng(43)
    for M, n, scale in ((1, 5000, 2.0 ** 16), (3, 40_000, 2.0 ** 12), (8, 12_345, 3.0)):
        gs = _f16_contributions(rng, n, M, scale)
        ours = float(np.sqrt(oracle.grad_sumsq_f16(gs, oracle.inv_scale(scale))))
        avg, fi = _torch_unscaled_average(gs, scale)
        assert not fi
        cuts = [0, n // 7, n // 3, n - 1, n]
        ps = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            p = torch.nn.Parameter(torch.zeros(b - a, dtype=torch.float64))
            p.grad = avg[a:b].double().clone()
            ps.append(p)
        ref = float(torch.nn.utils.clip_grad_norm_(ps, max_norm=1e30))
        assert abs(ours - ref) <= 1e-12 * ref, (M, n, ours, ref)


def test_f16_sumsq_constant_gradient_closed_form():
    """Every contribution c * scale, exact in fp16 (scale a power of two): the
    average is c exactly, so the sum of squares is c^2 S exactly and the norm
    |c| sqrt(S); S = 4^k makes the square root exact too."""
    for c, scale, M, S in ((3 * 2.0 ** -10, 2.0 ** 12, 4, 1 << 16),
                           (-5 * 2.0 ** -12, 2.0 ** 15, 3, 1 << 14),
                           (2.0 ** -7, 1.0, 1, 1 << 10)):
        h = oracle.f32_to_f16(np.full(S, c * scale, np.float32))
        assert np.all(oracle.f16_to_f32(h) == np.float32(c * scale))
        sumsq = oracle.grad_sumsq_f16([h] * M, oracle.inv_scale(scale))
        assert sumsq == c * c * S
        assert np.sqrt(sumsq) == abs(c) * np.sqrt(S)


def test_amp_clipped_sequence_matches_torch_gradscaler():
    """fp16 contributions of a scaled loss, the clip binding on alternate steps,
    an overflow every ninth step: torch's GradScaler drives torch AdamW
    (unscale_, then clip_grad_norm_ on the unscaled gradient, then step, then
    update) and the oracle's amp_step must follow it -- the same skips, scale,
    growth count, applied steps and reported norm, and parameters within the
    few-ulp moment rounding difference."""
    rng = np.random.default_rng(44)
    n, M, steps = 6000, 2, 30
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    sc = oracle.Scaler(scale=2.0 ** 15, growth_interval=3)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    pf = np.zeros(n, np.uint16)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False, fused=False)
    gsc = torch.amp.GradScaler("cpu", init_scale=2.0 ** 15, growth_factor=2.0,
                               backoff_factor=0.5, growth_interval=3)
    bound = 0
    for s in range(steps):
        scale = float(sc.scale[0])
        loss_scaled = gsc.scale(torch.ones(()))   # what backward would be run on
        assert scale == float(loss_scaled) == gsc.get_scale()
        gs = _f16_contributions(rng, n, M, scale)
        if s % 9 == 4:
            gs[1][321] = 0x7C00
        max_norm = 0.01 if s % 2 else 1e3     # ||g|| is about 0.055: binding, then not
        fi, norm = oracle.amp_step(gs, p, m, v, pf, None, sc, max_grad_norm=max_norm, **HP)
        acc = gs[0].view(np.float16).astype(np.float32)
        for g in gs[1:]:
            acc = acc + g.view(np.float16).astype(np.float32)
        tp.grad = torch.from_numpy(acc / np.float32(M))
        gsc.unscale_(opt)
        tfi = sum(v.item() for v in gsc._found_inf_per_device(opt).values()) > 0
        assert fi == tfi == (s % 9 == 4)
        if not fi:
            tnorm = float(torch.linalg.vector_norm(tp.grad.double()))
            assert abs(norm - tnorm) <= 1e-12 * tnorm
            clipped_to = float(torch.nn.utils.clip_grad_norm_([tp], max_norm))
            assert abs(clipped_to - tnorm) <= 1e-6 * tnorm
            bound += norm > max_norm
        gsc.step(opt)
        gsc.update()
        assert sc.scale[0] == np.float32(gsc.get_scale())
        assert sc.tracker[0] == int(gsc._growth_tracker.item())
    assert bound == sum(1 for s in range(steps) if s % 2 and s % 9 != 4)
    assert sc.applied == opt.state[tp]["step"].item() == steps - sum(
        1 for s in range(steps) if s % 9 == 4)
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-6, atol=5e-8)
    assert np.array_equal(pf, oracle.f32_to_f16(p))


def test_scale_growth_keeps_finite_scale_near_flt_max():
    """Growth that would take the scale to Inf leaves it where it is and restarts
    the growth count (torch._amp_update_scale_), from the largest finite fp32
    scale and from 2^127 with growth every step."""
    fmax = float(np.finfo(np.float32).max)
    for start in (fmax, 2.0 ** 127, 2.0 ** 126):
        sc = oracle.Scaler(scale=start, growth_factor=2.0, backoff_factor=0.5, growth_interval=1)
        ts = torch.tensor([start], dtype=torch.float32)
        tg = torch.zeros(1, dtype=torch.int32)
        for k in range(6):
            fi = k == 4
            sc.update(fi)
            torch._amp_update_scale_(ts, tg, torch.tensor([1.0 if fi else 0.0]), 2.0, 0.5, 1)
            assert np.isfinite(sc.scale[0])
            assert sc.scale[0] == np.float32(ts.item()) and sc.tracker[0] == tg.item(), (start, k)
