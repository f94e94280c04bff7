"""Pins of the oracle's fp16 variant with dynamic loss scaling.

* fp16 -> fp32 over all 65,536 patterns against numpy's, and fp32 -> fp16 over
  all 2^32 patterns against torch's (library routines, round to nearest even);
* the scale update against torch._amp_update_scale_ and the unscale + found-inf
  test against torch._amp_foreach_non_finite_check_and_unscale_ (library
  routines, CPU);
* the whole sequence (skips, backoff, growth, applied-step count) against
  torch.optim.AdamW driven the way torch's GradScaler drives it.
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
