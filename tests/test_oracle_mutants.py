"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped term,
a wrong sign or constant, transposed operands, a skipped contribution, a
truncating conversion, FMA contraction), builds it on the CPU, and runs the
pin checks of the test_oracle_* modules against that build in this process:
at least one must fail.  The unmodified source, built the same way, must pass
all of them.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_adamw as A
import test_oracle_amp as P
import test_oracle_bf16 as B
import test_oracle_clip as K
import test_oracle_reduce as R
import test_oracle_rounding as X
import test_oracle_shard as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the pin checks, cheapest first
PINS = [
    lambda: R.test_ring_allreduce_worked_example(),
    lambda: R.test_accumulated_mean_equals_big_batch_gradient_bf16_exact(5),
    lambda: R.test_accumulated_mean_equals_big_batch_gradient_f64(3),
    lambda: X.test_reduce_is_sequential_single_rounded(3),
    lambda: X.test_reduce_is_sequential_single_rounded(4),
    lambda: X.test_step_is_single_rounded_per_operation(1),
    lambda: X.test_step_is_single_rounded_per_operation(7),
    lambda: A.test_zero_gradient_is_pure_decay(),
    lambda: A.test_first_step_closed_form(),
    lambda: A.test_scale_invariance_at_zero_eps(),
    lambda: A.test_f64_matches_torch_adamw_f64(),
    lambda: A.test_f64_wd0_matches_torch_adam(),
    lambda: A.test_f32_matches_torch_adamw_f32(),
    lambda: A.test_constant_gradient_closed_form_1000_steps(0.1),
    lambda: B.test_f32_to_bf16_special_cases(),
    lambda: B.test_bf16_to_f32_exhaustive(),
    lambda: Z.test_padding_is_inert(1),
    lambda: Z.test_sharded_equals_unsharded(3, 0, 0.05),
    lambda: K.test_norm_of_constant_gradient_closed_form(),
    lambda: K.test_norm_and_coef_match_torch_clip_grad_norm(),
    lambda: X.test_pow_int_against_exact_rationals(),
    lambda: X.test_step_constants_exactly_rounded(1000),
    lambda: P.test_f32_to_f16_special_cases(),
    lambda: P.test_f16_to_f32_exhaustive(),
    lambda: P.test_scale_update_matches_torch(),
    lambda: P.test_unscale_and_found_inf_match_torch(),
    lambda: P.test_amp_sequence_matches_torch_adamw_and_gradscaler(),
    lambda: P.test_f16_sumsq_constant_gradient_closed_form(),
    lambda: P.test_f16_sumsq_matches_clip_grad_norm_f64(),
    lambda: P.test_scale_growth_keeps_finite_scale_near_flt_max(),
    lambda: P.test_amp_clipped_sequence_matches_torch_gradscaler(),
]

U, C = "zo_update.inc", "zo.c"
MUTANTS = [
    ("c1-uses-beta2", C, "k.c1 = 1.0 - beta1;", "k.c1 = 1.0 - beta2;"),
    ("no-bias-correction-m", C, "k.alpha = lr / bc1;", "k.alpha = lr;"),
    ("no-bias-correction-v", C, "k.bhat = sqrt(bc2);", "k.bhat = 1.0;"),
    ("betas-swapped", C, "    k.beta1 = beta1;\n    k.beta2 = beta2;\n    k.c1 = (float)d.c1;",
     "    k.beta1 = beta2;\n    k.beta2 = beta1;\n    k.c1 = (float)d.c1;"),
    ("decay-sign", C, "k.decay_mul = 1.0 - lr * wd;", "k.decay_mul = 1.0 + lr * wd;"),
    ("no-eps", U, "ZO_REAL den = q + k->eps;", "ZO_REAL den = q;"),
    ("update-sign", U, "*p = p1 - w;", "*p = p1 + w;"),
    ("no-decay", U, "ZO_REAL p1 = *p * d;", "ZO_REAL p1 = *p;"),
    ("v-uses-g", U, "ZO_REAL gg = g * g;", "ZO_REAL gg = g;"),
    ("m-drops-1-beta1", U, "ZO_REAL mG = k->c1 * g;", "ZO_REAL mG = g;"),
    ("sqrt-transposed", U, "ZO_REAL q = r / k->bhat;", "ZO_REAL q = k->bhat / r;"),
    ("no-sqrt", U, "ZO_REAL r = ZO_SQRT(v1);", "ZO_REAL r = v1;"),
    ("m-over-den-transposed", U, "ZO_REAL u = m1 / den;", "ZO_REAL u = den / m1;"),
    ("reduce-skips-last", C, "for (int32_t j = 1; j < M; j++)\n        s = s + bf16_to_f32",
     "for (int32_t j = 1; j < M - 1; j++)\n        s = s + bf16_to_f32"),
    ("reduce-no-divide", C, "return s / (float)M;", "return s;"),
    ("bf16-truncates", C, "return (uint16_t)((u + 0x7fffu + lsb) >> 16);",
     "return (uint16_t)(u >> 16);"),
    ("bf16-ties-away", C, "uint32_t lsb = (u >> 16) & 1u;", "uint32_t lsb = 1u;"),
    ("norm-not-squared", C, "double g = (double)mean_f32(grads, M, i);\n            acc += g * g;",
     "double g = (double)mean_f32(grads, M, i);\n            acc += g < 0 ? -g : g;"),
    ("clip-no-guard", C, "double c = (double)max_norm / (norm + 1e-6);",
     "double c = (double)max_norm / norm;"),
    ("clip-not-clamped", C, "    if (c > 1.0)\n        c = 1.0;\n    return (float)c;",
     "    return (float)c;"),
    ("pow-int-wrong-square", C, "        x = x * x;", "        x = x * b;"),
    ("f16-no-unscale", C, "    return g * inv_scale;", "    return g;"),
    ("f16-truncates", C, "uint32_t r = (m + 0xfffu + ((m >> 13) & 1u)) >> 13;",
     "uint32_t r = m >> 13;"),
    ("f16-subnormal-ties-up", C, "if (rem > half || (rem == half && (q & 1u)))",
     "if (rem >= half)"),
    ("f16-widen-subnormal-scale", C, "float f = (float)mant * 5.9604644775390625e-8f;",
     "float f = (float)mant * 1.1920928955078125e-7f;"),
    ("scaler-no-backoff", C, "*scale = *scale * backoff_factor;", "*scale = *scale;"),
    ("scaler-growth-late", C, "if (good == growth_interval) {", "if (good > growth_interval) {"),
    ("scaler-grows-to-inf", C, "            if (isfinite(grown))\n                *scale = grown;",
     "            *scale = grown;"),
    ("f16-norm-not-squared", C,
     "double g = (double)mean_f16_unscaled(grads, M, i, inv_scale);\n            acc += g * g;",
     "double g = (double)mean_f16_unscaled(grads, M, i, inv_scale);\n            acc += g < 0 ? -g : g;"),
    ("f16-norm-on-scaled-average", C,
     "double g = (double)mean_f16_unscaled(grads, M, i, inv_scale);",
     "double g = (double)mean_f16_unscaled(grads, M, i, 1.0f);"),
    ("amp-coef-from-scaled-norm", C,
     "float coef = use_coef ? zo_coef_from_norm(norm, max_norm) : 1.0f;",
     "float coef = use_coef ? zo_coef_from_norm(norm * (double)*scale, max_norm) : 1.0f;"),
    ("amp-clip-ignored", C, "int32_t use_coef = max_norm > 0.0f;", "int32_t use_coef = 0;"),
    ("amp-skip-advances-t", C, "        *applied += 1;\n    }\n    zo_scaler_update(",
     "    }\n    *applied += 1;\n    zo_scaler_update("),
    ("fma-contraction", None, None, None),
]


def _build(tmp, replace=None, extra=()):
    src = os.path.join(ROOT, "oracle")
    for f in (C, U):
        shutil.copy(os.path.join(src, f), tmp / f)
    if replace:
        fname, old, new = replace
        text = (tmp / fname).read_text()
        assert text.count(old) == 1, f"mutation anchor not found once: {old!r}"
        (tmp / fname).write_text(text.replace(old, new))
    lib = tmp / "libzo_mut.so"
    flags = [f for f in oracle.CFLAGS if f != "-ffp-contract=off" or not extra] + list(extra)
    subprocess.run(["gcc", *flags, "-o", str(lib), str(tmp / C), "-lm"], check=True)
    return str(lib)


def _pins_pass(lib) -> bool:
    """True when every pin check passes against the build at `lib`."""
    oracle.use_library(lib)
    try:
        for check in PINS:
            try:
                check()
            except (AssertionError, ValueError):
                return False
        return True
    finally:
        oracle.use_library(None)


def test_unmodified_source_passes_the_pins(tmp_path):
    assert _pins_pass(_build(tmp_path))


@pytest.mark.parametrize("name,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, fname, old, new):
    if name == "fma-contraction":
        lib = _build(tmp_path, extra=("-ffp-contract=fast", "-mfma"))
    else:
        lib = _build(tmp_path, (fname, old, new))
    assert not _pins_pass(lib), f"no pin caught the planted mistake '{name}'"
