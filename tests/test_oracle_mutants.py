"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case copies oracle.c, applies one plausible mistake (a dropped term, a
wrong sign, index or operand, a changed order or rounding), builds it with the
same flags, swaps it in, and runs the pins until one fails.  A mutant that
passes every pin means the pins leave that part of the oracle unchecked.
Everything here runs on the CPU.
"""
import os
import subprocess

import pytest

import oracle as O
from oracle import build as obuild
import pins

MUTANTS = [
    ("reduce_reverse_order",
     "float s = load_elem(replicas[0], dtype, i);\n    for (int k = 1; k < P; ++k) s = s + load_elem(replicas[k], dtype, i);",
     "float s = load_elem(replicas[P - 1], dtype, i);\n    for (int k = P - 2; k >= 0; --k) s = s + load_elem(replicas[k], dtype, i);"),
    ("reduce_no_average", "g_out[i] = s * inv_scale;", "g_out[i] = s;"),
    ("omb1_from_rounded_beta", "out->omb1 = (float)(1.0 - beta1);", "out->omb1 = 1.0f - (float)beta1;"),
    ("no_bias_correction_m", "out->step_size = (float)(lr / bc1);", "out->step_size = (float)lr;"),
    ("bias_correction_v_uses_beta1", "double bc2 = 1.0 - oracle_pow_u(beta2, t);",
     "double bc2 = 1.0 - oracle_pow_u(beta1, t);"),
    ("pow_off_by_one", "double result = 1.0;", "double result = base;"),
    ("decay_after_update",
     "float th = master[i] * s->decay;\n    th = fmaf(-s->step_size, u, th);",
     "float th = fmaf(-s->step_size, u, master[i]);\n    th = th * s->decay;"),
    ("eps_inside_sqrt",
     "float root = sqrtf(vi);\n    float d = root / s->sqrt_bc2;\n    d = d + s->eps;",
     "float d = sqrtf(vi / (s->sqrt_bc2 * s->sqrt_bc2) + s->eps);"),
    ("update_sign", "th = fmaf(-s->step_size, u, th);", "th = fmaf(s->step_size, u, th);"),
    ("v_uses_beta1", "float vi = fmaf(s->b2, v[i], t3);", "float vi = fmaf(s->b1, v[i], t3);"),
    ("m_not_grad", "float t1 = s->omb1 * gc;", "float t1 = s->omb1 * g[i] * g[i];"),
    ("clip_not_applied", "float gc = g[i] * coef;", "float gc = g[i];"),
    ("v_first_power", "float t3 = t2 * gc;", "float t3 = t2;"),
    ("decay_not_applied", "out->decay = (float)(1.0 - lr_wd);", "out->decay = 1.0f;"),
    ("norm_squares_in_f32", "q = xd * xd; /* exact", "q = (double)(x * x); /* exact"),
    ("norm_group_order", "double S = (a[0] + a[1]) + (a[2] + a[3]);",
     "double S = ((a[0] + a[1]) + a[2]) + a[3];"),
    ("norm_drops_last_lane", "for (int t = 0; t < 8; ++t) {\n        size_t i = gs", "for (int t = 0; t < 7; ++t) {\n        size_t i = gs"),
    ("nonfinite_not_counted", "acc->nonfinite += 1;", "(void)0;"),
    ("fixed_point_shift", "int shift = e - 53 + 128;", "int shift = e - 52 + 128;"),
    ("acc_add_drops_carry", "    dst->w[k] = (uint32_t)t;\n    carry = t >> 32;",
     "    dst->w[k] = (uint32_t)t;\n    carry = 0;"),
    ("sumsq_truncates", "if (round_bit && (sticky || (mant & 1u))) {", "if (0) {"),
    ("clip_without_sqrt", "double norm = sqrt(sumsq);", "double norm = sumsq;"),
    ("clip_no_clamp", "return (c < 1.0) ? (float)c : 1.0f;", "return (float)c;"),
    ("clip_no_eps", "double denom = norm + 1e-6;", "double denom = norm;"),
    ("gate_skips_without_check", "if (check_overflow && acc->nonfinite > 0) return 1;",
     "if (acc->nonfinite > 0) return 1;"),
    ("gate_clip_ignores_nonfinite", "    if (acc->nonfinite > 0)\n      *coef = 0.0f;\n    else\n      *coef",
     "    if (0)\n      *coef = 0.0f;\n    else\n      *coef"),
    ("norm_drops_large_groups", "    oracle_acc_add_fixed(acc, S);\n  }\n}",
     "    if (S < 18446744073709551616.0) oracle_acc_add_fixed(acc, S);\n  }\n}"),
    ("acc_narrow_256_bits", "while (carry != 0 && k < ACC_WORDS) {", "while (carry != 0 && k < 8) {"),
    ("u_by_reciprocal", "float u = mi / d;", "float u = mi * (1.0f / d);"),
    ("m_mul_then_add", "float mi = fmaf(s->b1, m[i], t1);", "float mi = s->b1 * m[i] + t1;"),
    ("v_mul_then_add", "float vi = fmaf(s->b2, v[i], t3);", "float vi = s->b2 * v[i] + t3;"),
    ("update_mul_then_add", "th = fmaf(-s->step_size, u, th);", "th = -s->step_size * u + th;"),
    ("gc_flushes_subnormals", "float gc = g[i] * coef;",
     "float gc = g[i] * coef; if (fabsf(gc) < 1.17549435e-38f) gc = 0.0f;"),
    ("v_flushes_subnormals", "float vi = fmaf(s->b2, v[i], t3);",
     "float vi = fmaf(s->b2, v[i], t3); if (vi < 1.17549435e-38f) vi = 0.0f;"),
    ("other_ranks_ignored", "for (int k = 0; k < n_extra; ++k) oracle_acc_add",
     "for (int k = 0; k < 0; ++k) oracle_acc_add"),
    ("bf16_ties_up", "up = (lo_mag & 1u) ? 1 : 0; /* tie", "up = 1; /* tie"),
    ("bf16_nan_unsigned", "if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);",
     "if (isnan(x)) return (uint16_t)0x7FC0u;"),
    ("e4m3_nan_on_saturation", "if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
     "if (a >= 448.0) return (uint8_t)(sign | 0x7F);"),
    ("e4m3_round_half_up", "return (fmod(k, 2.0) == 0.0) ? k : k + 1.0;", "return k + 1.0;"),
    ("e4m3_subnormal_step", "double k = rne_int(ldexp(a, 9));", "double k = rne_int(ldexp(a, 8));"),
    ("mx_scale_emax", "int e_s = E - 8;", "int e_s = E - 7;"),
    ("mx_scale_no_clamp", "if (e_s < -127) e_s = -127;", "(void)0;"),
    ("mx_zero_block_scale", "      scale[b] = 0x00;\n", "      scale[b] = 0x7F;\n"),
    ("mx_inf_not_special", "if (!isfinite(val))", "if (isnan(val))"),
    ("mx_decode_bias", "out[i] = (float)ldexp(val, (int)sb - 127);", "out[i] = (float)ldexp(val, (int)sb - 126);"),
    ("mx_decode_nan_scale", "if (sb == 0xFF || isnan(val)) {", "if (isnan(val)) {"),
    ("mx_decode_block_index", "uint8_t sb = scale[i / 32];", "uint8_t sb = scale[i / 16];"),
]


def _build_mutant(tmpdir, name, old, new):
    src = open(obuild.SRC[0]).read()
    assert src.count(old) == 1, f"mutation site of {name} not unique/found"
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmpdir, f"lib{name}.so")
    subprocess.run(["gcc", *obuild.CFLAGS, "-Wno-unused", "-I", os.path.dirname(obuild.SRC[0]),
                    "-o", so, path, "-lm"], check=True, capture_output=True)
    return so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    so = _build_mutant(str(tmp_path), name, old, new)
    prev = O.use_library(so)
    caught = None
    try:
        for check in pins.ALL_CHEAP_FIRST:
            try:
                check()
            except Exception as e:  # AssertionError, or a crash-free error
                caught = (check.__name__, type(e).__name__)
                break
    finally:
        O.use_library(prev if prev is not None else obuild.LIB)
    assert caught is not None, f"mutant {name} passed every pin"
