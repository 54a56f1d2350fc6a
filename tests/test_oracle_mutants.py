"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pins in test_oracle_pins.py catch every one of them.

Each mutant is built from a textual edit of oracle.c in a temporary
directory (the committed oracle is never touched) and loaded as a separate
module object.  A mutant "survives" if every pin still passes; the test fails
if any mutant survives.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

import tests.test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")

MUTANTS = {
    "drop_inv_sqrt2": ("(x[a] * pre) * (x[b] * pre) * inv_sqrt2;", "(x[a] * pre) * (x[b] * pre);"),
    "wrong_prescale": ("pow((double)d, -0.25)", "pow((double)d, -0.5)"),
    "drop_linear_feature": ("out[1 + a] = x[a] * pre;", "out[1 + a] = 0.0 * x[a];"),
    "drop_constant_feature": ("out[0] = 1.0;", "out[0] = 0.0;"),
    "quadratic_exclusive_causal": ("for (int j = 0; j <= i; ++j) {", "for (int j = 0; j < i; ++j) {"),
    "quadratic_no_half": ("const double a = 1.0 + s + 0.5 * s * s;", "const double a = 1.0 + s + s * s;"),
    "quadratic_sign": ("const double a = 1.0 + s + 0.5 * s * s;", "const double a = 1.0 - s + 0.5 * s * s;"),
    "eps_outside": ("num[c] / (den + eps);", "num[c] / den + eps;"),
    "z_from_query": ("z[f] += phik[f];", "z[f] += phiq[f];"),
    "state_transposed_value": ("Sf[c] += phik[f] * vt[c];", "Sf[c] += phik[f] * vt[dv - 1 - c];"),
    "window_one_extra_key": ("const int j0 = i - window + 1 > 0 ? i - window + 1 : 0;",
                             "const int j0 = i - window > 0 ? i - window : 0;"),
    "window_no_exp": ("logit[jj] = exp(logit[jj] - m);", "logit[jj] = 1.0 + logit[jj] - m;"),
    "ring_slot_shift": ("const int slot = (int)(p % window);", "const int slot = (int)((p + 1) % window);"),
    "ring_one_key_short": ("p - window + 1 > 0 ? p - window + 1 : 0", "p - window + 2 > 0 ? p - window + 2 : 0"),
    "ring_no_key_write": ("kh[(size_t)slot * dqk + e] = k[(size_t)h * dqk + e];",
                          "kh[(size_t)slot * dqk + e] = kh[(size_t)slot * dqk + e];"),
    "fill_wrong_slot": ("const int slot = p % window;", "const int slot = (p + 1) % window;"),
    "ring_no_exp": ("const double e = exp(logit[jj] - m);", "const double e = 1.0 + logit[jj] - m;"),
    "bwd_no_linear_term": ("const double gs = ga * (1.0 + sij) * inv_sqrt_d;", "const double gs = ga * sij * inv_sqrt_d;"),
    "bwd_denominator_sign": ("gD[i] = -dy_dot_y / Di;", "gD[i] = dy_dot_y / Di;"),
    "bwd_dv_unweighted": ("dvh[(size_t)j * dv + c] += aij * gN[(size_t)i * dv + c];",
                          "dvh[(size_t)j * dv + c] += gN[(size_t)i * dv + c];"),
    "bwd_exclusive_causal": ("for (int j = i; j >= 0; --j) {", "for (int j = i - 1; j >= 0; --j) {"),
    "bwd_dk_from_key": ("dkh[(size_t)j * d + e] += gs * qh[(size_t)i * d + e];",
                        "dkh[(size_t)j * d + e] += gs * kh[(size_t)i * d + e];"),
    "rbwd_jacobian_one_side": ("acc += (u[1 + d + c * d + b] + u[1 + d + b * d + c]) * (x[b] * pre) * inv_sqrt2;",
                               "acc += u[1 + d + c * d + b] * (x[b] * pre) * inv_sqrt2;"),
    "rbwd_jacobian_prescale": ("const double pre = 1.0 / sqrt(sqrt((double)d));", "const double pre = 1.0 / sqrt((double)d);"),
    "rbwd_dq_no_normaliser": ("double acc = gD[i] * z[f];", "double acc = 0.0 * z[f];"),
    "rbwd_reverse_exclusive": ("oracle_taylor_features(kh + (size_t)j * d, d, phik);\n            for (int f = 0; f < F; ++f) {\n                double acc = z[f];",
                               "oracle_taylor_features(kh + (size_t)j * d, d, phik);\n            for (int f = 0; f < F; ++f) {\n                double acc = z[f] - phiq[f] * gD[j];"),
    "rbwd_dv_from_query": ("for (int f = 0; f < F; ++f) acc += phik[f] * S[(size_t)f * dv + c];",
                           "for (int f = 0; f < F; ++f) acc += phiq[f] * S[(size_t)f * dv + c];"),
    "swabwd_one_key_short": ("const int j0 = i + 1 - window < 0 ? 0 : i + 1 - window;",
                             "const int j0 = i + 2 - window < 0 ? 0 : i + 2 - window;"),
    "swabwd_no_D": ("const double dl = p[jj] * (dp[jj] - D) * scale;", "const double dl = p[jj] * dp[jj] * scale;"),
    "swabwd_no_scale": ("const double dl = p[jj] * (dp[jj] - D) * scale;", "const double dl = p[jj] * (dp[jj] - D);"),
    "swabwd_unnormalised": ("                p[jj] /= l;\n", ""),
    "swabwd_dk_from_key": ("dkh[(size_t)j * dqk + e] += dl * qh[(size_t)i * dqk + e];",
                           "dkh[(size_t)j * dqk + e] += dl * kh[(size_t)i * dqk + e];"),
    "swabwd_dv_unweighted": ("dvh[(size_t)j * dv + c] += p[jj] * dyh[(size_t)i * dv + c];",
                             "dvh[(size_t)j * dv + c] += dyh[(size_t)i * dv + c];"),
}

# pins that take only the oracle module
PIN_FUNCS = [
    lambda m: pins.test_p1_features_taylor_limit(m, 16),
    pins.test_p1_kernel_identity_random,
    lambda m: pins.test_p2_quadratic_equals_recurrent(m, 37, 64),
    pins.test_p3_normaliser_state,
    pins.test_p4_zero_query_is_running_mean,
    pins.test_p4_constant_values,
    pins.test_p4_linearity_and_columns,
    lambda m: pins.test_p5_window_matches_library_softmax(m, 5, 16),
    pins.test_p5_window_special_cases,
    pins.test_p6_decode_continues_prefill,
    pins.test_p7_small_logits_approach_softmax,
    lambda m: pins.test_p8_window_decode_continues_window(m, 7, 30),
    lambda m: pins.test_p8_window_decode_continues_window(m, 64, 10),
    lambda m: pins.test_p9_backward_matches_autograd(m, 16, 37, 8),
    pins.test_p9_backward_finite_differences,
    lambda m: pins.test_p10_recurrent_backward_matches_autograd(m, 16, 37, 8),
    pins.test_p10_recurrent_backward_equals_closed_form,
    pins.test_hand_taylor_cases,
    pins.test_hand_window_cases,
    lambda m: pins.test_p11_window_backward_matches_autograd(m, 5, 16, 40),
    pins.test_p11_window_backward_finite_differences,
    pins.test_p11_window_backward_special_cases,
]


def _mutant_module(tmpdir, name, old, new):
    src = open(os.path.join(ORACLE_DIR, "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/absent"
    d = os.path.join(tmpdir, name)
    os.makedirs(d)
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), d)
    shutil.copy(os.path.join(ORACLE_DIR, "__init__.py"), d)
    with open(os.path.join(d, "oracle.c"), "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    os.path.join(d, "oracle.c"), "-o", os.path.join(d, "liboracle.so"), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", os.path.join(d, "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_killed(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _mutant_module(str(tmp_path), name, old, new)
    killed_by = []
    for fn in PIN_FUNCS:
        try:
            fn(mod)
        except AssertionError:
            killed_by.append(getattr(fn, "__name__", "lambda"))
    assert killed_by, f"planted mistake {name!r} survived every pin"
