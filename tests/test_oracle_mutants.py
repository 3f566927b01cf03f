"""Plant plausible mistakes in copies of the oracle's C source (on the CPU) and
require every one of them to fail at least one pin.  This is what makes the
pins a check of the oracle rather than a restatement of it."""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement): each is a mistake someone could make.
MUTANTS = [
    ("dropped_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("mask_off_by_one", "if (j >= visible) { s[j] = -INFINITY; continue; }",
     "if (j > visible) { s[j] = -INFINITY; continue; }"),
    ("wrong_sign_in_exp", "p[j] = exp(s[j] - m);", "p[j] = exp(m - s[j]);"),
    ("lse_without_max", "*lse = m + log(l);", "*lse = log(l);"),
    ("q_dot_q", "for (long t = 0; t < d; ++t) dot += q[t] * k[t];",
     "for (long t = 0; t < d; ++t) dot += q[t] * q[t];"),
    ("missing_normalisation", "for (long j = 0; j < n; ++j) p[j] /= l;",
     "for (long j = 0; j < n; ++j) p[j] /= 1.0;"),
    ("value_without_weight", "for (long t = 0; t < d; ++t) o[t] += p[j] * v[t];",
     "for (long t = 0; t < d; ++t) o[t] += v[t];"),
    ("transposed_value_index", "const double *v = V + j * d;",
     "const double *v = V + (n - 1 - j) * d;"),
    ("softmax_not_normalised", "y[j] = exp(x[j] - m) / s;", "y[j] = exp(x[j] - m);"),
    ("softmax_max_is_first", "if (x[j] > m) m = x[j];", "if (j == 0) m = x[j];"),
    ("online_correction_sign",
     "double correction = (m == -INFINITY) ? 0.0 : exp(m - m_new);",
     "double correction = (m == -INFINITY) ? 0.0 : exp(m_new - m);"),
    ("online_no_accumulator_rescale",
     "for (long t = 0; t < d; ++t) a[r * d + t] *= corr;",
     "for (long t = 0; t < d; ++t) a[r * d + t] *= 1.0;"),
    ("online_causal_off_by_one",
     "if (causal && j > i) { S[r * bc + c] = -INFINITY; continue; }",
     "if (causal && j >= i) { S[r * bc + c] = -INFINITY; continue; }"),
    ("online_denominator_not_rescaled", "l[r] = corr * l[r] + psum;",
     "l[r] = l[r] + psum;"),
    ("merge_weight_sign", "double wb = exp(m_b - m_new);", "double wb = exp(m_new - m_b);"),
    ("merge_denominator_unweighted", "l = wa * l + wb * 1.0;", "l = l + 1.0;"),
    ("merge_accumulator_not_rescaled",
     "for (long t = 0; t < d; ++t) a[t] = wa * a[t] + wb * a_b[t];",
     "for (long t = 0; t < d; ++t) a[t] = a[t] + wb * a_b[t];"),
    ("merge_lse_without_max", "lse[r] = m + log(l);", "lse[r] = log(l);"),
    ("merge_keeps_first_partial_only", "if (m_b == -INFINITY) continue;",
     "if (m_b == -INFINITY || s > 0) continue;"),
    ("bwd_softmax_jacobian_sign",
     "for (long j = 0; j < N; ++j) dS[i * N + j] = P[i * N + j] * (dS[i * N + j] - D);",
     "for (long j = 0; j < N; ++j) dS[i * N + j] = P[i * N + j] * (D - dS[i * N + j]);"),
    ("bwd_missing_row_term",
     "for (long j = 0; j < N; ++j) dS[i * N + j] = P[i * N + j] * (dS[i * N + j] - D);",
     "for (long j = 0; j < N; ++j) dS[i * N + j] = P[i * N + j] * dS[i * N + j];"),
    ("bwd_dq_without_scale", "dQs[r * d + t] = scale * aq;", "dQs[r * d + t] = aq;"),
    ("bwd_dk_from_keys", "ak += dS[i * N + r] * Qs[i * d + t];", "ak += dS[i * N + r] * Ks[i * d + t];"),
    ("bwd_dv_transposed_p", "av += P[i * N + r] * dOs[i * d + t];", "av += P[r * N + i] * dOs[i * d + t];"),
    ("bwd_dp_from_keys", "for (long t = 0; t < d; ++t) dp += dOs[i * d + t] * Vs[j * d + t];",
     "for (long t = 0; t < d; ++t) dp += dOs[i * d + t] * Ks[j * d + t];"),
    ("fp8_exponent_bias_8", "v = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("fp8_mantissa_over_16", "v = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "v = ldexp(1.0 + (double)m / 16.0, e - 7);"),
    ("fp8_subnormal_scale", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("fp8_no_nan", "if (e == 15 && m == 7)", "if (e == 16)"),
    ("fp8_scale_dropped", "y[i] = (sign ? -v : v) * s;", "y[i] = (sign ? -v : v);"),
    ("encode_ties_away", "int q = (int)rint((ldexp(a, -E) - 1.0) * 8.0);",
     "int q = (int)round((ldexp(a, -E) - 1.0) * 8.0);"),
    ("encode_subnormal_step", "c = (int)rint(a * 512.0);", "c = (int)rint(a * 256.0);"),
    ("encode_exponent_bias", "c = ((E + 7) << 3) | q;", "c = ((E + 8) << 3) | q;"),
    ("encode_sign_dropped", "*code = (unsigned char)((sign << 7) | c);", "*code = (unsigned char)c;"),
    ("encode_scale_multiplies", "if (fp8_e4m3_encode_one(x[i] / s, &out[i]) != 0) return -3;",
     "if (fp8_e4m3_encode_one(x[i] * s, &out[i]) != 0) return -3;"),
    ("hadamard_not_normalised", "Y[r * d + k] = acc * norm;", "Y[r * d + k] = acc;"),
    ("hadamard_sign_on_output", "acc += x[t] * signs[t] * (odd ? -1.0 : 1.0);",
     "acc += x[t] * signs[k] * (odd ? -1.0 : 1.0);"),
    ("hadamard_parity_of_or", "__builtin_popcountl((unsigned long)(t & k)) & 1",
     "__builtin_popcountl((unsigned long)(t | k)) & 1"),
    ("mx_scale_not_smallest", "while (amax <= 448.0 * ldexp(1.0, e - 1)) --e;",
     "while (amax <= 448.0 * ldexp(1.0, e - 2)) --e;"),
    ("mx_fit_strict", "while (amax <= 448.0 * ldexp(1.0, e - 1)) --e;",
     "while (amax < 448.0 * ldexp(1.0, e - 1)) --e;"),
    ("mx_scale_bias", "scales[r * (d / 32) + blk] = (unsigned char)(e + 127);",
     "scales[r * (d / 32) + blk] = (unsigned char)(e + 128);"),
    ("mx_decode_rows_block_index", "scales[r * (d / 32) + t / 32] - 127",
     "scales[r * (d / 32) + t % (d / 32)] - 127"),
    ("mx_cols_block_short", "r1 = (32 * i + 32 < n) ? 32 * i + 32 : n;",
     "r1 = (32 * i + 31 < n) ? 32 * i + 31 : n;"),
    ("mx_decode_cols_row_block", "scales[(sl * nb + r / 32) * d + t] - 127",
     "scales[(sl * nb + r / 33) * d + t] - 127"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    so = oracle_build.build(src=str(src), out=str(tmp_path / "liboracle_mutant.so"))
    mutant = oracle.Oracle(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
