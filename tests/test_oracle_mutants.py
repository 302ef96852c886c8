"""Plant mistakes in copies of the oracle (CPU only) and check the pins catch each.

Every mutant is a textual patch of oracle/path_oracle.c compiled into a
temporary library; the real oracle is never modified.  A mutant survives if
every pin in oracle_pins passes on it, which fails this test.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "path_oracle.c")

# (id, text to replace, replacement, expected occurrences)
MUTANTS = [
    ("off_by_one_H", "apply_h(u, w + (size_t)(j + 1) * d, beta[j + 1], d);", "apply_h(u, w + (size_t)j * d, beta[j], d);", 2),
    ("apply_h_no_beta", "u[c] -= beta * wu * w[c];", "u[c] -= wu * w[c];", 1),
    ("apply_h_sign", "u[c] -= beta * wu * w[c];", "u[c] += beta * wu * w[c];", 1),
    ("apply_h_drop_dot_term", "wu += w[c] * u[c];", "wu += w[c];", 1),
    ("fox_bias_index", "if (logf) bias += logf[j + 1];", "if (logf) bias += logf[j];", 2),
    ("scale_dropped", "sbuf[j] = scale * kt + bias;", "sbuf[j] = kt + bias;", 1),
    ("scale_on_bias", "sbuf[j] = scale * kt + bias;", "sbuf[j] = scale * (kt + bias);", 1),
    ("scores_scale_on_bias", "S[(size_t)i * L + j] = scale * kt + bias;", "S[(size_t)i * L + j] = scale * (kt + bias);", 1),
    ("key_operand_swapped", "for (int c = 0; c < d; ++c) kt += k[(size_t)j * d + c] * u[c];\n        sbuf",
     "for (int c = 0; c < d; ++c) kt += v[(size_t)j * d + c] * u[c];\n        sbuf", 1),
    ("no_normalise", "for (int c = 0; c < d; ++c) o[c] /= z;", "", 1),
    ("lse_no_max", "*lse = m + log(z);\n}\n\ntypedef struct {\n    const double *q", "*lse = log(z);\n}\n\ntypedef struct {\n    const double *q", 1),
    ("transport_reversed", "for (int s = hi; s >= lo; --s) apply_h", "for (int s = lo; s <= hi; ++s) apply_h", 1),
    ("causal_diag_excluded", "for (int j = 0; j <= i; ++j) {\n        double p", "for (int j = 0; j < i; ++j) {\n        double p", 1),
    ("decode_no_update", "for (int64_t j = 0; j < n; ++j) apply_h(kc + (size_t)j * d, w, beta, d);", "", 1),
    ("decode_new_key_transformed",
     "        if (logf) fc[n] = ct;\n        nt = n + 1;\n    }",
     "        if (logf) fc[n] = ct;\n        nt = n + 1;\n        apply_h(kc + (size_t)n * d, w, beta, d);\n    }", 1),
    ("decode_scale_dropped", "double p = exp(scale * s + (logf ? ct - fc[j] : 0.0) - m);",
     "double p = exp(s + (logf ? ct - fc[j] : 0.0) - m);", 1),
    ("decode_gate_sign", "double p = exp(scale * s + (logf ? ct - fc[j] : 0.0) - m);",
     "double p = exp(scale * s + (logf ? fc[j] - ct : 0.0) - m);", 1),
    ("decode_gate_no_newest", "const double ct = logf ? (n > 0 ? fc[n - 1] : 0.0) + *logf : 0.0;",
     "const double ct = logf ? (n > 0 ? fc[n - 1] : 0.0) : 0.0;", 1),
    ("decode_gate_row_index", "double p = exp(scale * s + (logf ? ct - fc[j] : 0.0) - m);",
     "double p = exp(scale * s + (logf ? ct - (j > 0 ? fc[j - 1] : 0.0) : 0.0) - m);", 1),
    ("cache_order_reversed", "for (int s = j + 1; s < L; ++s) apply_h(u, wg + (size_t)s * d, bg[s], d);",
     "for (int s = L - 1; s > j; --s) apply_h(u, wg + (size_t)s * d, bg[s], d);", 1),
    ("cache_includes_own_H", "for (int s = j + 1; s < L; ++s) apply_h(u, wg", "for (int s = j; s < L; ++s) apply_h(u, wg", 1),
    ("cache_drops_last_H", "for (int s = j + 1; s < L; ++s) apply_h(u, wg", "for (int s = j + 1; s < L - 1; ++s) apply_h(u, wg", 1),
    ("produce_taps_reversed", "acc += cwh[(size_t)c * 3 + tau] * x", "acc += cwh[(size_t)c * 3 + (2 - tau)] * x", 1),
    ("produce_centred_window", "const int src = t - 2 + tau;\n                    if (src >= 0)",
     "const int src = t - 1 + tau;\n                    if (src >= 0 && src < L)", 1),
    ("produce_no_normalise", "for (int c = 0; c < d; ++c) y[c] /= nrm;", "", 1),
    ("produce_beta_no_two", "double b = 2.0 / (1.0 + exp(-z", "double b = 1.0 / (1.0 + exp(-z", 1),
    ("produce_clip_ignored", "if (beta_clip > 0.0 && b > beta_clip) b = beta_clip;", "", 1),
    ("produce_head_index", "cwh = cw + (size_t)(g % H) * d * 3;", "cwh = cw + (size_t)(g / (G / H)) * d * 3;", 1),
    ("bwd_states_off_by_one", "apply_h(U + (size_t)j * d, w + (size_t)(j + 1) * d, beta[j + 1], d);",
     "apply_h(U + (size_t)j * d, w + (size_t)j * d, beta[j], d);", 1),
    ("bwd_dbeta_sign", "dbeta[j] -= a * b;", "dbeta[j] += a * b;", 1),
    ("bwd_dw_drop_term", "(b * lam[c] + a * uj[c])", "(b * lam[c])", 1),
    ("bwd_dw_wrong_state", "*uj = U + (size_t)j * d;", "*uj = U + (size_t)(j - 1) * d;", 1),
    ("bwd_adjoint_skips_H", "lam[c] += -beta[j] * a * wj[c] + scale", "lam[c] += scale", 1),
    ("bwd_dk_no_scale", "dk[(size_t)j * d + c] += scale * s[j] * U", "dk[(size_t)j * d + c] += s[j] * U", 1),
    ("bwd_dlse_dropped", "s[j] = P * (dp - D + gl);", "s[j] = P * (dp - D);", 1),
    ("bwd_dv_unweighted", "dv[(size_t)j * d + c] += P * doi[c];", "dv[(size_t)j * d + c] += doi[c];", 1),
    ("bwd_dlogf_index", "acc += s[t - 1];", "acc += s[t];", 1),
    ("bwd_adjoint_init_no_scale", "lam[c] = scale * s[0] * k[c];", "lam[c] = s[0] * k[c];", 1),
    ("bwd_dq_key_operand", "scale * s[j] * k[(size_t)j * d + c];", "scale * s[j] * v[(size_t)j * d + c];", 1),
]


@pytest.mark.parametrize("mid,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(mid, old, new, count, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == count, "patch for %s no longer matches the oracle source" % mid
    mutant = tmp_path / ("oracle_%s.c" % mid)
    mutant.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(mutant), str(tmp_path / ("liboracle_%s.so" % mid)))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, "mutant %s survived every pin" % mid
