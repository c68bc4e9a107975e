"""Plant plausible mistakes in copies of the C oracle; every one must trip a pin.

Each mutant is a textual edit of oracle/kda_oracle.c compiled into a temporary
directory (the real oracle is never touched).  A mutant that passes every pin
would mean the pins cannot tell that mistake from the correct definition.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    # update order: predict from the undecayed state (decay moved after the error)
    "predict_before_decay": [
        ("""            for (int c = 0; c < DK; ++c) {           /* decay */
                const double a = exp(gt[c]);
                for (int j = 0; j < DV; ++j) S[c * DV + j] *= a;
            }
            for (int j = 0; j < DV; ++j) {           /* predict, error */
                double pred = 0.0;
                for (int c = 0; c < DK; ++c) pred += S[c * DV + j] * kt[c];
                e[j] = delta_rule ? vt[j] - pred : vt[j];
            }""",
         """            for (int j = 0; j < DV; ++j) {           /* predict, error */
                double pred = 0.0;
                for (int c = 0; c < DK; ++c) pred += S[c * DV + j] * kt[c];
                e[j] = delta_rule ? vt[j] - pred : vt[j];
            }
            for (int c = 0; c < DK; ++c) {           /* decay */
                const double a = exp(gt[c]);
                for (int j = 0; j < DV; ++j) S[c * DV + j] *= a;
            }""")],
    "error_sign": [("e[j] = delta_rule ? vt[j] - pred : vt[j];",
                    "e[j] = delta_rule ? pred - vt[j] : vt[j];")],
    "beta_dropped": [("S[c * DV + j] += bt * kt[c] * e[j];", "S[c * DV + j] += kt[c] * e[j];")],
    "decay_sign": [("const double a = exp(gt[c]);", "const double a = exp(-gt[c]);")],
    "decay_on_columns": [("const double a = exp(gt[c]);\n                for (int j = 0; j < DV; ++j) S[c * DV + j] *= a;",
                          "(void)gt;\n                for (int j = 0; j < DV; ++j) S[c * DV + j] *= exp(gt[j % DK]);")],
    "prediction_uses_q": [("pred += S[c * DV + j] * kt[c];", "pred += S[c * DV + j] * qt[c];")],
    "readout_uses_k": [("acc += S[c * DV + j] * qt[c];", "acc += S[c * DV + j] * kt[c];")],
    "readout_transposed": [("acc += S[c * DV + j] * qt[c];", "acc += S[(j % DK) * DV + (c % DV)] * qt[c];")],
    "scale_dropped": [("ot[j] = scale * acc;", "ot[j] = acc;")],
    "h0_ignored": [("S[i] = h0 ? h0[sbase + i] : 0.0;", "S[i] = 0.0;")],
    "conv_taps_reversed": [("acc += w[c * W + i] * xe[j + i];", "acc += w[c * W + (W - 1 - i)] * xe[j + i];")],
    "conv_off_by_one": [("acc += w[c * W + i] * xe[j + i];", "acc += w[c * W + i] * xe[j + i + (i == W - 1 ? 0 : 1)];")],
    "conv_history_ignored": [("xe[i] = state_in ? state_in[((int64_t)n * H + i) * C + c] : 0.0;", "xe[i] = 0.0;")],
    "conv_state_out_first": [("state_out[((int64_t)n * H + i) * C + c] = xe[L + i];",
                              "state_out[((int64_t)n * H + i) * C + c] = xe[i + 1];")],
    "silu_wrong": [("if (silu) acc = acc / (1.0 + exp(-acc));", "if (silu) acc = acc / (1.0 + exp(acc));")],
    "l2_no_sqrt": [("const double inv = 1.0 / sqrt(ss + eps);", "const double inv = 1.0 / (ss + eps);")],
    "bias_dropped": [("double acc = bias ? bias[c] : 0.0;", "double acc = 0.0;")],
    "bf16_truncates": [("x[i] = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "x[i] = ldexp(trunc(ldexp(m, 8)), e - 8);")],
    "bf16_round_half_up": [("x[i] = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "x[i] = ldexp(round(ldexp(m, 8)), e - 8);")],
    "gate_alog_not_exponentiated": [("const double a = exp(a_log ? a_log[h] : 0.0);",
                                     "const double a = a_log ? a_log[h] : 1.0;")],
    "gate_bias_multiplied": [("(z[i] + (dt_bias ? dt_bias[(int64_t)h * D + c] : 0.0))",
                              "(z[i] * (dt_bias ? dt_bias[(int64_t)h * D + c] : 1.0))")],
    "gate_bias_per_head": [("dt_bias[(int64_t)h * D + c]", "dt_bias[h]")],
    "gate_sigmoid_sign": [("g[i] = lower_bound / (1.0 + exp(-y));", "g[i] = lower_bound / (1.0 + exp(y));")],
    "gate_bound_dropped": [("g[i] = lower_bound / (1.0 + exp(-y));", "g[i] = -1.0 / (1.0 + exp(-y));")],
    "norm_no_mean": [("const double inv = 1.0 / sqrt(ss / D + eps);", "const double inv = 1.0 / sqrt(ss + eps);")],
    "norm_no_sqrt": [("const double inv = 1.0 / sqrt(ss / D + eps);", "const double inv = 1.0 / (ss / D + eps);")],
    "norm_eps_outside": [("const double inv = 1.0 / sqrt(ss / D + eps);", "const double inv = 1.0 / (sqrt(ss / D) + eps);")],
    "norm_over_all_heads": [("for (int c = 0; c < D; ++c) ss += orow[c] * orow[c];",
                             "for (int c = 0; c < D; ++c) ss += o[(r / H) * H * D + c] * o[(r / H) * H * D + c];")],
    "out_gate_not_sigmoid": [("y[r * D + c] = orow[c] * inv * (w ? w[c] : 1.0) / (1.0 + exp(-grow[c]));",
                              "y[r * D + c] = orow[c] * inv * (w ? w[c] : 1.0) * grow[c];")],
    "out_weight_dropped": [("y[r * D + c] = orow[c] * inv * (w ? w[c] : 1.0) / (1.0 + exp(-grow[c]));",
                            "y[r * D + c] = orow[c] * inv / (1.0 + exp(-grow[c]));")],
}


def _build_mutant(tmp_path, name, edits):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        assert src.count(old) == 1, "mutation %s does not match the oracle source" % name
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), name + ".c")
    with open(path, "w") as f:
        f.write(src)
    return oracle.OracleLib(oracle.compile_library(path, path[:-2] + ".so"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    orc = _build_mutant(tmp_path, name, MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name
