"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is an edited copy of oracle/ssd_oracle.c compiled to a temporary
library; the real oracle source is never changed.  Every mutant must fail at
least one pin, which shows that the pins would catch that kind of mistake
(dropped term, wrong sign, wrong index, transposed operand, wrong order).
"""
import os
import tempfile

import pytest

import oracle
from oracle.build import SRC, build
from tests.oracle_pins import ALL_PINS

MUTANTS = {
    "linear_w_transposed": ("acc += x[(size_t)m * K + k] * w[(size_t)n * K + k];",
                            "acc += x[(size_t)m * K + k] * w[(size_t)k * N + n];"),
    "linear_drops_last_k": ("for (int k = 0; k < K; ++k) acc += x[(size_t)m * K + k]",
                            "for (int k = 0; k < K - 1; ++k) acc += x[(size_t)m * K + k]"),
    "linear_float_accumulate": ("double acc = 0.0;\n            for (int k = 0; k < K; ++k) acc += x",
                                "float acc = 0.0f;\n            for (int k = 0; k < K; ++k) acc += x"),
    "no_decay": ("S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];\n                    acc += S[p * N + n] * Ct[n];",
                 "S[p * N + n] = S[p * N + n] + dt * xt[p] * Bt[n];\n                    acc += S[p * N + n] * Ct[n];"),
    "no_dt_input_scale": ("S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];\n                    acc += S[p * N + n] * Ct[n];",
                          "S[p * N + n] = a * S[p * N + n] + xt[p] * Bt[n];\n                    acc += S[p * N + n] * Ct[n];"),
    "no_skip_D": ("yt[p] = acc + d_skip * xt[p];", "yt[p] = acc;"),
    "softplus_is_exp": ("return log1p(exp(z));", "return exp(z);"),
    "softplus_large_drops_z": ("if (z > 30.0) return z + log1p(exp(-z));",
                               "if (z > 30.0) return log1p(exp(-z));"),
    "decay_sign": ("const double a = exp(dt * A[h]);\n            const double *xt = x + (tok * H + h) * P;",
                   "const double a = exp(-dt * A[h]);\n            const double *xt = x + (tok * H + h) * P;"),
    "B_C_swapped": ("const double *Bt = B + (tok * G + g) * N;\n            const double *Ct = C + (tok * G + g) * N;",
                    "const double *Bt = C + (tok * G + g) * N;\n            const double *Ct = B + (tok * G + g) * N;"),
    "group_map_modulo": ("const int g = h / heads_per_group;\n        const size_t row_off",
                         "const int g = h % G;\n        const size_t row_off"),
    "output_before_update": ("S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];\n                    acc += S[p * N + n] * Ct[n];",
                             "acc += S[p * N + n] * Ct[n];\n                    S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];"),
    "initial_state_ignored": ("if (initial_state)\n            memcpy(S,", "if (0)\n            memcpy(S,"),
    "dt_bias_ignored": ("const double bias = dt_bias ? dt_bias[h] : 0.0;\n        const double d_skip",
                        "const double bias = 0.0;\n        const double d_skip"),
    "conv_taps_reversed": ("u += w[(size_t)c * K + k] * v;", "u += w[(size_t)c * K + (K - 1 - k)] * v;"),
    "conv_no_silu": ("os[(size_t)t * CH + c] = silu(u);", "os[(size_t)t * CH + c] = u;"),
    "conv_crosses_sequences": ("if (tau >= start[s]) v = xs[(size_t)tau * CH + c];\n                    else if (st) v = st[(size_t)(tau - start[s] + K - 1) * CH + c];\n                    else v = 0.0;\n                    u +=",
                               "if (tau >= 0) v = xs[(size_t)tau * CH + c];\n                    else if (st) v = st[(size_t)(tau - start[s] + K - 1) * CH + c];\n                    else v = 0.0;\n                    u +="),
    "decode_no_shift": ("cs[(size_t)r * CH + c] = cs[(size_t)(r + 1) * CH + c];", "(void)0;"),
    "decode_state_transposed": ("S[p * N + n] = a * S[p * N + n] + dt * xv[h * P + p] * Bv[g * N + n];",
                                "S[p * N + n] = a * S[p * N + n] + dt * xv[h * P + (n % P)] * Bv[g * N + (p % N)];"),
    "norm_divides_by_width": ("const double rms = sqrt(ss / group_size + eps);",
                              "const double rms = sqrt(ss / CH + eps);"),
    "norm_no_sqrt": ("const double rms = sqrt(ss / group_size + eps);",
                     "const double rms = ss / group_size + eps;"),
    "norm_eps_outside_sqrt": ("const double rms = sqrt(ss / group_size + eps);",
                              "const double rms = sqrt(ss / group_size) + eps;"),
    "norm_weight_group_local": ("double o = v / rms * w[(size_t)gi * group_size + c];",
                                "double o = v / rms * w[c];"),
    "norm_gate_ignored_in_rms": ("if (z && !norm_before_gate) v *= silu(z[base + c]);\n                ss += v * v;",
                                 "ss += v * v;"),
    "norm_gate_sigmoid_only": ("if (z && norm_before_gate) o *= silu(z[base + c]);",
                               "if (z && norm_before_gate) o *= silu(z[base + c]) / z[base + c];"),
    "mimo_prev_term_not_decayed": ("(1.0 - l) * dt * a * prev;", "(1.0 - l) * dt * prev;"),
    "mimo_lambda_swapped": ("a * S[p * N + n] + l * dt * cur + (1.0 - l) * dt * a * prev;",
                            "a * S[p * N + n] + (1.0 - l) * dt * cur + l * dt * a * prev;"),
    "mimo_prev_not_replaced": ("memcpy(prev_x, x, sizeof(double) * (size_t)batch * H * P * R);", "(void)0;"),
    "mimo_rank_truncated": ("for (int r = 0; r < R; ++r) {\n                        cur +=",
                            "for (int r = 0; r < 1; ++r) {\n                        cur +="),
    "mimo_output_column_zero": ("acc += S[p * N + n] * Cm[n * R + r];", "acc += S[p * N + n] * Cm[n * R];"),
    "bwd_no_decay_term": ("const double ddt = xgb + A[h] * a * gs;", "const double ddt = xgb;"),
    "bwd_no_sigmoid": ("const double dz = ddt / (1.0 + exp(-z));", "const double dz = ddt;"),
    "bwd_decay_uses_new_state": ("gs += Gt[p * N + n] * Sp[p * N + n];", "gs += Gt[p * N + n] * St[p * N + n];"),
    "bwd_dB_without_dt": ("hBt[n] = dt * s;", "hBt[n] = s;"),
    "bwd_adjoint_not_decayed": ("for (size_t e = 0; e < PN; ++e) Gt[e] *= a;", "(void)0;"),
    "bwd_dC_from_adjoint": ("for (int p = 0; p < P; ++p) s += St[p * N + n] * dyt[p];\n                    hCt[n] = s;",
                            "for (int p = 0; p < P; ++p) s += Gt[p * N + n] * dyt[p];\n                    hCt[n] = s;"),
    "decode_no_D": ("y[((size_t)b * H + h) * P + p] = acc + (D ? D[h] : 0.0) * xv[h * P + p];",
                    "y[((size_t)b * H + h) * P + p] = acc;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle._load(build(str(mpath), str(tmp_path / "libmutant.so"), extra=("-Wno-unused",)))
    # the pins of the mutant's own part first; the first pin that fails is enough
    for pin in sorted(ALL_PINS, key=lambda f: not _related(name, f.__name__)):
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            return
    pytest.fail(f"mutant {name} passed every pin")


_PARTS = (("conv", ("conv",)), ("norm", ("norm",)), ("mimo", ("mimo", "trapezoid")),
          ("trapezoid", ("trapezoid", "mimo")), ("bwd", ("backward",)), ("decode", ("decode",)),
          ("softplus", ("softplus", "dt_zero")), ("linear", ("linear",)))


def _related(mutant, pin):
    for key, pins in _PARTS:
        if key in mutant:
            return any(k in pin for k in pins)
    return not any(k in pin for _, ks in _PARTS for k in ks)  # scan mutants: the scan pins
