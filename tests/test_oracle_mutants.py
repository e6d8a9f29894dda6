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
    "no_decay": ("S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];",
                 "S[p * N + n] = S[p * N + n] + dt * xt[p] * Bt[n];"),
    "no_dt_input_scale": ("S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];",
                          "S[p * N + n] = a * S[p * N + n] + xt[p] * Bt[n];"),
    "no_skip_D": ("yt[p] = acc + d_skip * xt[p];", "yt[p] = acc;"),
    "softplus_is_exp": ("return log1p(exp(z));", "return exp(z);"),
    "decay_sign": ("const double a = exp(dt * A[h]);\n            const double *xt",
                   "const double a = exp(-dt * A[h]);\n            const double *xt"),
    "B_C_swapped": ("const double *Bt = B + (tok * G + g) * N;\n            const double *Ct = C + (tok * G + g) * N;",
                    "const double *Bt = C + (tok * G + g) * N;\n            const double *Ct = B + (tok * G + g) * N;"),
    "group_map_modulo": ("const int g = h / heads_per_group;\n        const size_t row_off",
                         "const int g = h % G;\n        const size_t row_off"),
    "output_before_update": ("S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];\n                    acc += S[p * N + n] * Ct[n];",
                             "acc += S[p * N + n] * Ct[n];\n                    S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];"),
    "initial_state_ignored": ("if (initial_state)\n            memcpy(S,", "if (0)\n            memcpy(S,"),
    "dt_bias_ignored": ("const double bias = dt_bias ? dt_bias[h] : 0.0;", "const double bias = 0.0;"),
    "conv_taps_reversed": ("u += w[(size_t)c * K + k] * v;", "u += w[(size_t)c * K + (K - 1 - k)] * v;"),
    "conv_no_silu": ("os[(size_t)t * CH + c] = silu(u);", "os[(size_t)t * CH + c] = u;"),
    "conv_crosses_sequences": ("if (tau >= start[s]) v = xs[(size_t)tau * CH + c];\n                    else if (st) v = st[(size_t)(tau - start[s] + K - 1) * CH + c];\n                    else v = 0.0;\n                    u +=",
                               "if (tau >= 0) v = xs[(size_t)tau * CH + c];\n                    else if (st) v = st[(size_t)(tau - start[s] + K - 1) * CH + c];\n                    else v = 0.0;\n                    u +="),
    "decode_no_shift": ("cs[(size_t)r * CH + c] = cs[(size_t)(r + 1) * CH + c];", "(void)0;"),
    "decode_state_transposed": ("S[p * N + n] = a * S[p * N + n] + dt * xv[h * P + p] * Bv[g * N + n];",
                                "S[p * N + n] = a * S[p * N + n] + dt * xv[h * P + (n % P)] * Bv[g * N + (p % N)];"),
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
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
