"""The oracle pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and checks that at least one pin fails.
The real oracle is never modified.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from oracle.build import SRC, build
from tests import oracle_pins

MUTANTS = {
    "decay_after_add": ("lam * S[(int64_t)a * dv + c] + kt[a] * vt[c]",
                        "lam * (S[(int64_t)a * dv + c] + kt[a] * vt[c])"),
    "no_decay": ("lam * S[(int64_t)a * dv + c] + kt[a] * vt[c]",
                 "S[(int64_t)a * dv + c] + kt[a] * vt[c]"),
    "inverse_decay": ("exp((double)g_gamma[h])", "exp(-(double)g_gamma[h])"),
    "q_for_k": ("out_row[c] += qt[a] * S", "out_row[c] += kt[a] * S"),
    "k_for_q": ("lam * S[(int64_t)a * dv + c] + kt[a] * vt[c]",
                "lam * S[(int64_t)a * dv + c] + qt[a] * vt[c]"),
    "kv_head_modulo": ("const int kvh = h / group;", "const int kvh = h % num_kv_heads;"),
    "no_scale": ("= scale * out_row[c]", "= out_row[c]"),
    "scale_twice": ("= scale * out_row[c]", "= scale * scale * out_row[c]"),
    "ignore_reverse": ("reverse ? row0 + len - 1 - step : row0 + step", "row0 + step"),
    "ignore_initial_state": ("initial_state ? (double)initial_state[st_base + i] : 0.0", "0.0"),
    "varlen_from_row0": ("row0 = cu_seqlens[n];", "row0 = 0;"),
    "gamma_plus": ("(1.0 - (double)layer_idx / (double)num_layers)",
                   "(1.0 + (double)layer_idx / (double)num_layers)"),
    "gamma_head_offset": ("volatile float hv = (float)h;", "volatile float hv = (float)(h + 1);"),
    "gamma_fp64_product": ("out[h] = coef32 * hv;", "out[h] = (float)(coef * (double)hv);"),
    "bf16_low_half": ("<< 16;", "<< 0;"),
    # backward
    "bwd_final_grad_decayed": ("step == 0 ? 1.0 : lam", "lam"),
    "bwd_D_unscaled": ("+ scale * qt[a] * dot[c]", "+ qt[a] * dot[c]"),
    "bwd_dq_unscaled": ("dq[(row * num_heads + h) * dk + a] = scale * acc;",
                        "dq[(row * num_heads + h) * dk + a] = acc;"),
    "bwd_dk_uses_dO": ("acc += D[(int64_t)a * dv + c] * vt[c];", "acc += D[(int64_t)a * dv + c] * dot[c];"),
    "bwd_dv_uses_q": ("acc += kt[a] * D[(int64_t)a * dv + c];", "acc += qt[a] * D[(int64_t)a * dv + c];"),
    "bwd_dinit_undecayed": ("(len > 0 ? lam * D[i]", "(len > 0 ? D[i]"),
    "bwd_sweep2_forward_order": ("const int64_t row = reverse ? row0 + step : row0 + len - 1 - step;",
                                 "const int64_t row = reverse ? row0 + len - 1 - step : row0 + step;"),
    "bwd_gqa_overwrites": ("dk_out[ko + a] += acc;", "dk_out[ko + a] = acc;"),
    # gated forward
    "gated_gv_on_key_axis": ("lb[c] = gv ? in_value(gv, in_dtype, gvo + c) : 0.0;",
                             "lb[c] = gv ? in_value(gv, in_dtype, go + c) : 0.0;"),
    "gated_gk_ignored": ("+ (gk ? in_value(gk, in_dtype, go + a) : 0.0);", ";"),
    "gated_value_decay_dropped": ("exp(la[a] + lb[c]) * S", "exp(la[a]) * S"),
    "gated_decay_after_add": ("exp(la[a] + lb[c]) * S[(int64_t)a * dv + c] + kt[a] * vt[c];",
                              "exp(la[a] + lb[c]) * (S[(int64_t)a * dv + c] + kt[a] * vt[c]);"),
    "gated_g_gamma_ignored": ("const double base = g_gamma ? (double)g_gamma[h] : 0.0;",
                              "const double base = 0.0;"),
    "bwd_dq_state_before_update": ("S[(int64_t)a * dv + c] = lam * S[(int64_t)a * dv + c] + kt[a] * vt[c];\n"
                                   "                for (int a = 0; a < dk; ++a) {",
                                   "(void)0;\n                for (int a = 0; a < dk; ++a) {"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    # Sites shared by the forward and backward functions are mutated at their first
    # occurrence, which is in the forward function (it comes first in the file).
    assert source.count(old) >= 1, f"mutation site for {name} not found"
    src = os.path.join(tmp_path, "mutant.c")
    with open(src, "w") as f:
        f.write(source.replace(old, new, 1))
    lib = build(src, os.path.join(tmp_path, "libmutant.so"))
    orc = oracle.load(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {name}"
