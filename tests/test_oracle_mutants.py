"""Plant plausible mistakes in a copy of the oracle and check that the pins see them.

Each mutant is one textual edit of ``oracle/oracle.c`` (a dropped term, a wrong
sign, a transposed operand, an off-by-one in the index rule, ...).  The edited
copy is compiled into a temporary library on the CPU and the whole pin suite is
run against it: at least one pin must fail for every mutant.  The real oracle is
never modified.
"""

import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "softcap_slope_not_squared": ("return 1.0 / (ch * ch);", "return 1.0 / ch;"),
    "softcap_outer_cap_dropped": ("return c * tanh(x / c);", "return tanh(x / c);"),
    "lse_without_max": ("double lse = m + log(z);", "double lse = log(z);"),
    "exp_not_shifted": ("z += exp(y[v] - m);", "z += exp(y[v]);"),
    "target_zero_ignored": ("return t >= 0 && t < V;", "return t > 0 && t < V;"),
    "logp_grad_sign": ("gr[v] = (h[v] - b.p[v] * G) * b.s[v];",
                       "gr[v] = (h[v] + b.p[v] * G) * b.s[v];"),
    "logp_grad_slope_dropped": ("gr[v] = (h[v] - b.p[v] * G) * b.s[v];",
                                "gr[v] = (h[v] - b.p[v] * G);"),
    "topk_duplicates_overwrite": ("h[tj] += g[i * k + j];", "h[tj] = g[i * k + j];"),
    "topk_G_counts_ignored": ("                if (target_valid(tj, V)) {\n"
                              "                    G += g[i * k + j];",
                              "                G += g[i * k + j];\n"
                              "                if (target_valid(tj, V)) {"),
    "entropy_sign": ("H -= b->p[v] * b->logp[v];", "H += b->p[v] * b->logp[v];"),
    "entropy_grad_H_sign": ("(-b.p[v] * (b.logp[v] + H))", "(-b.p[v] * (b.logp[v] - H))"),
    "entropy_grad_H_dropped": ("(-b.p[v] * (b.logp[v] + H))", "(-b.p[v] * (b.logp[v]))"),
    "kl_operands_transposed": ("D += A->p[v] * (A->logp[v] - B->logp[v]);",
                               "D += A->p[v] * (B->logp[v] - A->logp[v]);"),
    "kl_weights_from_B": ("D += A->p[v] * (A->logp[v] - B->logp[v]);",
                          "D += B->p[v] * (A->logp[v] - B->logp[v]);"),
    "kl_mismatch_rule_dropped": (
        "if (A->logp[v] > -INFINITY && B->logp[v] == -INFINITY) return INFINITY;", ";"),
    "kl_direction_ignored": ("dir == ORC_KL_REVERSE ? row_kl(&P, &R, V) : row_kl(&R, &P, V)",
                             "row_kl(&P, &R, V)"),
    "reverse_kl_grad_D_dropped": ("((P.logp[v] - R.logp[v]) - D)", "((P.logp[v] - R.logp[v]))"),
    "reverse_kl_mismatch_nan_off_support": (
        "if (P.logp[v] == -INFINITY)\n                    gr[v] = 0.0;\n"
        "                else if (D == INFINITY)\n                    gr[v] = NAN;",
        "if (D == INFINITY)\n                    gr[v] = NAN;\n"
        "                else if (P.logp[v] == -INFINITY)\n                    gr[v] = 0.0;"),
    "forward_kl_grad_sign": ("(P.p[v] - R.p[v])", "(R.p[v] - P.p[v])"),
    "forward_kl_grad_slope_dropped": ("g[i] * (P.p[v] - R.p[v]) * P.s[v];",
                                      "g[i] * (P.p[v] - R.p[v]);"),
    "kl_ref_cap_uses_policy_cap": ("row_prologue(ref + i * V, V, cap_ref, R.y, R.s);\n"
                                   "        int ep = row_log_softmax(P.y, V, P.logp, P.p);\n"
                                   "        int er = row_log_softmax(R.y, V, R.logp, R.p);\n"
                                   "        if (ep || er)\n            out[i] = NAN;",
                                   "row_prologue(ref + i * V, V, cap_pol, R.y, R.s);\n"
                                   "        int ep = row_log_softmax(P.y, V, P.logp, P.p);\n"
                                   "        int er = row_log_softmax(R.y, V, R.logp, R.p);\n"
                                   "        if (ep || er)\n            out[i] = NAN;"),
    "ref_grad_reverse_sign": ("g[i] * (R.p[v] - P.p[v]) * R.s[v]",
                              "g[i] * (P.p[v] - R.p[v]) * R.s[v]"),
    "ref_grad_reverse_slope_of_policy": ("g[i] * (R.p[v] - P.p[v]) * R.s[v]",
                                         "g[i] * (R.p[v] - P.p[v]) * P.s[v]"),
    "ref_grad_forward_D_dropped": ("((R.logp[v] - P.logp[v]) - D)", "((R.logp[v] - P.logp[v]))"),
    "ref_grad_forward_weights_from_policy": ("g[i] * R.p[v] * ((R.logp",
                                             "g[i] * P.p[v] * ((R.logp"),
    "ref_grad_forward_uses_reverse_D": ("double D = row_kl(&R, &P, V);",
                                        "double D = row_kl(&P, &R, V);"),
    "ref_grad_forward_mismatch_nan_dropped": (
        "else if (D == INFINITY)\n                    gr[v] = NAN;\n"
        "                else\n                    gr[v] = g[i] * R.p[v]",
        "else\n                    gr[v] = g[i] * R.p[v]"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    path = tmp_path / "oracle_mut.c"
    path.write_text(source.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(path),
                    "-o", lib, "-lm"], check=True)
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin notices the mutant {name}"
