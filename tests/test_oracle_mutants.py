"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (CPU only; gcc builds each mutant in a temp dir).

A pin set that a dropped term, a flipped sign, a wrong index or a transposed
operand can slip past would not be worth trusting; this test is the evidence
that ours cannot."""
import os

import pytest

import oracle
from oracle.build import HERE, build
from oracle_pins import failing_pins

SRC = os.path.join(HERE, "kda_oracle.c")

# (name, exact text in kda_oracle.c, replacement)
MUTANTS = [
    ("decay_dropped", "S[c * dv + j] *= alpha[c];", "S[c * dv + j] *= 1.0 + 0.0 * alpha[c];"),
    ("decay_on_value_axis", "S[c * dv + j] *= alpha[c];", "S[c * dv + j] *= alpha[j % dk];"),
    ("erase_sign_flipped", "((double)vv[j] - erase[j])", "((double)vv[j] + erase[j])"),
    ("beta_dropped", "kc * beta * ((double)vv[j] - erase[j])", "kc * ((double)vv[j] - erase[j])"),
    ("erase_without_key", "acc += (double)kv[c] * S[c * dv + j];",
     "acc += (double)qv[c] * S[c * dv + j];"),
    ("output_reads_key", "acc += (double)qv[c] * S[c * dv + j];",
     "acc += (double)kv[c] * S[c * dv + j];"),
    ("sigmoid_sign", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("exp_A_dropped", "logistic(exp(a_h) * z)", "logistic(z)"),
    ("A_not_exponentiated", "logistic(exp(a_h) * z)", "logistic(a_h * z)"),
    ("g_min_sign", "return g_min * logistic", "return -g_min * logistic"),
    ("chunk_restart_off_by_one", "if (t % C == 0)", "if (t % C == 1)"),
    ("wrong_head_gate", "beta[row], A[h], g_min", "beta[row], A[0], g_min"),
    ("state_not_carried", "S[e] = S0 ? (double)S0[sbase + e] : 0.0;", "S[e] = 0.0;"),
    ("decode_wrong_beta", "beta[u], A[h]", "beta[h], A[h]"),
    ("write_uses_query", "double kc = kv[c];", "double kc = qv[c];"),
    # the reverse sweep
    ("bwd_dq_from_previous_state", "acc += Scur[c * DV + j] * (double)dov[j];",
     "acc += Sprev[c * DV + j] * (double)dov[j];"),
    ("bwd_dp_sign", "const double dp = -bt * de[j];", "const double dp = bt * de[j];"),
    ("bwd_state_grad_not_decayed", "dS[c * DV + j] = a[c] * dSp[c * DV + j];",
     "dS[c * DV + j] = dSp[c * DV + j];"),
    ("bwd_dA_without_x", "dA_unit[u] += dx * xs[c];", "dA_unit[u] += dx;"),
    ("bwd_dz_without_expA", "dz[row * DK + c] = dx * eA;", "dz[row * DK + c] = dx;"),
    ("bwd_dbeta_uses_e", "db += acc * uu[j];", "db += acc * bt * uu[j];"),
    ("bwd_sigmoid_derivative", "g_min * sg[c] * (1.0 - sg[c])", "g_min * sg[c]"),
    ("bwd_da_uses_decayed_state", "dac += dSp[c * DV + j] * Sprev[c * DV + j];",
     "dac += dSp[c * DV + j] * a[c] * Sprev[c * DV + j];"),
    ("bwd_dST_ignored", "dS[e] = dST ? (double)dST[sbase + e] : 0.0;", "dS[e] = 0.0;"),
    ("bwd_dk_write_term_dropped", "dkc += dS[c * DV + j] * bt * uu[j] + sprime * dp;",
     "dkc += sprime * dp;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / f"kda_oracle_{name}.c"
    src.write_text(text.replace(old, new, 1))
    lib = build(src=str(src), out=str(tmp_path / f"lib_{name}.so"))
    bad = failing_pins(oracle.Oracle(lib))
    assert bad, f"mutant {name} passed every pin"
