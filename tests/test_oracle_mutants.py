"""The pins must be able to fail: plant plausible mistakes in a copy of the C
oracle (on the CPU, in a temporary directory), load the mutant in place of
the oracle, and require that at least one pin rejects each mutant."""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_bwd as bwd_pins
from tests import test_oracle_bwd2 as bwd2_pins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, original text, planted mistake).  Every mutant keeps all memory
# accesses in bounds.
MUTANTS = [
    ("error_sign", "u[j] = beta * (v[j] - pred);", "u[j] = beta * (v[j] + pred);"),
    ("beta_dropped", "u[j] = beta * (v[j] - pred);", "u[j] = (v[j] - pred);"),
    ("no_decay", "for (int i = 0; i < Dk * Dv; ++i) S[i] *= decay;", ";"),
    ("decay_sign", "const double decay = exp(g);", "const double decay = exp(-g);"),
    ("write_with_query", "for (int j = 0; j < Dv; ++j) S[i * Dv + j] += k[i] * u[j];\n    if (o)",
     "for (int j = 0; j < Dv; ++j) S[i * Dv + j] += q[i] * u[j];\n    if (o)"),
    ("scale_dropped", "o[j] = scale * acc;", "o[j] = acc;"),
    ("predict_with_query", "pred += S[i * Dv + j] * k[i];", "pred += S[i * Dv + j] * q[i];"),
    ("gdn2_erase_gate_dropped", "e[i] = bt[i] * kt[i];", "e[i] = kt[i];"),
    ("gdn2_write_gate_dropped", "u[j] = wt[j] * vt[j] - pred;", "u[j] = vt[j] - pred;"),
    ("gdn2_write_gate_on_error", "u[j] = wt[j] * vt[j] - pred;", "u[j] = wt[j] * (vt[j] - pred);"),
    ("gdn2_decay_uniform", "const double a = exp(la[i]);", "const double a = exp(la[0]);"),
    ("gdn2_readout_scale", "ot[j] = scale * acc;", "ot[j] = acc;"),
    ("bwd_dq_pre_edit_state", "a += St[i * Dv + j] * dot[j];", "a += spx[i * Dv + j] * dot[j];"),
    ("bwd_dk_erase_term_dropped", "dkt[i] -= bt * a;", "dkt[i] -= 0.0 * a;"),
    ("bwd_dbeta_raw_value", "db += a * (vt[j] - px[j]);", "db += a * vt[j];"),
    ("bwd_no_state_decay", "for (size_t i = 0; i < SS; ++i) D[i] *= decay;", "for (size_t i = 0; i < SS; ++i) D[i] *= 1.0;"),
    ("bwd_dg_post_edit_state", "for (size_t i = 0; i < SS; ++i) dgt += D[i] * spx[i];",
     "for (size_t i = 0; i < SS; ++i) dgt += D[i] * St[i];"),
    ("bwd_output_grad_unscaled", "D[i * Dv + j] += scale * qt[i] * dot[j];", "D[i * Dv + j] += qt[i] * dot[j];"),
    ("bwd2_dw_wrong_operand", "dwt[j] = a * vt[j];", "dwt[j] = a * wt[j];"),
    ("bwd2_de_sign", "de[i] = -a;", "de[i] = a;"),
    ("bwd2_dk_erase_term_dropped", "dkt[i] += de[i] * bt[i];", "dkt[i] += 0.0 * bt[i];"),
    ("bwd2_dla_post_edit_state", "a += D[i * Dv + j] * px[i * Dv + j];", "a += D[i * Dv + j] * St[i * Dv + j];"),
    ("bwd2_erase_with_raw_key", "D[i * Dv + j] -= ei * du[j];", "D[i * Dv + j] -= kt[i] * du[j];"),
]

PIN_FUNCS = [
    pins.test_hand_worked_gdn,
    pins.test_hand_worked_gdn2,
    pins.test_matrix_form_gdn,
    pins.test_matrix_form_gdn2,
    pins.test_beta0_pure_decay_closed_form,
    pins.test_beta1_unit_key_writes_exactly,
    pins.test_gdn2_b1_unit_key_writes_gated_value,
    pins.test_single_token_closed_form,
    pins.test_two_token_hand_expansion,
    pins.test_one_hot_keys_are_scalar_emas,
    pins.test_gdn2_one_hot_keys_are_channel_emas,
    pins.test_hand_worked_gdn2_step,
    bwd_pins.pin_backward_fd,
    bwd2_pins.pin_backward2_fd,
]


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(text.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(path), "-o", str(so), "-lm"],
                   check=True)
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, monkeypatch, name, old, new):
    so = _build_mutant(tmp_path, name, old, new)
    lib = oracle.configure(ctypes.CDLL(so))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = []
    for f in PIN_FUNCS:
        kwargs = {}
        if "gp" in inspect.signature(f).parameters:
            kwargs["gp"] = -800.0
        try:
            f(**kwargs)
        except AssertionError:
            caught.append(f.__name__)
    assert caught, f"no pin rejects mutant {name}"


# Planted mistakes in a copy of the prologue oracle (oracle/prologue.py); each
# must be rejected by a pin of tests/test_oracle_prologue.py.
PROLOGUE_SRC = os.path.join(os.path.dirname(oracle.__file__), "prologue.py")
PROLOGUE_MUTANTS = [
    ("silu_negated_argument", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    ("sigmoid_negated_argument", "return 1.0 / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(x))"),
    ("softplus_negated_argument", "return np.logaddexp(0.0, x)", "return np.logaddexp(0.0, -x)"),
    ("beta_of_minus_b", "    beta = sigmoid(b)\n", "    beta = sigmoid(-b)\n"),
    ("dt_bias_outside_softplus", "softplus(a + dt_bias[None, None, :])",
     "(softplus(a) + dt_bias[None, None, :])"),
    ("A_log_not_exponentiated", "g = -np.exp(A_log)[None, None, :]", "g = -A_log[None, None, :]"),
    ("g_positive", "g = -np.exp(A_log)[None, None, :]", "g = np.exp(A_log)[None, None, :]"),
    ("l2norm_eps_outside_root", "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
     "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)"),
    ("conv_taps_reversed", "y[:, t] += w[:, j] * full[:, t + j]", "y[:, t] += w[:, CONV - 1 - j] * full[:, t + j]"),
    ("v_without_silu", "v = silu(yv).reshape(B, T, H, Dv)", "v = yv.reshape(B, T, H, Dv)"),
    ("q_not_normalised", "q = l2norm(silu(yq).reshape(B, T, H, Dk))", "q = silu(yq).reshape(B, T, H, Dk)"),
    ("rmsnorm_sum_not_mean", "np.mean(o * o, axis=-1, keepdims=True)", "np.sum(o * o, axis=-1, keepdims=True)"),
    ("rmsnorm_sigmoid_gate", "+ eps) * w * silu(z)\n", "+ eps) * w * sigmoid(z)\n"),
]


@pytest.mark.parametrize("name,old,new", PROLOGUE_MUTANTS, ids=[m[0] for m in PROLOGUE_MUTANTS])
def test_prologue_pins_reject_mutant(tmp_path, name, old, new):
    import importlib.util

    from tests import test_oracle_prologue as ppins
    text = open(PROLOGUE_SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"prologue_{name}.py"
    path.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"prologue_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for f in ppins.PINS:
        try:
            f(mod)
        except AssertionError:
            caught.append(f.__name__)
    assert caught, f"no prologue pin rejects mutant {name}"
