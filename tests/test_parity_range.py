"""Operand range of the bf16-input paths (GPU, through the C ABI).

The bf16 paths round some intermediate values to fp16 for the MFMA: on the
Gated DeltaNet path the chunk residuals R = beta (v - gamma K S), the new
values, T - I and P; on the Gated DeltaNet-2 path also the decayed keys and
queries and the state's hi + lo parts.  include/gdn.h states the range this
allows; these tests run inputs at its upper end and well inside its lower end
and require parity with the oracle there (the parity metric is relative, and
the map is linear in (v, h0), so only range effects can move it)."""
import numpy as np
import pytest

import gated_delta_rule_34_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import TOL, gdn_dev_args, gdn_ref_args, host, rel_err, dev

pytestmark = pytest.mark.gpu

FP16_BOUND = 32768.0   # the stated bound: half of fp16's largest finite value


def _bf16(a):
    """fp64 values rounded to bf16 (RNE), as bits and as fp64."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float64).numpy()


def _gdn_state_bound(x):
    """max over (b, h, c) of max_t |v| + sqrt(|h0[:, c]|^2 + sum_t beta_t v_{t,c}^2):
    the bound on |R| and |new values| that unit-norm keys, beta in [0, 1] and
    g <= 0 give (the state column norm never grows by more than beta v^2 in
    square per token)."""
    v, beta = x["v_f64"], x["beta_f64"]
    h0 = x["h0_f64"]
    acc = np.sum(beta[..., None] * v * v, axis=1)                    # [B, H, Dv]
    if h0 is not None:
        acc = acc + np.sum(h0 * h0, axis=2)
    return float((np.abs(v).max(axis=1) + np.sqrt(acc)).max())


def _scale_gdn_values(x, s):
    vb, vf = _bf16(x["v_f64"] * s)
    x["v"], x["v_f64"] = vb, vf
    if x["h0"] is not None:
        x["h0"] = (x["h0_f64"] * s).astype(np.float32)
        x["h0_f64"] = x["h0"].astype(np.float64)


def test_gdn_bf16_at_upper_range_bound():
    """No decay (g = 0, so nothing is forgotten) and values scaled until the
    stated bound is just under 32,768: finite output, parity holds."""
    x = gi.gdn_inputs(1, 256, 2, 128, 128, seed=91, dtype="bf16", h0=True)
    x["g"][:] = 0.0
    x["g_f64"][:] = 0.0
    s = 0.97 * FP16_BOUND / _gdn_state_bound(x)
    _scale_gdn_values(x, s)
    assert 0.9 * FP16_BOUND < _gdn_state_bound(x) <= FP16_BOUND
    o, S = gdn.gdn_chunk_fwd(*gdn_dev_args(x), scale=x["scale"])
    o, S = host(o), host(S)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    ro, rS = oracle.gdn_fwd(*gdn_ref_args(x), scale=x["scale"])
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(S, rS) <= TOL["bf16"]


@pytest.mark.parametrize("s", [2.0 ** -6, 2.0 ** -3])
def test_gdn_bf16_small_values(s):
    """Values and initial state scaled down (entries around 2^-6 .. 2^-3 of the
    unit-variance case), still inside fp16's normal range: parity holds."""
    x = gi.gdn_inputs(1, 256, 2, 128, 128, seed=92, dtype="bf16", h0=True, a_range=(0.01, 0.5))
    _scale_gdn_values(x, s)
    o, S = gdn.gdn_chunk_fwd(*gdn_dev_args(x), scale=x["scale"])
    ro, rS = oracle.gdn_fwd(*gdn_ref_args(x), scale=x["scale"])
    assert rel_err(host(o), ro) <= TOL["bf16"] and rel_err(host(S), rS) <= TOL["bf16"]


NAMES2 = ("q", "k", "v", "log_alpha", "b", "w", "h0")


@pytest.mark.parametrize("s", [2.0 ** -6, 256.0])
def test_gdn2_bf16_scaled_values(s):
    """GDN-2 with values and initial state scaled by 2^-6 and by 256 (state
    entries stay far below 32,768 under the configured decay): parity holds
    and everything is finite."""
    x = gi.gdn2_inputs(1, 256, 2, 128, 128, seed=93, dtype="bf16", h0=True)
    vb, vf = _bf16(x["v_f64"] * s)
    x["v"], x["v_f64"] = vb, vf
    x["h0"] = (x["h0_f64"] * s).astype(np.float32)
    x["h0_f64"] = x["h0"].astype(np.float64)
    o, S = gdn.gdn2_chunk_fwd(*[dev(x[n]) for n in NAMES2], scale=x["scale"])
    o, S = host(o), host(S)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    ro, rS = oracle.gdn2_fwd(*[x[n + "_f64"] for n in NAMES2], scale=x["scale"])
    assert np.abs(rS).max() < FP16_BOUND
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(S, rS) <= TOL["bf16"]
