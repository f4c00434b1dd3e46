"""GPU parity of the prologue (short convolution, SiLU, L2 norm, gates) and of
the gated RMSNorm epilogue, through the C ABI, against the fp64 definitions in
oracle/prologue.py.

Tolerances.  q, k, v and y leave the kernels in bf16: the kernel computes in
fp32 (relative error ~1e-6) and rounds once to nearest, which moves a value
by at most half a bf16 ulp; bf16 carries 8 significant bits, so that is at
most 2^-8 |x|.  The bar 2^-7 |ref| + 1e-6 is that bound with a factor-2
margin for the fp32 arithmetic before the rounding (the 1e-6 absolute term
covers sums that cancel to near zero).  g and beta
stay fp32: a few ulp of exp / log1p / division, bar 1e-5 relative.  The new
convolution state is a copy of inputs: bit-exact."""
import numpy as np
import pytest

import gated_delta_rule_34_amd as gdn
import gdn_inputs as gi
from oracle import prologue as op
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

NAMES = ("xq", "xk", "xv", "a", "b", "wq", "wk", "wv", "A_log", "dt_bias")


def _bf16_close(x, ref, what):
    err = np.abs(x - ref) - (2.0 ** -7 * np.abs(ref) + 1e-6)
    assert err.max() <= 0, f"{what}: worst excess {err.max():.3e}"


def _f32_close(x, ref, what, rtol=1e-5):
    err = np.abs(x - ref) - rtol * np.abs(ref)
    assert err.max() <= 0, f"{what}: worst excess {err.max():.3e}"


def _run(x, conv=None, inplace=False):
    conv_t = dev(conv) if conv is not None else None
    outs = gdn.gdn_prologue(*[dev(x[n]) for n in NAMES], conv_state=conv_t, update_conv_state=inplace)
    q, k, v, g, beta, st = outs
    if inplace:
        assert st is conv_t
    return [host(t) for t in (q, k, v, g, beta, st)]


def _check(x, got, conv_f64=None):
    ref = op.prologue(*[x[n + "_f64"] for n in NAMES], conv_state=conv_f64)
    for name, a, r in zip(("q", "k", "v"), got[:3], ref[:3]):
        _bf16_close(a, r, name)
    _f32_close(got[3], ref[3], "g")
    _f32_close(got[4], ref[4], "beta")
    np.testing.assert_array_equal(got[5], ref[5])   # new convolution state: exact copies


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_prologue_ragged(Dk, Dv):
    x = gi.layer_inputs(2, 150, 3, Dk, Dv, seed=800 + Dk + Dv)
    _check(x, _run(x))


@pytest.mark.parametrize("T", [1, 2, 3, 4, 67])
def test_prologue_with_carried_state(T):
    x = gi.layer_inputs(3, T, 2, 128, 128, seed=820 + T, conv_state=True)
    _check(x, _run(x, x["conv"]), x["conv_f64"])


@pytest.mark.parametrize("T", [1, 2, 5])
def test_prologue_updates_state_in_place(T):
    x = gi.layer_inputs(2, T, 4, 128, 64, seed=840 + T, conv_state=True)
    _check(x, _run(x, x["conv"], inplace=True), x["conv_f64"])


def test_prologue_decode_sequence_matches_full_sequence():
    """Feeding tokens one at a time through the carried state equals one call
    over the whole sequence (the convolution cache is exact)."""
    import torch
    x = gi.layer_inputs(2, 9, 2, 64, 64, seed=860)
    full = _run(x)
    C = 2 * (2 * 64 + 64)
    state = torch.zeros((2, 3, C), dtype=torch.float32, device="cuda")
    for t in range(9):
        step = {n: x[n] for n in NAMES}
        for n in ("xq", "xk", "xv", "a", "b"):
            step[n] = np.ascontiguousarray(x[n][:, t:t + 1])
        got = gdn.gdn_prologue(*[dev(step[n]) for n in NAMES], conv_state=state, update_conv_state=True)
        for i in range(5):
            np.testing.assert_array_equal(host(got[i]), full[i][:, t:t + 1])
    np.testing.assert_array_equal(host(state), full[5])


def test_prologue_full_layer_sampled():
    """The full layer shape (B 8, T 4096, H 8, Dk = Dv = 128) in the launch the
    layer benchmark uses, checked on token windows against the oracle run on
    the window with the 3 preceding inputs as its convolution state."""
    x = gi.workload("layer_full_bf16")
    got = _run(x)
    H, Dk, Dv = x["H"], x["Dk"], x["Dv"]
    for b, t0, t1 in ((0, 0, 70), (3, 2000, 2064), (7, 4030, 4096)):
        win = {n: x[n + "_f64"] for n in ("wq", "wk", "wv", "A_log", "dt_bias")}
        for n in ("xq", "xk", "xv", "a", "b"):
            win[n] = x[n + "_f64"][b:b + 1, t0:t1]
        conv = None
        if t0 >= 3:
            hist = [x[n + "_f64"][b:b + 1, t0 - 3:t0].reshape(1, 3, -1) for n in ("xq", "xk", "xv")]
            conv = np.concatenate(hist, axis=2)
        ref = op.prologue(*[win[n] for n in NAMES], conv_state=conv)
        for i, name in enumerate(("q", "k", "v")):
            _bf16_close(got[i][b:b + 1, t0:t1], ref[i], f"{name} window {b},{t0}")
        _f32_close(got[3][b:b + 1, t0:t1], ref[3], "g")
        _f32_close(got[4][b:b + 1, t0:t1], ref[4], "beta")
    assert got[5].shape == (8, 3, H * (2 * Dk + Dv))


@pytest.mark.parametrize("Dv", [128, 64])
def test_gated_rmsnorm(Dv):
    rng = np.random.default_rng(870 + Dv)
    o = (0.5 * rng.standard_normal((3, 77, 5, Dv))).astype(np.float32)
    x = gi.layer_inputs(3, 77, 5, 64, Dv, seed=880 + Dv)
    y = host(gdn.gdn_gated_rmsnorm(dev(o), dev(x["z"]), dev(x["norm_w"]), eps=1e-5))
    _bf16_close(y, op.gated_rmsnorm(o.astype(np.float64), x["z_f64"], x["norm_w_f64"], eps=1e-5), "y")


def test_gated_rmsnorm_zero_rows_and_large_eps():
    """A row of zeros stays zero (no division by zero), and a large eps gives
    the unnormalised product o * w * SiLU(z) / sqrt(eps)."""
    o = np.zeros((4, 128), dtype=np.float32)
    o[1] = np.linspace(-1, 1, 128, dtype=np.float32)
    x = gi.layer_inputs(1, 4, 1, 64, 128, seed=890)
    z, w = x["z"].reshape(4, 128), x["norm_w"]
    y = host(gdn.gdn_gated_rmsnorm(dev(o), dev(z), dev(w), eps=1e-5))
    assert np.all(y[0] == 0) and np.all(y[2:] == 0)
    _bf16_close(y, op.gated_rmsnorm(o.astype(np.float64), x["z_f64"].reshape(4, 128), x["norm_w_f64"]), "y")
    y = host(gdn.gdn_gated_rmsnorm(dev(o), dev(z), dev(w), eps=1e6))
    _bf16_close(y, op.gated_rmsnorm(o.astype(np.float64), x["z_f64"].reshape(4, 128), x["norm_w_f64"], 1e6), "y")
