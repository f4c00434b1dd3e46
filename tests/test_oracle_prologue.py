"""Pins of the plain definitions around the rule (oracle/prologue.py): library
routines (torch's conv1d, SiLU, sigmoid, softplus, scipy's expit), printed
constants and closed forms, so that a dropped term, a wrong sign or a wrong
tap order fails here.

Each pin takes the module under test as its argument; the tests below run
them on oracle/prologue.py, and tests/test_oracle_mutants.py runs them on
copies with planted mistakes, each of which some pin must reject."""
import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

from oracle import prologue as PRO


def pin_activations_against_library(P):
    """SiLU, sigmoid and softplus against torch's and scipy's float64 routines
    and against closed forms: silu(x) - silu(-x) = x, sigmoid(x) + sigmoid(-x) = 1,
    softplus(x) - softplus(-x) = x, softplus(0) = ln 2, and printed values of
    the logistic function (sigmoid(1) = e / (1 + e), sigmoid(2) = e^2 / (1 + e^2))."""
    x = np.linspace(-30.0, 30.0, 1201)
    xt = torch.from_numpy(x)
    np.testing.assert_allclose(P.silu(x), F.silu(xt).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(P.sigmoid(x), torch.sigmoid(xt).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(P.sigmoid(x), scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    # torch switches softplus to the identity above `threshold`; lift it out of the range
    np.testing.assert_allclose(P.softplus(x), F.softplus(xt, threshold=1e9).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(P.silu(x) - P.silu(-x), x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(P.sigmoid(x) + P.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(P.softplus(x) - P.softplus(-x), x, rtol=1e-13, atol=1e-13)
    assert abs(P.softplus(np.array(0.0)) - 0.6931471805599453) < 1e-16
    assert abs(P.sigmoid(np.array(1.0)) - 0.7310585786300049) < 1e-16
    assert abs(P.sigmoid(np.array(2.0)) - 0.8807970779778823) < 1e-16
    assert abs(P.silu(np.array(1.0)) - 0.7310585786300049) < 1e-16
    assert abs(P.silu(np.array(-1.0)) + 0.2689414213699951) < 1e-16


def pin_short_conv_equals_grouped_conv1d(P):
    """Causal depthwise conv = torch conv1d with groups = C and 3 leading zeros
    (conv1d is a cross-correlation, so its taps line up with ours unflipped)."""
    rng = np.random.default_rng(1)
    B, T, C = 2, 11, 5
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, 4))
    y, _ = P.short_conv(x, w)
    xt = torch.from_numpy(x).permute(0, 2, 1)                         # [B, C, T]
    ref = F.conv1d(F.pad(xt, (3, 0)), torch.from_numpy(w)[:, None, :], groups=C).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(y, ref, atol=1e-13)


def pin_short_conv_last_tap_and_state(P):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 9, 3))
    w = np.zeros((3, 4))
    w[:, 3] = 1.0
    np.testing.assert_array_equal(P.short_conv(x, w)[0], x)
    w = rng.standard_normal((3, 4))
    y_all, s_all = P.short_conv(x, w)
    y1, s1 = P.short_conv(x[:, :2], w)            # fewer tokens than the cache
    y2, s2 = P.short_conv(x[:, 2:], w, s1)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y_all, atol=1e-14)
    np.testing.assert_allclose(s2, s_all, atol=0)
    np.testing.assert_array_equal(s_all, x[:, -3:])


def _layer_case(seed=3):
    rng = np.random.default_rng(seed)
    B, T, H, Dk, Dv = 2, 6, 3, 8, 6
    c = dict(B=B, T=T, H=H, Dk=Dk, Dv=Dv)
    c["xq"] = rng.standard_normal((B, T, H, Dk))
    c["xk"] = rng.standard_normal((B, T, H, Dk))
    c["xv"] = rng.standard_normal((B, T, H, Dv))
    c["a"] = rng.standard_normal((B, T, H)) * 4
    c["b"] = rng.standard_normal((B, T, H)) * 3
    c["wq"] = rng.standard_normal((H * Dk, 4))
    c["wk"] = rng.standard_normal((H * Dk, 4))
    c["wv"] = rng.standard_normal((H * Dv, 4))
    c["A_log"] = np.log(rng.uniform(1, 16, H))
    c["dt_bias"] = rng.standard_normal(H)
    c["state"] = rng.standard_normal((B, 3, H * (2 * Dk + Dv)))
    return c


def pin_prologue_against_torch(P):
    """The whole prologue against the same steps in torch float64 ops: grouped
    conv1d over the carried state, F.silu, division by sqrt(sum of squares +
    1e-6), F.softplus, torch.sigmoid.  The gate map is
    g = -exp(A_log) * softplus(a + dt_bias) with softplus taken of the sum, and
    beta = sigmoid(b)."""
    c = _layer_case()
    B, T, H, Dk, Dv = c["B"], c["T"], c["H"], c["Dk"], c["Dv"]
    q, k, v, g, beta, st = P.prologue(c["xq"], c["xk"], c["xv"], c["a"], c["b"], c["wq"], c["wk"], c["wv"],
                                      c["A_log"], c["dt_bias"], c["state"])
    tt = torch.from_numpy
    xs = [c["xq"].reshape(B, T, H * Dk), c["xk"].reshape(B, T, H * Dk), c["xv"].reshape(B, T, H * Dv)]
    cut = [0, H * Dk, 2 * H * Dk, 2 * H * Dk + H * Dv]
    outs = []
    for i, (x, w) in enumerate(zip(xs, (c["wq"], c["wk"], c["wv"]))):
        past = tt(c["state"][:, :, cut[i]:cut[i + 1]])
        full = torch.cat([past, tt(x)], 1).permute(0, 2, 1)            # [B, C, T + 3]
        y = F.conv1d(full, tt(w)[:, None, :], groups=x.shape[-1]).permute(0, 2, 1)
        outs.append(F.silu(y))
    rq = outs[0].reshape(B, T, H, Dk)
    rk = outs[1].reshape(B, T, H, Dk)
    rq = rq / torch.sqrt((rq * rq).sum(-1, keepdim=True) + 1e-6)
    rk = rk / torch.sqrt((rk * rk).sum(-1, keepdim=True) + 1e-6)
    rv = outs[2].reshape(B, T, H, Dv)
    rg = -torch.exp(tt(c["A_log"])) * F.softplus(tt(c["a"]) + tt(c["dt_bias"]), threshold=1e9)
    rb = torch.sigmoid(tt(c["b"]))
    for got, ref in ((q, rq), (k, rk), (v, rv), (g, rg), (beta, rb)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)
    full_all = np.concatenate([c["state"], np.concatenate(xs, 2)], 1)
    np.testing.assert_array_equal(st, full_all[:, -3:])


def pin_l2norm_and_gate_closed_forms(P):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 7, 16)) * 3
    np.testing.assert_allclose(np.linalg.norm(P.l2norm(x), axis=-1), 1.0, atol=1e-7)
    # |l2norm(x)| = sqrt(s / (s + eps)), s = |x|^2: pins where eps enters
    s = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(P.l2norm(x), axis=-1), np.sqrt(s / (s + 1e-6)), rtol=1e-13)
    small = np.full((1, 4), 1e-4)                       # s = 4e-8, well below eps
    np.testing.assert_allclose(P.l2norm(small), small / np.sqrt(4e-8 + 1e-6), rtol=1e-13)
    c = _layer_case(5)
    H = c["H"]
    one = {n: c[n][:1, :1] for n in ("xq", "xk", "xv", "b")}
    # softplus asymptotes: g -> -exp(A_log) (a + dt) for large a + dt, g -> 0 for very negative a
    big = np.full((1, 1, H), 60.0)
    g_big = P.prologue(one["xq"], one["xk"], one["xv"], big, one["b"], c["wq"], c["wk"], c["wv"], c["A_log"],
                       c["dt_bias"])[3]
    np.testing.assert_allclose(g_big[0, 0], -np.exp(c["A_log"]) * (60.0 + c["dt_bias"]), rtol=1e-12)
    # a + dt_bias = 0 exactly: g = -exp(A_log) ln 2
    g0 = P.prologue(one["xq"], one["xk"], one["xv"], -c["dt_bias"][None, None, :], one["b"], c["wq"], c["wk"],
                    c["wv"], c["A_log"], c["dt_bias"])[3]
    np.testing.assert_allclose(g0[0, 0], -np.exp(c["A_log"]) * np.log(2.0), rtol=1e-14)
    out = P.prologue(one["xq"], one["xk"], one["xv"], -big, np.zeros((1, 1, H)), c["wq"], c["wk"], c["wv"],
                     c["A_log"], c["dt_bias"])
    assert np.abs(out[3]).max() < 1e-20
    np.testing.assert_array_equal(out[4], 0.5)
    # beta = sigmoid(b) at b = 2: e^2 / (1 + e^2), a printed constant
    b2 = np.full((1, 1, H), 2.0)
    beta2 = P.prologue(one["xq"], one["xk"], one["xv"], big, b2, c["wq"], c["wk"], c["wv"], c["A_log"],
                       c["dt_bias"])[4]
    np.testing.assert_allclose(beta2, 0.8807970779778823, rtol=1e-15)


def pin_gated_rmsnorm(P):
    rng = np.random.default_rng(4)
    o = rng.standard_normal((3, 4, 32))
    z = rng.standard_normal((3, 4, 32))
    w = rng.standard_normal(32)
    y = P.gated_rmsnorm(o, z, w, eps=0.0)
    np.testing.assert_allclose(P.gated_rmsnorm(7.5 * o, z, w, eps=0.0), y, atol=1e-13)   # scale invariance
    cst = np.full((1, 1, 32), -2.0)
    np.testing.assert_allclose(P.gated_rmsnorm(cst, z[:1, :1], w, eps=0.0), -w * F.silu(torch.from_numpy(
        z[:1, :1])).numpy(), atol=1e-14)
    # against torch: rms over the last axis, eps inside the root, SiLU gate
    tt = torch.from_numpy
    ref = tt(o) * torch.rsqrt((tt(o) ** 2).mean(-1, keepdim=True) + 0.25) * tt(w) * F.silu(tt(z))
    np.testing.assert_allclose(P.gated_rmsnorm(o, z, w, eps=0.25), ref.numpy(), rtol=1e-13, atol=1e-14)


PINS = [
    pin_activations_against_library,
    pin_short_conv_equals_grouped_conv1d,
    pin_short_conv_last_tap_and_state,
    pin_prologue_against_torch,
    pin_l2norm_and_gate_closed_forms,
    pin_gated_rmsnorm,
]


def test_activations_against_library():
    pin_activations_against_library(PRO)


def test_short_conv_equals_grouped_conv1d():
    pin_short_conv_equals_grouped_conv1d(PRO)


def test_short_conv_last_tap_is_identity_and_state_continues():
    pin_short_conv_last_tap_and_state(PRO)


def test_prologue_against_torch():
    pin_prologue_against_torch(PRO)


def test_l2norm_and_gates_closed_forms():
    pin_l2norm_and_gate_closed_forms(PRO)


def test_gated_rmsnorm_invariants():
    pin_gated_rmsnorm(PRO)
