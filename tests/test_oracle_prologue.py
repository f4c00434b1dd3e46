"""Pins of the plain definitions around the rule (oracle/prologue.py): a
library routine for the convolution, closed forms and invariants for the
rest, so that a dropped term, a wrong sign or tap order fails here."""
import numpy as np
import torch

from oracle import prologue as P


def test_short_conv_equals_grouped_conv1d():
    """Causal depthwise conv = torch conv1d with groups = C and 3 leading zeros,
    kernel flipped into conv1d's cross-correlation order (same taps)."""
    rng = np.random.default_rng(1)
    B, T, C = 2, 11, 5
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, 4))
    y, _ = P.short_conv(x, w)
    xt = torch.from_numpy(x).permute(0, 2, 1)                         # [B, C, T]
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (3, 0)), torch.from_numpy(w)[:, None, :],
                                     groups=C).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(y, ref, atol=1e-13)


def test_short_conv_last_tap_is_identity_and_state_continues():
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


def test_l2norm_unit_rows_and_gates_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 7, 16)) * 3
    np.testing.assert_allclose(np.linalg.norm(P.l2norm(x), axis=-1), 1.0, atol=1e-7)
    B, T, H = 2, 5, 3
    xq = rng.standard_normal((B, T, H, 8))
    xv = rng.standard_normal((B, T, H, 6))
    a = rng.standard_normal((B, T, H)) * 4
    b = rng.standard_normal((B, T, H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt_bias = rng.standard_normal(H)
    w8 = rng.standard_normal((H * 8, 4))
    w6 = rng.standard_normal((H * 6, 4))
    q, k, v, g, beta, st = P.prologue(xq, xq, xv, a, b, w8, w8, w6, A_log, dt_bias)
    assert (g <= 0).all() and (beta > 0).all() and (beta < 1).all()
    # |l2norm(x)| = sqrt(s / (s + eps)) with s = |x|^2 of the activated convolution output
    yq = P.silu(P.short_conv(xq.reshape(B, T, H * 8), w8)[0]).reshape(B, T, H, 8)
    s2 = np.sum(yq * yq, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), np.sqrt(s2 / (s2 + 1e-6)), rtol=1e-13)
    # softplus asymptotes: g -> -exp(A_log) (a + dt) for large a, g -> 0 for very negative a
    big = np.full((1, 1, H), 60.0)
    _, _, _, g_big, _, _ = P.prologue(xq[:1, :1], xq[:1, :1], xv[:1, :1], big, b[:1, :1], w8, w8, w6, A_log, dt_bias)
    np.testing.assert_allclose(g_big[0, 0], -np.exp(A_log) * (60.0 + dt_bias), rtol=1e-12)
    _, _, _, g_small, beta0, _ = P.prologue(xq[:1, :1], xq[:1, :1], xv[:1, :1], -big, 0 * b[:1, :1], w8, w8, w6,
                                            A_log, dt_bias)
    assert np.abs(g_small).max() < 1e-20
    np.testing.assert_array_equal(beta0, 0.5)
    assert st.shape == (B, 3, H * (8 + 8 + 6))


def test_gated_rmsnorm_invariants():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((3, 4, 32))
    z = rng.standard_normal((3, 4, 32))
    w = rng.standard_normal(32)
    y = P.gated_rmsnorm(o, z, w, eps=0.0)
    np.testing.assert_allclose(P.gated_rmsnorm(7.5 * o, z, w, eps=0.0), y, atol=1e-13)   # scale invariance
    c = np.full((1, 1, 32), -2.0)
    np.testing.assert_allclose(P.gated_rmsnorm(c, z[:1, :1], w, eps=0.0), -w * P.silu(z[:1, :1]), atol=1e-14)
    np.testing.assert_allclose(np.sqrt(np.mean((y / (w * P.silu(z))) ** 2, axis=-1)), 1.0, atol=1e-12)
