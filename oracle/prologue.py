"""Plain fp64 definitions of the operations around the gated delta rule --
TEST INFRASTRUCTURE ONLY (tests, smoke check and benchmark CPU leg; the
product path never imports this module).

GatedDeltaNet walkthrough (yfxerp.com): the data-flow overview and the
sections on the short convolution and the gates.  Before the rule, q, k and v
each pass a depthwise causal convolution over the last 4 positions with SiLU
activation (its 3 past inputs are the decode-time cache), q and k are
L2-normalised, the decay is g = -exp(A_log) * softplus(a + dt_bias) (one A_log
and dt_bias per head) and the write strength beta = sigmoid(b).  After the
rule the output passes a fused RMSNorm with a Swish (SiLU) output gate.  The
Gated DeltaNet-2 article (7minutos.es, block-design section) describes the
same q/k/v paths and the RMS-normalised, SiLU-gated output.

Readings where the pages leave details open: the convolution has no bias and
its last tap multiplies the current token, y_t = sum_{j=0..3} w[:, j] x_{t-3+j};
the RMSNorm weight is one value per channel, shared by all heads, and the
norm is taken over the channels of one head, y = o / sqrt(mean(o^2) + eps) * w * silu(z).
"""
from __future__ import annotations

import numpy as np

CONV = 4  # taps of the short convolution


def silu(x):
    return x / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, x)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def short_conv(x, w, state=None):
    """Causal depthwise convolution over time, per channel.
    x [B, T, C], w [C, 4], state [B, 3, C] (the 3 inputs before t = 0; zero when None).
    Returns (y [B, T, C], new_state [B, 3, C] = the last 3 inputs of state ++ x)."""
    B, T, C = x.shape
    past = np.zeros((B, CONV - 1, C)) if state is None else np.asarray(state, dtype=np.float64)
    full = np.concatenate([past, np.asarray(x, dtype=np.float64)], axis=1)   # [B, T + 3, C]
    y = np.zeros((B, T, C))
    for t in range(T):
        for j in range(CONV):
            y[:, t] += w[:, j] * full[:, t + j]
    return y, full[:, -(CONV - 1):].copy()


def l2norm(x, eps=1e-6):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prologue(xq, xk, xv, a, b, wq, wk, wv, A_log, dt_bias, conv_state=None):
    """q, k, v, g, beta of the op from the projections.
    xq, xk [B, T, H, Dk]; xv [B, T, H, Dv]; a, b [B, T, H]; wq, wk [H*Dk, 4]; wv [H*Dv, 4];
    A_log, dt_bias [H]; conv_state [B, 3, H*(2 Dk + Dv)] (q, k, v channels in that order) or None.
    Returns q, k, v, g, beta and the new conv state."""
    B, T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    cq, ck = H * Dk, H * Dk
    st = [None, None, None] if conv_state is None else [conv_state[:, :, :cq], conv_state[:, :, cq:cq + ck],
                                                        conv_state[:, :, cq + ck:]]
    yq, sq = short_conv(xq.reshape(B, T, cq), wq, st[0])
    yk, sk = short_conv(xk.reshape(B, T, ck), wk, st[1])
    yv, sv = short_conv(xv.reshape(B, T, H * Dv), wv, st[2])
    q = l2norm(silu(yq).reshape(B, T, H, Dk))
    k = l2norm(silu(yk).reshape(B, T, H, Dk))
    v = silu(yv).reshape(B, T, H, Dv)
    g = -np.exp(A_log)[None, None, :] * softplus(a + dt_bias[None, None, :])
    beta = sigmoid(b)
    return q, k, v, g, beta, np.concatenate([sq, sk, sv], axis=2)


def gated_rmsnorm(o, z, w, eps=1e-5):
    """o, z [..., D]; w [D]: o / sqrt(mean(o^2) + eps) * w * silu(z)."""
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w * silu(z)
