"""Seeded synthetic inputs for the gated delta rule forward, shared by the
oracle side and the device side.

This module only draws random numbers and quantises them; it holds none of
the delta-rule arithmetic.  The gate maps it applies (sigmoid for the write
strength, -A*softplus for the log-decay) produce *inputs* of the op, as the
layer in front of it would (GatedDeltaNet walkthrough, yfxerp.com, section on
the gating mechanism; Gated DeltaNet-2 article, 7minutos.es, section on the
block design).

Recipe (one numpy PCG64 stream per workload, fp64 draws, then quantised):
  q, k, v ~ N(0, 1); q and k L2-normalised per (b, t, h) in fp64;
  beta = sigmoid(N(0, 1));  g = -A_h * softplus(N(0, 1) + dt_bias), A_h ~ U(1, 16)
  per head, dt_bias = 0;  h0 ~ N(0, 0.02) (standard deviation 0.02) when asked.
  GDN-2: log_alpha = -softplus(N(0,1)) per key channel (kept in log space),
  b = sigmoid(N(0,1)) per key channel, w = sigmoid(N(0,1)) per value channel.
Draw order is fixed (q, k, v, then gates, then h0) so a seed names one input.

Floating outputs are returned twice: ``*_f64`` holds the exact values the
device receives (bf16 -> fp64 and fp32 -> fp64 are exact), and the device
copy is returned as raw bits (``uint16`` for bf16) or ``float32``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f64",
    "bf16_bits_to_f64",
    "quantise",
    "gdn_inputs",
    "gdn2_inputs",
    "step_inputs",
    "WORKLOADS",
    "step2_inputs",
    "layer_inputs",
]

# Named workloads: shapes and dtypes of the measured and parity cases.
WORKLOADS = {
    "tiny_fp32": dict(kind="gdn", B=1, H=2, T=256, Dk=64, Dv=64, dtype="fp32", h0=False, seed=1000),
    "layer_bf16": dict(kind="gdn", B=8, H=8, T=4096, Dk=128, Dv=128, dtype="bf16", h0=False, seed=1001),
    "long_bf16": dict(kind="gdn", B=1, H=16, T=65536, Dk=128, Dv=128, dtype="bf16", h0=True, seed=1002),
    "decode_bf16": dict(kind="step", B=256, H=16, Dk=128, Dv=128, dtype="bf16", seed=1003),
    "gdn2_bf16": dict(kind="gdn2", B=4, H=8, T=4096, Dk=128, Dv=128, dtype="bf16", h0=False, seed=1004),
    "decode2_bf16": dict(kind="step2", B=256, H=16, Dk=128, Dv=128, dtype="bf16", seed=1005),
    "layer_bwd_bf16": dict(kind="gdn", B=8, H=8, T=4096, Dk=128, Dv=128, dtype="bf16", h0=False, seed=1001),
    "gdn2_bwd_bf16": dict(kind="gdn2", B=4, H=8, T=4096, Dk=128, Dv=128, dtype="bf16", h0=False, seed=1004),
    "layer_full_bf16": dict(kind="layer", B=8, H=8, T=4096, Dk=128, Dv=128, dtype="bf16", conv_state=False,
                            seed=1006),
}


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 -> fp32 -> bf16 with round-to-nearest-even; returns uint16 bits."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def quantise(x: np.ndarray, dtype: str):
    """Return (device_array, exact_f64_values) for dtype 'bf16' or 'fp32'."""
    if dtype == "bf16":
        bits = bf16_bits_from_f64(x)
        return bits, bf16_bits_to_f64(bits)
    if dtype == "fp32":
        x32 = np.ascontiguousarray(x, dtype=np.float32)
        return x32, x32.astype(np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _f32(x):
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return x32, x32.astype(np.float64)


def _pack(out: dict, name: str, x: np.ndarray, dtype: str):
    dev, f64 = quantise(x, dtype)
    out[name] = dev
    out[name + "_f64"] = f64


def gdn_inputs(B, T, H, Dk, Dv, seed, dtype="bf16", h0=False, a_range=(1.0, 16.0),
               dt_bias=0.0):
    """Inputs of the chunked GDN forward, layout [B, T, H, D] / gates [B, T, H]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(rng.standard_normal((B, T, H, Dk)))
    k = _l2n(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    beta = _sigmoid(rng.standard_normal((B, T, H)))
    glogit = rng.standard_normal((B, T, H))
    A = rng.uniform(a_range[0], a_range[1], size=(H,))
    g = -A[None, None, :] * _softplus(glogit + dt_bias)
    out = {"B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "dtype": dtype,
           "scale": 1.0 / np.sqrt(Dk)}
    _pack(out, "q", q, dtype)
    _pack(out, "k", k, dtype)
    _pack(out, "v", v, dtype)
    out["g"], out["g_f64"] = _f32(g)
    out["beta"], out["beta_f64"] = _f32(beta)
    if h0:
        out["h0"], out["h0_f64"] = _f32(0.02 * rng.standard_normal((B, H, Dk, Dv)))
    else:
        out["h0"], out["h0_f64"] = None, None
    return out


def gdn2_inputs(B, T, H, Dk, Dv, seed, dtype="bf16", h0=False):
    """Inputs of the chunked GDN-2 forward: per-channel log-decay, erase and write gates."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(rng.standard_normal((B, T, H, Dk)))
    k = _l2n(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    log_alpha = -_softplus(rng.standard_normal((B, T, H, Dk)))
    b = _sigmoid(rng.standard_normal((B, T, H, Dk)))
    w = _sigmoid(rng.standard_normal((B, T, H, Dv)))
    out = {"B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "dtype": dtype,
           "scale": 1.0 / np.sqrt(Dk)}
    _pack(out, "q", q, dtype)
    _pack(out, "k", k, dtype)
    _pack(out, "v", v, dtype)
    out["log_alpha"], out["log_alpha_f64"] = _f32(log_alpha)
    _pack(out, "b", b, dtype)
    _pack(out, "w", w, dtype)
    if h0:
        out["h0"], out["h0_f64"] = _f32(0.02 * rng.standard_normal((B, H, Dk, Dv)))
    else:
        out["h0"], out["h0_f64"] = None, None
    return out


def step_inputs(B, H, Dk, Dv, seed, dtype="bf16", a_range=(1.0, 16.0)):
    """Inputs of one recurrent decode step: [B, H, D] token tensors, [B, H] gates,
    fp32 state S ~ N(0, 0.02) of shape [B, H, Dk, Dv]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(rng.standard_normal((B, H, Dk)))
    k = _l2n(rng.standard_normal((B, H, Dk)))
    v = rng.standard_normal((B, H, Dv))
    beta = _sigmoid(rng.standard_normal((B, H)))
    glogit = rng.standard_normal((B, H))
    A = rng.uniform(a_range[0], a_range[1], size=(H,))
    g = -A[None, :] * _softplus(glogit)
    S = 0.02 * rng.standard_normal((B, H, Dk, Dv))
    out = {"B": B, "H": H, "Dk": Dk, "Dv": Dv, "dtype": dtype, "scale": 1.0 / np.sqrt(Dk)}
    _pack(out, "q", q, dtype)
    _pack(out, "k", k, dtype)
    _pack(out, "v", v, dtype)
    out["g"], out["g_f64"] = _f32(g)
    out["beta"], out["beta_f64"] = _f32(beta)
    out["S"], out["S_f64"] = _f32(S)
    return out


def step2_inputs(B, H, Dk, Dv, seed, dtype="bf16"):
    """Inputs of one GDN-2 decode step: [B, H, D] token tensors and gates
    (per-channel log-decay, erase and write gates drawn as in gdn2_inputs),
    fp32 state S ~ N(0, 0.02) of shape [B, H, Dk, Dv]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(rng.standard_normal((B, H, Dk)))
    k = _l2n(rng.standard_normal((B, H, Dk)))
    v = rng.standard_normal((B, H, Dv))
    log_alpha = -_softplus(rng.standard_normal((B, H, Dk)))
    b = _sigmoid(rng.standard_normal((B, H, Dk)))
    w = _sigmoid(rng.standard_normal((B, H, Dv)))
    S = 0.02 * rng.standard_normal((B, H, Dk, Dv))
    out = {"B": B, "H": H, "Dk": Dk, "Dv": Dv, "dtype": dtype, "scale": 1.0 / np.sqrt(Dk)}
    _pack(out, "q", q, dtype)
    _pack(out, "k", k, dtype)
    _pack(out, "v", v, dtype)
    out["log_alpha"], out["log_alpha_f64"] = _f32(log_alpha)
    _pack(out, "b", b, dtype)
    _pack(out, "w", w, dtype)
    out["S"], out["S_f64"] = _f32(S)
    return out


def layer_inputs(B, T, H, Dk, Dv, seed, conv_state=False):
    """Inputs of the layer around the rule: the projections entering the short
    convolution (bf16), the gate pre-activations a, b (fp32), the convolution
    taps, A_log and dt_bias (fp32), the output gate z (bf16) and the RMSNorm
    weight (fp32); conv_state [B, 3, H*(2Dk+Dv)] fp32 when asked.
    Recipe: projections, a, b, z ~ N(0, 1); taps ~ U(-0.5, 0.5) (a depthwise
    convolution's default bound 1/sqrt(4)); A = exp(A_log) ~ U(1, 16);
    dt_bias = softplus^-1(dt) with log dt ~ U(log 1e-3, log 0.1); RMSNorm
    weight 1 + 0.1 N(0, 1); conv_state ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "dtype": "bf16", "scale": 1.0 / np.sqrt(Dk)}
    _pack(out, "xq", rng.standard_normal((B, T, H, Dk)), "bf16")
    _pack(out, "xk", rng.standard_normal((B, T, H, Dk)), "bf16")
    _pack(out, "xv", rng.standard_normal((B, T, H, Dv)), "bf16")
    out["a"], out["a_f64"] = _f32(rng.standard_normal((B, T, H)))
    out["b"], out["b_f64"] = _f32(rng.standard_normal((B, T, H)))
    out["wq"], out["wq_f64"] = _f32(rng.uniform(-0.5, 0.5, size=(H * Dk, 4)))
    out["wk"], out["wk_f64"] = _f32(rng.uniform(-0.5, 0.5, size=(H * Dk, 4)))
    out["wv"], out["wv_f64"] = _f32(rng.uniform(-0.5, 0.5, size=(H * Dv, 4)))
    out["A_log"], out["A_log_f64"] = _f32(np.log(rng.uniform(1.0, 16.0, size=(H,))))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=(H,)))
    out["dt_bias"], out["dt_bias_f64"] = _f32(dt + np.log(-np.expm1(-dt)))
    _pack(out, "z", rng.standard_normal((B, T, H, Dv)), "bf16")
    out["norm_w"], out["norm_w_f64"] = _f32(1.0 + 0.1 * rng.standard_normal((Dv,)))
    if conv_state:
        out["conv"], out["conv_f64"] = _f32(rng.standard_normal((B, 3, H * (2 * Dk + Dv))))
    else:
        out["conv"], out["conv_f64"] = None, None
    return out


def workload(name: str, **overrides):
    """Build the inputs of a named workload (see WORKLOADS); keyword overrides
    replace shape or seed fields (used for reduced-size parity cases)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "gdn":
        return gdn_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"],
                          dtype=cfg["dtype"], h0=cfg["h0"])
    if kind == "gdn2":
        return gdn2_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"],
                           dtype=cfg["dtype"], h0=cfg["h0"])
    if kind == "step":
        return step_inputs(cfg["B"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"], dtype=cfg["dtype"])
    if kind == "step2":
        return step2_inputs(cfg["B"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"], dtype=cfg["dtype"])
    if kind == "layer":
        return layer_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"],
                            conv_state=cfg["conv_state"])
    raise ValueError(kind)
