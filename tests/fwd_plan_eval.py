"""The chunked Gated DeltaNet forward evaluated with the bf16 path's rounding
points, and with the operand plans that were weighed against it: test
infrastructure that makes the precision plan reproducible.  Not a reference
for parity (the fp64 oracle is).

The chunk equations are those of oracle/chunked.py (GatedDeltaNet
walkthrough, chunked-kernel section), restated so that each operand can be
rounded as the fused kernel rounds it:
  - q, k, v are bf16 numbers; gate sums, decay factors, the elementwise steps
    and every accumulation are float32;
  - K K^T and Q K^T are exact products of bf16 numbers;
  - T - I and the strict part of P enter their products as fp16, and so do
    the residuals R and the new values Vnew they multiply;
  - the state enters K S and Q S as the plan says (below); the update
    K^T (d . Vnew) takes d . Vnew as bf16 hi + lo against the exact keys;
  - the diagonal terms beta_i v_i and (q_i . k_i) vnew_i stay float32.
Plans for the two state reads K S and Q S:
  "hilo"    the kernel's: bf16 hi + lo parts of the float32 state (~16 bits);
  "bf16"    one bf16 rounding of the state for both reads;
  "bf16_q"  hi + lo for K S, one bf16 rounding for Q S;
  "fp16"    one fp16 rounding of the state for both reads, and the decayed
            keys k_j 2^(G_C - G_j) of the update rounded to fp16 (an earlier
            kernel's plan).

    python -m tests.fwd_plan_eval     # every plan on the two evaluation cases
"""
import numpy as np

from oracle import chunked as ch

LOG2E = 1.4426950408889634
PLANS = ("hilo", "bf16", "bf16_q", "fp16")


def _f32(x):
    return np.asarray(x, np.float32).astype(np.float64)


def _f16(x):
    return np.asarray(x, np.float16).astype(np.float64)


def _bf16(x):
    """Round to bfloat16 (nearest, ties to even), as float64."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _hilo(x):
    """x (float32) as bf16 hi + lo, the sum of the two parts."""
    hi = _bf16(x)
    return hi + _bf16(_f32(x) - hi)


def _mm(a, b):
    """A product with float32 accumulation of the given (already rounded) operands."""
    return (np.asarray(a, np.float32) @ np.asarray(b, np.float32)).astype(np.float64)


def fwd_head_plan(q, k, v, g, beta, S0, scale, plan="hilo", C=64):
    """o [T, Dv] and the final state of one head with the given state-read plan."""
    T = q.shape[0]
    S = _f32(S0)
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, bc = q[s:e], k[s:e], v[s:e], _f32(beta[s:e])
        n = e - s
        G2 = _f32(np.cumsum(g[s:e]) * LOG2E)
        lower = np.tril(np.ones((n, n), dtype=bool))
        D = _f32(np.exp2(np.where(lower, _f32(G2[:, None] - G2[None, :]), -np.inf)))
        gam = _f32(np.exp2(G2))
        A = _f32(np.tril(bc[:, None] * _mm(K, K.T) * D, -1))
        TmI = _f16(ch._tri_inverse(A) - np.eye(n))
        QK = _mm(Q, K.T)
        Pstrict = _f16(np.tril(QK * D, -1))
        pdiag = np.diag(QK)
        if plan == "hilo":
            Sk = Sq = _hilo(S)
        elif plan == "bf16":
            Sk = Sq = _bf16(S)
        elif plan == "bf16_q":
            Sk, Sq = _hilo(S), _bf16(S)
        else:
            Sk = Sq = _f16(S)
        X = _mm(K, Sk)
        Y = _mm(Q, Sq)
        R = _f32(bc[:, None] * (V - gam[:, None] * X))
        Vn = _f32(R + _mm(TmI, _f16(R)))
        o[s:e] = scale * _f32(gam[:, None] * Y + pdiag[:, None] * Vn + _mm(Pstrict, _f16(Vn)))
        d = _f32(np.exp2(_f32(G2[-1] - G2)))
        if plan == "fp16":
            upd = _mm(_f16(K * d[:, None]).T, _f16(Vn))
        else:
            upd = _mm(K.T, _hilo(d[:, None] * Vn))
        S = _f32(gam[-1] * S + upd)
    return o, S


def rel_err(x, ref):
    return float(np.abs(x - ref).max() / max(np.sqrt(np.mean(ref * ref)), 1e-300))


def plan_errors(x, plan):
    """(o error, S error), the worst over the heads, of a plan against the fp64 chunked forward."""
    B, T, H = x["g"].shape
    eo = es = 0.0
    for b in range(B):
        for h in range(H):
            args = [x[n + "_f64"][b, :, h] for n in ("q", "k", "v", "g", "beta")]
            S0 = x["h0_f64"][b, h]
            ro, rS, _ = ch.gdn_chunk_head(*args, S0, x["scale"])
            go, gS = fwd_head_plan(*args, S0, x["scale"], plan)
            eo, es = max(eo, rel_err(go, ro)), max(es, rel_err(gS, rS))
    return eo, es


def cases():
    """The two evaluation cases: the layer workload's gate range and weak decay
    (the state carried across many chunks), B 1, T 1024, two heads, d 128."""
    import gdn_inputs as gi
    return {"layer gates": gi.gdn_inputs(1, 1024, 2, 128, 128, seed=81, dtype="bf16", h0=True),
            "weak decay": gi.gdn_inputs(1, 1024, 2, 128, 128, seed=82, dtype="bf16", h0=True,
                                        a_range=(0.001, 0.01))}


if __name__ == "__main__":
    for name, x in cases().items():
        for plan in PLANS:
            eo, es = plan_errors(x, plan)
            print(f"{name:12s} {plan:7s} o {eo:.2e}  S {es:.2e}")
