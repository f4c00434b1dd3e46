"""The chunked Gated DeltaNet-2 backward evaluated with float32 products: the
arithmetic floor that the GPU backward's tolerance bars in
tests/test_parity_bwd2.py are set against.  Not a reference for parity (the
fp64 oracle is); test infrastructure that makes those bars reproducible.

The chunk equations are those of the Gated DeltaNet-2 article's chunked
training section, differentiated in reverse chunk order (the same equations
as oracle/chunked.py's gdn2_chunk_bwd_head, restated here so that each
product can be rounded).  As on the GPU's fp32 path:
  - the per-channel gate sums run in float64 and are rounded once to
    float32 (times log2 e), and every decay factor is exp2 of a float32
    difference of them, rounded to float32;
  - A, P, the decayed operands Ehat, Qhat, Khat, T = (I + A)^-1 and the entry
    states are float32 numbers;
  - every matrix product and every channel contraction of the key side takes
    float32 operands and accumulates in float32;
  - the elementwise steps stay in float64.

    python -m tests.fp32_bwd2_eval            # the GDN-2 workload, every head

prints, per gradient, the worst over the 32 heads of max|diff| / rms against
the fp64 chunked oracle."""
import numpy as np

from oracle import chunked as ch

LOG2E = 1.4426950408889634
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dh0")


def _f32(x):
    return np.asarray(x, np.float32)


def _mm(a, b):
    """One product as float32 hardware forms it (fp32 operands and result)."""
    return (_f32(a) @ _f32(b)).astype(np.float64)


def _ein(spec, *ops):
    """A channel contraction with float32 operands, accumulated in float32."""
    return np.einsum(spec, *[_f32(o) for o in ops]).astype(np.float64)


def bwd2_head_fp32(q, k, v, log_alpha, bgate, wgate, S0, dO, dST, scale, C=64):
    """dq, dk, dv, dlog_alpha, db, dw, dS0 of one head with float32 products.
    Entry states come from the fp64 chunked forward, rounded to float32."""
    T, Dk = q.shape
    Dv = v.shape[1]
    starts = []
    S = np.array(S0, dtype=np.float64, copy=True)
    for s in range(0, T, C):
        starts.append(S)
        _, S, _ = ch.gdn2_chunk_head(q[s:s + C], k[s:s + C], v[s:s + C], log_alpha[s:s + C], bgate[s:s + C],
                                     wgate[s:s + C], S, scale, C)
    dq, dk, dla, db = (np.zeros((T, Dk)) for _ in range(4))
    dv, dw = np.zeros((T, Dv)), np.zeros((T, Dv))
    dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    for ci in range(len(starts) - 1, -1, -1):
        s, e = ci * C, min(ci * C + C, T)
        n = e - s
        S = _f32(starts[ci]).astype(np.float64)
        Q, K, V, Bg, Wg, dOc = q[s:e], k[s:e], v[s:e], bgate[s:e], wgate[s:e], dO[s:e]
        G2 = _f32(np.cumsum(log_alpha[s:e], axis=0) * LOG2E)            # [n, Dk], float32
        lower = np.tril(np.ones((n, n), dtype=bool))
        diff = (G2[:, None, :] - G2[None, :, :]).astype(np.float32)      # float32 differences
        D3 = np.where(lower[:, :, None], _f32(np.exp2(diff.astype(np.float64))), np.float32(0)).astype(np.float64)
        Gam = _f32(np.exp2(G2.astype(np.float64))).astype(np.float64)
        dec = _f32(np.exp2((G2[-1][None, :] - G2).astype(np.float32).astype(np.float64))).astype(np.float64)
        E = Bg * K
        Z = Wg * V
        A = _f32(np.tril(_ein("ic,jc,ijc->ij", E, K, D3), -1)).astype(np.float64)
        Tm = _f32(ch._tri_inverse(A)).astype(np.float64)
        P = _f32(_ein("ic,jc,ijc->ij", Q, K, D3)).astype(np.float64)
        Eh = _f32(Gam * E).astype(np.float64)
        Qh = _f32(Gam * Q).astype(np.float64)
        Kh = _f32(K * dec).astype(np.float64)
        R = Z - _mm(Eh, S)
        Dl = _mm(Tm, R)
        dSp = dS
        dDl = scale * _mm(P.T, dOc) + _mm(Kh, dSp)
        dR = _mm(Tm.T, dDl)
        dEh = -_mm(dR, S.T)
        dA = -np.tril(_mm(dR, Dl.T), -1)
        dP = scale * np.tril(_mm(dOc, Dl.T))
        dQh = scale * _mm(dOc, S.T)
        dKh = _mm(Dl, dSp.T)
        dS = Gam[-1][:, None] * dSp + scale * _mm(Qh.T, dOc) - _mm(Eh.T, dR)
        dG = np.zeros((n, Dk))
        dE = np.zeros((n, Dk))
        dKc = np.zeros((n, Dk))
        dQc = np.zeros((n, Dk))
        dw[s:e] = dR * V
        dv[s:e] = dR * Wg
        dE += Gam * dEh
        dG += Gam * E * dEh
        dQc += Gam * dQh
        dG += Gam * Q * dQh
        dE += _ein("ij,jc,ijc->ic", dA, K, D3)
        dKc += _ein("ij,ic,ijc->jc", dA, E, D3)
        dG += _ein("ij,ic,jc,ijc->ic", dA, E, K, D3) - _ein("ij,ic,jc,ijc->jc", dA, E, K, D3)
        dQc += _ein("ij,jc,ijc->ic", dP, K, D3)
        dKc += _ein("ij,ic,ijc->jc", dP, Q, D3)
        dG += _ein("ij,ic,jc,ijc->ic", dP, Q, K, D3) - _ein("ij,ic,jc,ijc->jc", dP, Q, K, D3)
        dKc += dec * dKh
        t = dKh * Kh
        dG -= t
        dG[-1] += t.sum(axis=0) + Gam[-1] * np.sum(dSp * S, axis=1)
        db[s:e] = dE * K
        dKc += dE * Bg
        dq[s:e] = dQc
        dk[s:e] = dKc
        dla[s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dv, dla, db, dw, dS


def per_head_errors(x, do, dht):
    """[heads, 7] of max|diff| / rms (dq, dk, dv, dlog_alpha, db, dw, dh0) for
    every (batch, head) of generator output x against the fp64 chunked oracle."""
    B, T, H = x["log_alpha"].shape[:3]
    names = ("q", "k", "v", "log_alpha", "b", "w")
    out = []
    for b in range(B):
        for h in range(H):
            args = [x[n + "_f64"][b, :, h] for n in names]
            Dk, Dv = args[0].shape[1], args[2].shape[1]
            S0 = x["h0_f64"][b, h] if x["h0_f64"] is not None else np.zeros((Dk, Dv))
            dST = None if dht is None else dht[b, h]
            ref = ch.gdn2_chunk_bwd_head(*args, S0, do[b, :, h], dST, x["scale"])
            got = bwd2_head_fp32(*args, S0, do[b, :, h], dST, x["scale"])
            out.append([float(np.abs(a - r).max() / max(np.sqrt(np.mean(r * r)), 1e-300)) for a, r in zip(got, ref)])
    return np.array(out)


_WORKLOAD = {}


def _gdn2_workload():
    """The full-size GDN-2 backward test's inputs (tests/test_parity_bwd2.py), once per process."""
    if not _WORKLOAD:
        import gdn_inputs as gi
        x = gi.workload("gdn2_bf16")
        rng = np.random.default_rng(960)
        B, T, H, Dk, Dv = x["B"], x["T"], x["H"], x["Dk"], x["Dv"]
        _WORKLOAD["x"] = x
        _WORKLOAD["do"] = rng.standard_normal((B, T, H, Dv)).astype(np.float32).astype(np.float64)
        _WORKLOAD["dht"] = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32).astype(np.float64)
    return _WORKLOAD["x"], _WORKLOAD["do"], _WORKLOAD["dht"]


def _one(args):
    b, h = args
    x, do, dht = _gdn2_workload()
    sub = {n: x[n][b:b + 1, :, h:h + 1] for n in x
           if n.endswith("_f64") and x[n] is not None and x[n].ndim >= 3 and n != "h0_f64"}
    sub["log_alpha"] = x["log_alpha"][b:b + 1, :, h:h + 1]
    sub["h0_f64"] = None if x["h0_f64"] is None else x["h0_f64"][b:b + 1, h:h + 1]
    sub["scale"] = x["scale"]
    return per_head_errors(sub, do[b:b + 1, :, h:h + 1], dht[b:b + 1, h:h + 1])[0]


if __name__ == "__main__":
    import multiprocessing as mp
    x, _, _ = _gdn2_workload()
    with mp.Pool(8) as pool:
        errs = np.array(pool.map(_one, [(b, h) for b in range(x["B"]) for h in range(x["H"])]))
    for i, name in enumerate(GRADS):
        print(f"{name}: worst head {errs[:, i].max():.2e}, median {np.median(errs[:, i]):.2e}")
