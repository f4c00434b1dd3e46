"""The chunked Gated DeltaNet backward evaluated with every matrix product in
float32: the arithmetic floor that the GPU backward's tolerance bars are set
against.  Not a reference for parity (the fp64 oracle is); test
infrastructure that makes the bars in tests/test_parity_bwd.py reproducible.

The chunk equations are those of the GatedDeltaNet walkthrough's chunked
section, differentiated in reverse chunk order (the same equations as
oracle/chunked.py's backward, restated here so that each product can be
rounded): operands are rounded to float32 before each product and the
product to float32 after it, while the gate sums, decay factors and the
elementwise steps stay in float64 (the GPU forms the gate sums in fp64 and
takes the decay factors from their differences).

    python -m tests.fp32_bwd_eval            # the layer workload, every head
    python -m tests.fp32_bwd_eval --plan     # the same with the bf16 part plan

prints, per gradient, the worst over the 64 heads of max|diff| / rms against
the fp64 oracle (about 90 s on 8 processes).  With --plan the five products
that the per-chunk kernel accumulates over the value columns take that
kernel's bf16 part splits (BF16_ACCUM_PLAN) instead of float32."""
import numpy as np

from oracle import chunked as ch


def _mm(a, b):
    """One product as float32 hardware forms it (fp32 operands and result)."""
    return (np.asarray(a, np.float32) @ np.asarray(b, np.float32)).astype(np.float64)


def _bf16(x):
    """Round float32 values to bfloat16 (nearest, ties to even), kept as float32."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _parts(x, n):
    """x (float32) as n bfloat16 parts, largest first: each part rounds what
    the earlier ones leave."""
    rest = np.asarray(x, np.float32).copy()
    out = []
    for _ in range(n):
        h = _bf16(rest)
        out.append(h.astype(np.float64))
        rest = (rest - h).astype(np.float32)
    return out


def mm_parts(n):
    """A product on bf16 MFMA with both float32 operands split into n bf16
    parts, keeping the part products of total order below n (3 of 4 for two
    parts, 6 of 9 for three), each accumulated into a float32 result."""
    def f(a, b):
        pa, pb = _parts(a, n), _parts(b, n)
        acc = np.zeros((pa[0].shape[0], pb[0].shape[1]), np.float32)
        for i, x in enumerate(pa):
            for j, y in enumerate(pb):
                if i + j < n:
                    acc = (acc + (x @ y).astype(np.float32)).astype(np.float32)
        return acc.astype(np.float64)
    return f


# The per-chunk GPU kernel's bf16 part plan for its products of two float32
# operands: of the five accumulated over the value columns, dR Vn^T and dR S^T
# take two parts on each side, dO Vn^T, dO S^T and Vn dS'^T three; of the row
# products, (T - I) R and (T - I)^T dVn take two, P^T dO three.
BF16_ACCUM_PLAN = {"dA": mm_parts(2), "dP": mm_parts(3), "dkR": mm_parts(2), "dqs": mm_parts(3),
                   "dKd": mm_parts(3), "TR": mm_parts(2), "PdO": mm_parts(3), "TdVn": mm_parts(2)}


def bwd_head_fp32(q, k, v, g, beta, S0, dO, dST, scale, C=64, prods=None):
    """dq, dk, dv, dg, dbeta, dS0 of one head with float32 products.  Entry
    states come from the fp64 chunked forward.  `prods` may replace the
    products of two float32 operands (keys dA, dP, dkR, dqs, dKd, TR, PdO,
    TdVn) by other roundings, such as BF16_ACCUM_PLAN."""
    pr = dict(prods or {})
    mmx = lambda name, a, b: pr.get(name, _mm)(a, b)
    T, Dk = q.shape
    Dv = v.shape[1]
    starts = []
    S = np.array(S0, dtype=np.float64, copy=True)
    for s in range(0, T, C):
        starts.append(S)
        _, S, _ = ch.gdn_chunk_head(q[s:s + C], k[s:s + C], v[s:s + C], g[s:s + C], beta[s:s + C], S, scale, C)
    dq, dk = np.zeros((T, Dk)), np.zeros((T, Dk))
    dv, dg, db = np.zeros((T, Dv)), np.zeros(T), np.zeros(T)
    dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    for ci in range(len(starts) - 1, -1, -1):
        s, e = ci * C, min(ci * C + C, T)
        S = starts[ci].astype(np.float32).astype(np.float64)
        Q, K, V, bc, dOc = q[s:e], k[s:e], v[s:e], beta[s:e], dO[s:e]
        n = e - s
        G = np.cumsum(g[s:e])
        gam = np.exp(G)
        D = np.exp(np.where(np.tril(np.ones((n, n), bool)), G[:, None] - G[None, :], -np.inf))
        KK = _mm(K, K.T)
        A = np.tril(bc[:, None] * KK * D, -1)
        Tm = ch._tri_inverse(A).astype(np.float32).astype(np.float64)   # T in fp32, as stored
        TmI = Tm - np.eye(n)
        KS = _mm(K, S)
        R = bc[:, None] * (V - gam[:, None] * KS)
        Vn = R + mmx('TR', TmI, R)
        P = _mm(Q, K.T) * D
        dec = np.exp(G[-1] - G)
        # reverse mode through the chunk, dS the gradient of the state leaving it
        dVn = scale * mmx('PdO', P.T, dOc) + dec[:, None] * _mm(K, dS)
        dR = dVn + mmx('TdVn', TmI.T, dVn)
        dA = -np.tril(mmx('dA', dR, Vn.T), -1)
        dP = scale * np.tril(mmx('dP', dOc, Vn.T))
        dS_in = gam[-1] * dS + scale * _mm((gam[:, None] * Q).T, dOc) - _mm(((bc * gam)[:, None] * K).T, dR)
        dG = np.zeros(n)
        dv[s:e] = bc[:, None] * dR
        db[s:e] += np.sum(dR * (V - gam[:, None] * KS), axis=1)
        dk[s:e] -= (bc * gam)[:, None] * mmx('dkR', dR, S.T)
        dG -= bc * gam * np.sum(dR * KS, axis=1)
        dAs = dA * D
        db[s:e] += np.sum(dAs * KK, axis=1)
        dk[s:e] += bc[:, None] * _mm(dAs, K) + _mm(dAs.T, bc[:, None] * K)
        dAA = dA * A
        dG += dAA.sum(axis=1) - dAA.sum(axis=0)
        dPs = dP * D
        dq[s:e] += _mm(dPs, K)
        dk[s:e] += _mm(dPs.T, Q)
        dPP = dP * P
        dG += dPP.sum(axis=1) - dPP.sum(axis=0)
        dq[s:e] += scale * gam[:, None] * mmx('dqs', dOc, S.T)
        dG += scale * gam * np.sum(dOc * _mm(Q, S), axis=1)
        dG[-1] += gam[-1] * np.sum(dS * S)
        dKd = mmx('dKd', Vn, dS.T)
        dk[s:e] += dec[:, None] * dKd
        t = np.sum(dKd * K * dec[:, None], axis=1)
        dG[-1] += t.sum()
        dG -= t
        dg[s:e] = np.cumsum(dG[::-1])[::-1]
        dS = dS_in
    return dq, dk, dv, dg, db, dS


def per_head_errors(x, do, dht, prods=None):
    """[heads, 6] of max|diff| / rms (dq, dk, dv, dg, dbeta, dh0) for every
    (batch, head) of generator output x against the fp64 chunked oracle."""
    B, T, H = x["g"].shape
    out = []
    for b in range(B):
        for h in range(H):
            args = [x[n + "_f64"][b, :, h] for n in ("q", "k", "v", "g", "beta")]
            S0 = x["h0_f64"][b, h] if x["h0_f64"] is not None else np.zeros((args[0].shape[1], args[2].shape[1]))
            dST = None if dht is None else dht[b, h]
            ref = ch.gdn_chunk_bwd_head(*args, S0, do[b, :, h], dST, x["scale"])
            got = bwd_head_fp32(*args, S0, do[b, :, h], dST, x["scale"], prods=prods)
            out.append([float(np.abs(a - r).max() / max(np.sqrt(np.mean(r * r)), 1e-300)) for a, r in zip(got, ref)])
    return np.array(out)


_WORKLOAD = {}


def _layer_workload():
    """The full-size backward test's inputs (tests/test_parity_bwd.py), once per process."""
    if not _WORKLOAD:
        import gdn_inputs as gi
        x = gi.gdn_inputs(8, 4096, 8, 128, 128, seed=643, dtype="bf16", h0=True)
        rng = np.random.default_rng(643 + 7)
        _WORKLOAD["x"] = x
        _WORKLOAD["do"] = rng.standard_normal((8, 4096, 8, 128)).astype(np.float32).astype(np.float64)
        _WORKLOAD["dht"] = rng.standard_normal((8, 8, 128, 128)).astype(np.float32).astype(np.float64)
    return _WORKLOAD["x"], _WORKLOAD["do"], _WORKLOAD["dht"]


def _one(args):
    b, h, plan = args
    x, do, dht = _layer_workload()
    sub = {n: x[n][b:b + 1, :, h:h + 1] for n in x if n.endswith("_f64") and x[n] is not None and x[n].ndim >= 3
           and n != "h0_f64"}
    sub["h0_f64"] = x["h0_f64"][b:b + 1, h:h + 1]
    sub["g"] = x["g"][b:b + 1, :, h:h + 1]
    sub["scale"] = x["scale"]
    return per_head_errors(sub, do[b:b + 1, :, h:h + 1], dht[b:b + 1, h:h + 1],
                           prods=BF16_ACCUM_PLAN if plan else None)[0]


if __name__ == "__main__":
    import multiprocessing as mp
    import sys
    plan = "--plan" in sys.argv[1:]
    with mp.Pool(8) as pool:
        errs = np.array(pool.map(_one, [(b, h, plan) for b in range(8) for h in range(8)]))
    for i, name in enumerate(("dq", "dk", "dv", "dg", "dbeta", "dh0")):
        print(f"{name}: worst head {errs[:, i].max():.2e}, median {np.median(errs[:, i]):.2e}")
