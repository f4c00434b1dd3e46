"""Pins of the oracle's Gated DeltaNet-2 backward (gdn2_bwd): central finite
differences of the oracle's GDN-2 forward for L = sum(dO * o) + sum(dST * S_T)
at random entries of every input, across the 64-token recomputation
segments; and the collapse to Gated DeltaNet (tied gates make the GDN-2 map
the GDN map, so its gradients must reduce to the separately pinned GDN
backward)."""
import numpy as np
import pytest

import oracle


def _case(B, T, H, Dk, Dv, seed):
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s)
    x = dict(q=n(B, T, H, Dk), k=n(B, T, H, Dk) / np.sqrt(Dk), v=n(B, T, H, Dv),
             log_alpha=-np.log1p(np.exp(n(B, T, H, Dk))), b=1 / (1 + np.exp(-n(B, T, H, Dk))),
             w=1 / (1 + np.exp(-n(B, T, H, Dv))), h0=0.3 * n(B, H, Dk, Dv))
    return x, n(B, T, H, Dv), n(B, H, Dk, Dv)


NAMES = ("q", "k", "v", "log_alpha", "b", "w", "h0")


def _loss(x, dO, dST, scale):
    o, S = oracle.gdn2_fwd(*[x[nm] for nm in NAMES], scale=scale)
    return float(np.sum(dO * o) + (np.sum(dST * S) if dST is not None else 0.0))


@pytest.mark.parametrize("T", [1, 64, 65, 150])
def test_gdn2_gradients_match_finite_differences(T):
    x, dO, dST = _case(2, T, 2, 6, 5, seed=500 + T)
    scale = 0.7
    grads = oracle.gdn2_bwd(*[x[nm] for nm in NAMES], dO, dST, scale=scale)
    rng = np.random.default_rng(T)
    for name, gr in zip(NAMES, grads):
        base = x[name]
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in base.shape)
            hstep = 1e-5 * max(1.0, abs(base[idx]))
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += hstep
            xm[name][idx] -= hstep
            fd = (_loss(xp, dO, dST, scale) - _loss(xm, dO, dST, scale)) / (2 * hstep)
            assert abs(gr[idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, gr[idx], fd)


def test_gdn2_no_final_state_gradient_and_no_h0():
    x, dO, _ = _case(1, 70, 1, 4, 3, seed=510)
    x["h0"] = None
    grads = oracle.gdn2_bwd(*[x[nm] for nm in NAMES], dO, None, scale=0.5)
    assert grads[6] is None
    rng = np.random.default_rng(5)
    for name, gr in zip(NAMES[:6], grads[:6]):
        for _ in range(4):
            idx = tuple(rng.integers(0, s) for s in x[name].shape)
            xp = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xm = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xp[name][idx] += 1e-5
            xm[name][idx] -= 1e-5
            fd = (_loss(xp, dO, None, 0.5) - _loss(xm, dO, None, 0.5)) / 2e-5
            assert abs(gr[idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, gr[idx], fd)


def test_gdn2_backward_collapses_to_gdn_backward():
    """log_alpha = g 1, b = beta 1, w = beta 1: the GDN-2 map is the GDN map, so
    dq, dk, dv agree, dg = sum_c dlog_alpha_c and dbeta = sum_c db_c + sum_j dw_j."""
    rng = np.random.default_rng(520)
    B, T, H, Dk, Dv = 1, 90, 2, 5, 4
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    v = rng.standard_normal((B, T, H, Dv))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    h0 = 0.3 * rng.standard_normal((B, H, Dk, Dv))
    dO = rng.standard_normal((B, T, H, Dv))
    dST = rng.standard_normal((B, H, Dk, Dv))
    ref = oracle.gdn_bwd(q, k, v, g, beta, h0, dO, dST, scale=0.6)
    la = np.repeat(g[..., None], Dk, axis=-1)
    bb = np.repeat(beta[..., None], Dk, axis=-1)
    ww = np.repeat(beta[..., None], Dv, axis=-1)
    dq, dk, dv, dla, db, dw, dh0 = oracle.gdn2_bwd(q, k, v, la, bb, ww, h0, dO, dST, scale=0.6)
    np.testing.assert_allclose(dq, ref[0], atol=1e-12)
    np.testing.assert_allclose(dk, ref[1], atol=1e-12)
    np.testing.assert_allclose(dv, ref[2], atol=1e-12)
    np.testing.assert_allclose(dla.sum(-1), ref[3], atol=1e-12)
    np.testing.assert_allclose(db.sum(-1) + dw.sum(-1), ref[4], atol=1e-12)
    np.testing.assert_allclose(dh0, ref[5], atol=1e-12)


def pin_backward2_fd():
    """Entry for the mutant check (not collected): the T = 150 finite-difference pin."""
    test_gdn2_gradients_match_finite_differences(150)


@pytest.mark.parametrize("T,C", [(150, 64), (100, 16), (64, 64), (1, 64), (9, 1)])
def test_gdn2_chunked_backward_equals_recurrence_backward(T, C):
    """The chunked GDN-2 backward in oracle/chunked.py (the chunk equations the
    GPU backward follows) equals the per-token backward to rounding."""
    from oracle import chunked
    x, dO, dST = _case(2, T, 2, 6, 5, seed=530 + T)
    ref = oracle.gdn2_bwd(*[x[nm] for nm in NAMES], dO, dST, scale=0.8)
    got = chunked.gdn2_chunk_bwd(*[x[nm] for nm in NAMES], dO, dST, scale=0.8, C=C)
    for name, a, r in zip(("dq", "dk", "dv", "dla", "db", "dw", "dh0"), got, ref):
        np.testing.assert_allclose(a, r, atol=1e-10, rtol=1e-10, err_msg=name)
