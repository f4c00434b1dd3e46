"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Each test checks the oracle (C recurrence) or the second CPU formulation
(numpy chunked WY form) against something other than itself: hand-worked
fractions, the matrix form of the recurrence as the pages print it, closed
forms of special cases, invariants, and the other formulation.  Chosen so
that a dropped term, a wrong sign, an off-by-one in the causal mask, a
transposed state or a swapped gate fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(B, T, H, Dk, Dv, seed, h0=True, g_scale=1.0):
    rng = np.random.default_rng(seed)
    nrm = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = nrm(rng.standard_normal((B, T, H, Dk)))
    k = nrm(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    g = -g_scale * np.logaddexp(0, rng.standard_normal((B, T, H)))
    S0 = 0.3 * rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, S0


def _rand2(B, T, H, Dk, Dv, seed, h0=True):
    rng = np.random.default_rng(seed)
    nrm = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = nrm(rng.standard_normal((B, T, H, Dk)))
    k = nrm(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    la = -np.logaddexp(0, rng.standard_normal((B, T, H, Dk)))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, Dv))))
    S0 = 0.3 * rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, la, b, w, S0


# ---------------------------------------------------------------- hand-worked


def test_hand_worked_gdn():
    ex = json.load(open(GOLDEN))["gdn_T2_d2"]
    a = lambda n: np.array(ex[n], dtype=np.float64)
    o, S = oracle.gdn_fwd(a("q"), a("k"), a("v"), np.log(a("g_exp")), a("beta"), a("h0"),
                          scale=ex["scale"])
    np.testing.assert_allclose(o, a("o"), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S, a("S"), rtol=0, atol=1e-14)


def test_hand_worked_gdn2():
    ex = json.load(open(GOLDEN))["gdn2_T1_d2"]
    a = lambda n: np.array(ex[n], dtype=np.float64)
    o, S = oracle.gdn2_fwd(a("q"), a("k"), a("v"), np.log(a("alpha")), a("b"), a("w"), a("h0"),
                           scale=ex["scale"])
    np.testing.assert_allclose(o, a("o"), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S, a("S"), rtol=0, atol=1e-14)


def test_hand_worked_chunked_forms():
    ex = json.load(open(GOLDEN))["gdn_T2_d2"]
    a = lambda n: np.array(ex[n], dtype=np.float64)
    o, S = chunked.gdn_chunk_fwd(a("q"), a("k"), a("v"), np.log(a("g_exp")), a("beta"), a("h0"),
                                 scale=ex["scale"], C=2)
    np.testing.assert_allclose(o, a("o"), atol=1e-14)
    np.testing.assert_allclose(S, a("S"), atol=1e-14)
    ex = json.load(open(GOLDEN))["gdn2_T1_d2"]
    o, S = chunked.gdn2_chunk_fwd(a("q"), a("k"), a("v"), np.log(a("alpha")), a("b"), a("w"),
                                  a("h0"), scale=ex["scale"])
    np.testing.assert_allclose(o, a("o"), atol=1e-14)
    np.testing.assert_allclose(S, a("S"), atol=1e-14)


# -------------------------------------------------- matrix form of the pages


def test_matrix_form_gdn():
    """S_t = (I - beta k k^T) exp(g) S_{t-1} + beta k v^T, built as explicit
    d_k x d_k matrices (the page's matrix form), against the loop oracle."""
    q, k, v, g, beta, S0 = _rand(1, 9, 1, 5, 3, 1)
    S = S0[0, 0].copy()
    o_ref = np.zeros((9, 3))
    for t in range(9):
        kt = k[0, t, 0][:, None]
        M = np.eye(5) - beta[0, t, 0] * (kt @ kt.T)
        S = M @ (np.exp(g[0, t, 0]) * S) + beta[0, t, 0] * kt @ v[0, t, 0][None, :]
        o_ref[t] = 0.7 * (S.T @ q[0, t, 0])
    o, Sf = oracle.gdn_fwd(q, k, v, g, beta, S0, scale=0.7)
    np.testing.assert_allclose(o[0, :, 0], o_ref, atol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], S, atol=1e-13)


def test_matrix_form_gdn2():
    q, k, v, la, b, w, S0 = _rand2(1, 9, 1, 5, 3, 2)
    S = S0[0, 0].copy()
    o_ref = np.zeros((9, 3))
    for t in range(9):
        kt = k[0, t, 0][:, None]
        et = (b[0, t, 0] * k[0, t, 0])[:, None]
        S = (np.eye(5) - kt @ et.T) @ np.diag(np.exp(la[0, t, 0])) @ S + kt @ (w[0, t, 0] * v[0, t, 0])[None, :]
        o_ref[t] = 0.5 * (S.T @ q[0, t, 0])
    o, Sf = oracle.gdn2_fwd(q, k, v, la, b, w, S0, scale=0.5)
    np.testing.assert_allclose(o[0, :, 0], o_ref, atol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], S, atol=1e-13)


# ------------------------------------------------------------- special cases


def test_beta0_g0_leaves_state():
    q, k, v, g, beta, S0 = _rand(2, 17, 3, 8, 6, 3)
    o, S = oracle.gdn_fwd(q, k, v, 0 * g, 0 * beta, S0, scale=0.25)
    np.testing.assert_allclose(S, S0, atol=0)
    o_ref = 0.25 * np.einsum("bthk,bhkv->bthv", q, S0)
    np.testing.assert_allclose(o, o_ref, atol=1e-14)


def test_beta0_pure_decay_closed_form():
    q, k, v, g, beta, S0 = _rand(1, 12, 2, 4, 5, 4)
    o, S = oracle.gdn_fwd(q, k, v, g, 0 * beta, S0, scale=1.0)
    G = np.cumsum(g, axis=1)                                   # [B,T,H]
    o_ref = np.exp(G)[..., None] * np.einsum("bthk,bhkv->bthv", q, S0)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(S, np.exp(G[:, -1])[..., None, None] * S0, atol=1e-13)


@pytest.mark.parametrize("gp", [-np.inf, -800.0])
def test_reset_token_restarts_memory(gp):
    """exp(g_p) = 0 wipes the state: from token p on, outputs equal a fresh run
    with zero initial state that starts at p."""
    q, k, v, g, beta, S0 = _rand(1, 20, 2, 6, 4, 5)
    p = 7
    g = g.copy()
    g[:, p] = gp
    o, S = oracle.gdn_fwd(q, k, v, g, beta, S0)
    o2, S2 = oracle.gdn_fwd(q[:, p:], k[:, p:], v[:, p:], g[:, p:], beta[:, p:], None)
    np.testing.assert_allclose(o[:, p:], o2, atol=1e-13)
    np.testing.assert_allclose(S, S2, atol=1e-13)


def test_beta1_unit_key_writes_exactly():
    """beta = 1 and |k| = 1: the key reads back exactly the value just written,
    k_t^T S_t = v_t^T, because k^T (I - k k^T) = 0."""
    q, k, v, g, beta, S0 = _rand(1, 6, 2, 7, 5, 6)
    for T in range(1, 7):
        _, S = oracle.gdn_fwd(q[:, :T], k[:, :T], v[:, :T], g[:, :T], np.ones_like(beta[:, :T]), S0)
        kS = np.einsum("bhk,bhkv->bhv", k[:, T - 1], S)
        np.testing.assert_allclose(kS, v[:, T - 1], atol=1e-12)


def test_gdn2_b1_unit_key_writes_gated_value():
    q, k, v, la, b, w, S0 = _rand2(1, 5, 2, 7, 5, 7)
    _, S = oracle.gdn2_fwd(q, k, v, la, np.ones_like(b), w, S0)
    kS = np.einsum("bhk,bhkv->bhv", k[:, -1], S)
    np.testing.assert_allclose(kS, w[:, -1] * v[:, -1], atol=1e-12)


def test_single_token_closed_form():
    q, k, v, g, beta, _ = _rand(2, 1, 3, 8, 4, 8)
    o, S = oracle.gdn_fwd(q, k, v, g, beta, None, scale=0.3)
    qk = np.sum(q * k, -1)                                     # [B,1,H]
    np.testing.assert_allclose(o, 0.3 * (beta * qk)[..., None] * v, atol=1e-14)
    np.testing.assert_allclose(S, beta[:, 0, :, None, None] * k[:, 0, :, :, None] * v[:, 0, :, None, :],
                               atol=1e-14)


def test_two_token_hand_expansion():
    """T = 2, h0 = 0:  S1 = b1 k1 v1^T;  u2 = b2 (v2 - e^{g2} (k1.k2) b1 v1);
    S2 = e^{g2} S1 + k2 u2^T;  o2 = e^{g2} b1 (q2.k1) v1 + (q2.k2) u2."""
    q, k, v, g, beta, _ = _rand(1, 2, 1, 6, 3, 9)
    o, S = oracle.gdn_fwd(q, k, v, g, beta, None, scale=1.0)
    q1, q2 = q[0, :, 0]
    k1, k2 = k[0, :, 0]
    v1, v2 = v[0, :, 0]
    b1, b2 = beta[0, :, 0]
    a2 = np.exp(g[0, 1, 0])
    u2 = b2 * (v2 - a2 * (k1 @ k2) * b1 * v1)
    np.testing.assert_allclose(o[0, 1, 0], a2 * b1 * (q2 @ k1) * v1 + (q2 @ k2) * u2, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], a2 * b1 * np.outer(k1, v1) + np.outer(k2, u2), atol=1e-14)


def test_one_hot_keys_are_scalar_emas():
    """k_t = e_{c_t}: each state row is an independent gated EMA.  The hit row
    follows s <- e^{g}(1-beta) s + beta v; the others s <- e^{g} s.  This pins
    the orientation of S (key rows, value columns)."""
    rng = np.random.default_rng(10)
    T, Dk, Dv = 30, 4, 3
    c = rng.integers(0, Dk, size=T)
    k = np.zeros((1, T, 1, Dk))
    k[0, np.arange(T), 0, c] = 1.0
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    beta = rng.uniform(0, 1, (1, T, 1))
    g = -rng.uniform(0, 2, (1, T, 1))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    o, S = oracle.gdn_fwd(q, k, v, g, beta, S0, scale=1.0)
    s = S0[0, 0].copy()
    for t in range(T):
        s *= np.exp(g[0, t, 0])
        s[c[t]] = (1 - beta[0, t, 0]) * s[c[t]] + beta[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], s.T @ q[0, t, 0], atol=1e-13)
    np.testing.assert_allclose(S[0, 0], s, atol=1e-13)


def test_gdn2_one_hot_keys_are_channel_emas():
    """GDN-2 with one-hot keys: hit row s <- alpha_c (1 - b_c) s + w . v, other
    rows s <- alpha_r s.  Pins that Diag(alpha) and b act on key rows and w on
    value columns."""
    rng = np.random.default_rng(11)
    T, Dk, Dv = 25, 5, 3
    c = rng.integers(0, Dk, size=T)
    k = np.zeros((1, T, 1, Dk))
    k[0, np.arange(T), 0, c] = 1.0
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    la = -rng.uniform(0, 1, (1, T, 1, Dk))
    b = rng.uniform(0, 1, (1, T, 1, Dk))
    w = rng.uniform(0, 1, (1, T, 1, Dv))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    o, S = oracle.gdn2_fwd(q, k, v, la, b, w, S0, scale=1.0)
    s = S0[0, 0].copy()
    for t in range(T):
        s = np.exp(la[0, t, 0])[:, None] * s
        r = c[t]
        s[r] = (1 - b[0, t, 0, r]) * s[r] + w[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], s.T @ q[0, t, 0], atol=1e-13)
    np.testing.assert_allclose(S[0, 0], s, atol=1e-13)


def test_gdn2_tied_gates_collapse_to_gdn():
    """b = w = beta * 1 and log alpha = g * 1 recover Gated DeltaNet
    (Gated DeltaNet-2 article, 7minutos.es, section 'Regla-2 del Delta cerrado')."""
    q, k, v, g, beta, S0 = _rand(2, 23, 2, 6, 5, 12)
    Dk, Dv = 6, 5
    o1, S1 = oracle.gdn_fwd(q, k, v, g, beta, S0)
    o2, S2 = oracle.gdn2_fwd(q, k, v, np.repeat(g[..., None], Dk, -1),
                             np.repeat(beta[..., None], Dk, -1), np.repeat(beta[..., None], Dv, -1), S0)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(S2, S1, atol=1e-13)


# -------------------------------------------------------- structural checks


@pytest.mark.parametrize("C", [1, 2, 5, 16, 64])
def test_chunked_form_equals_recurrence(C):
    q, k, v, g, beta, S0 = _rand(2, 37, 2, 8, 6, 13, g_scale=0.3)
    o1, S1 = oracle.gdn_fwd(q, k, v, g, beta, S0, scale=0.4)
    o2, S2 = chunked.gdn_chunk_fwd(q, k, v, g, beta, S0, scale=0.4, C=C)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(S2, S1, atol=1e-12)


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_gdn2_chunked_form_equals_recurrence(C):
    q, k, v, la, b, w, S0 = _rand2(1, 41, 2, 8, 6, 14)
    o1, S1 = oracle.gdn2_fwd(q, k, v, la, b, w, S0, scale=0.4)
    o2, S2 = chunked.gdn2_chunk_fwd(q, k, v, la, b, w, S0, scale=0.4, C=C)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(S2, S1, atol=1e-12)


def test_chunked_long_with_workload_gates():
    """Chunk form at BT = 64 over several chunks with the strong decays of the
    measured workloads (A ~ U(1,16)) and a ragged tail."""
    from gdn_inputs import gdn_inputs
    x = gdn_inputs(1, 200, 2, 16, 16, seed=77, dtype="fp32", h0=True)
    args = [x[n + "_f64"] for n in ("q", "k", "v", "g", "beta", "h0")]
    o1, S1 = oracle.gdn_fwd(*args)
    o2, S2 = chunked.gdn_chunk_fwd(*args, C=64)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(S2, S1, atol=1e-12)


def test_linearity_in_values_and_state():
    q, k, v, g, beta, S0 = _rand(1, 15, 2, 6, 4, 15)
    _, _, v2, _, _, S02 = _rand(1, 15, 2, 6, 4, 16)
    a, c = 0.7, -1.3
    o1, S1 = oracle.gdn_fwd(q, k, v, g, beta, S0)
    o2, S2 = oracle.gdn_fwd(q, k, v2, g, beta, S02)
    o3, S3 = oracle.gdn_fwd(q, k, a * v + c * v2, g, beta, a * S0 + c * S02)
    np.testing.assert_allclose(o3, a * o1 + c * o2, atol=1e-12)
    np.testing.assert_allclose(S3, a * S1 + c * S2, atol=1e-12)


def test_causality():
    q, k, v, g, beta, S0 = _rand(1, 40, 1, 6, 4, 17)
    o1, _ = oracle.gdn_fwd(q, k, v, g, beta, S0)
    t = 23
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    k2[:, t] = k2[:, t][..., ::-1]
    v2[:, t] += 1.0
    g2, b2 = g.copy(), beta.copy()
    g2[:, t] -= 0.5
    b2[:, t] = 0.9
    o2, _ = oracle.gdn_fwd(q2, k2, v2, g2, b2, S0)
    np.testing.assert_array_equal(o1[:, :t], o2[:, :t])
    assert np.abs(o1[:, t] - o2[:, t]).max() > 1e-3


def test_resume_split_equals_single_call():
    q, k, v, g, beta, S0 = _rand(2, 50, 2, 6, 5, 18)
    o, S = oracle.gdn_fwd(q, k, v, g, beta, S0)
    T1 = 21
    oa, Sa = oracle.gdn_fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
    ob, Sb = oracle.gdn_fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, atol=1e-14)
    np.testing.assert_allclose(Sb, S, atol=1e-14)


def test_step_equals_one_token_of_forward():
    q, k, v, g, beta, S0 = _rand(3, 1, 4, 8, 6, 19)
    o1, S1 = oracle.gdn_fwd(q, k, v, g, beta, S0, scale=0.35)
    o2, S2 = oracle.gdn_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, scale=0.35)
    np.testing.assert_allclose(o2, o1[:, 0], atol=1e-15)
    np.testing.assert_allclose(S2, S1, atol=1e-15)


def test_stability_bound():
    """|k| = 1, beta in [0,1], g <= 0: ||S_t||_2 <= e^{g_t} ||S_{t-1}||_2 + beta_t ||v_t||."""
    q, k, v, g, beta, S0 = _rand(1, 30, 1, 6, 5, 20, g_scale=0.05)
    prev = np.linalg.norm(S0[0, 0], 2)
    for t in range(30):
        _, S = oracle.gdn_fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1], beta[:, :t + 1], S0)
        cur = np.linalg.norm(S[0, 0], 2)
        assert cur <= np.exp(g[0, t, 0]) * prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12
        prev = cur


def test_chunk_intermediates_solve_the_triangular_system():
    """T = (I + A)^-1 is unit lower triangular and the new values satisfy
    (I + A) Delta = diag(beta) V - diag(beta gamma) K S0 (the derivation)."""
    q, k, v, g, beta, S0 = _rand(1, 64, 1, 8, 5, 21, g_scale=0.2)
    _, _, inter = chunked.gdn_chunk_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                                         S0[0, 0], 1.0, C=64, keep=True)
    it = inter[0]
    Tm = it["T"]
    np.testing.assert_allclose(np.triu(Tm, 1), 0, atol=0)
    np.testing.assert_allclose(np.diag(Tm), 1, atol=0)
    A = it["A"]
    gam = np.exp(np.cumsum(g[0, :, 0]))
    rhs = beta[0, :, 0, None] * v[0, :, 0] - (beta[0, :, 0] * gam)[:, None] * (k[0, :, 0] @ S0[0, 0])
    np.testing.assert_allclose((np.eye(64) + A) @ it["Vnew"], rhs, atol=1e-12)


# ------------------------------------------------------------- GDN-2 decode


def test_hand_worked_gdn2_step():
    """The hand-worked GDN-2 token (tests/golden) through the decode-step entry."""
    ex = json.load(open(GOLDEN))["gdn2_T1_d2"]
    a = lambda n: np.array(ex[n], dtype=np.float64)
    o, S = oracle.gdn2_step(a("q")[:, 0], a("k")[:, 0], a("v")[:, 0], np.log(a("alpha"))[:, 0], a("b")[:, 0],
                            a("w")[:, 0], a("h0"), scale=ex["scale"])
    np.testing.assert_allclose(o, a("o")[:, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S, a("S"), rtol=0, atol=1e-14)


def test_gdn2_step_tied_gates_is_gdn_step():
    """b = w = beta on every channel and log_alpha = g: one GDN-2 step is one
    Gated DeltaNet step (Gated DeltaNet-2 article, 'Regla-2 del Delta cerrado')."""
    q, k, v, g, beta, S0 = _rand(3, 1, 4, 8, 6, 21)
    Dk, Dv = q.shape[-1], v.shape[-1]
    o1, S1 = oracle.gdn_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, scale=0.3)
    o2, S2 = oracle.gdn2_step(q[:, 0], k[:, 0], v[:, 0], np.repeat(g[:, 0, :, None], Dk, -1),
                              np.repeat(beta[:, 0, :, None], Dk, -1), np.repeat(beta[:, 0, :, None], Dv, -1), S0,
                              scale=0.3)
    np.testing.assert_allclose(o2, o1, atol=1e-14)
    np.testing.assert_allclose(S2, S1, atol=1e-14)


def test_gdn2_steps_chain_to_forward():
    q, k, v, la, b, w, S0 = _rand2(2, 7, 3, 8, 6, 22, h0=True)
    o_f, S_f = oracle.gdn2_fwd(q, k, v, la, b, w, S0, scale=0.4)
    S = S0
    for t in range(q.shape[1]):
        o_t, S = oracle.gdn2_step(q[:, t], k[:, t], v[:, t], la[:, t], b[:, t], w[:, t], S, scale=0.4)
        np.testing.assert_allclose(o_t, o_f[:, t], atol=1e-13)
    np.testing.assert_allclose(S, S_f, atol=1e-13)
