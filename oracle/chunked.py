"""Chunked (WY-form) fp64 evaluation of the gated delta rule -- TEST INFRASTRUCTURE.

The pages say the forward runs in blocks of 64 tokens, turns the in-block
serial dependency into lower-triangular matrix work through the WY
representation, passes one state matrix between blocks, and scales the
cumulative gate by log2(e) so kernels can use exp2 (GatedDeltaNet
walkthrough, yfxerp.com, section "chunked parallel: how the Triton kernels
make the serial loop parallel"; Gated DeltaNet-2 article, 7minutos.es,
section on chunked training, block size C = 64).  They print no equations, so
the ones below are derived from the recurrence (written out in the design doc):

  Within a chunk with entry state S0, G_i = sum_{s<=i} g_s (chunk-local),
  gamma_i = exp(G_i), and delta_i the value actually written at token i:
      delta_i = beta_i v_i - beta_i gamma_i S0^T k_i
                - sum_{j<i} beta_i (k_i.k_j) exp(G_i - G_j) delta_j
  i.e. (I + A) Delta = diag(beta) V - diag(beta gamma) K S0 with
      A_ij = beta_i (k_i.k_j) exp(G_i - G_j)  (i > j, else 0),
      T = (I + A)^-1,  U = T diag(beta) V,  W = T diag(beta gamma) K,
      Delta = U - W S0                                   ("new values")
      O_i = scale * (gamma_i q_i^T S0 + sum_{j<=i} (q_i.k_j) exp(G_i - G_j) delta_j)
      S_end = gamma_C S0 + sum_j exp(G_C - G_j) k_j delta_j^T

  GDN-2 (per-key-channel log-decay G_{i,c}, e_i = b_i . k_i, z_i = w_i . v_i):
      A_ij = sum_c e_ic k_jc exp(G_ic - G_jc)  (i > j),   U = T Z,  W = T (Gamma . E)
      O_i = scale * ((Gamma_i . q_i)^T S0 + sum_{j<=i} P_ij delta_j),
            P_ij = sum_c q_ic k_jc exp(G_ic - G_jc)
      S_end = Diag(Gamma_C) S0 + sum_j (k_j . Gamma_C / Gamma_j) delta_j^T

Every decay is evaluated as exp of a non-positive difference.  Nothing here
is blocked or fused beyond the chunking itself; the triangular system is
solved with scipy's triangular solver.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

LOG2E = 1.4426950408889634


def _tri_inverse(A):
    n = A.shape[0]
    return solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)


def gdn_chunk_head(q, k, v, g, beta, S0, scale, C=64, keep=False):
    """One head: q,k [T,Dk], v [T,Dv], g,beta [T], S0 [Dk,Dv].
    Returns (o [T,Dv], S_final, intermediates or None)."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    inter = [] if keep else None
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, gc, bc = q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e]
        n = e - s
        G = np.cumsum(gc)
        gamma = np.exp(G)
        lower_incl = np.tril(np.ones((n, n), dtype=bool))
        diff = np.where(lower_incl, G[:, None] - G[None, :], -np.inf)
        D = np.exp(diff)
        A = np.tril(bc[:, None] * (K @ K.T) * D, -1)
        Tm = _tri_inverse(A)
        U = Tm @ (bc[:, None] * V)
        W = Tm @ ((bc * gamma)[:, None] * K)
        Vnew = U - W @ S
        P = (Q @ K.T) * D
        o[s:e] = scale * (gamma[:, None] * (Q @ S) + P @ Vnew)
        S_in = S
        S = gamma[-1] * S + (K * np.exp(G[-1] - G)[:, None]).T @ Vnew
        if keep:
            inter.append(dict(G=G, G2=G * LOG2E, A=A, T=Tm, U=U, W=W, Vnew=Vnew, P=P, S_in=S_in))
    return o, S, inter


def gdn_chunk_fwd(q, k, v, g, beta, h0=None, scale=None, C=64):
    """All heads, [B,T,H,D] layout.  Returns (o, S_final)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    o = np.zeros((B, T, H, Dv))
    S = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S0 = np.zeros((Dk, Dv)) if h0 is None else h0[b, h]
            o[b, :, h], S[b, h], _ = gdn_chunk_head(q[b, :, h], k[b, :, h], v[b, :, h],
                                                    g[b, :, h], beta[b, :, h], S0, scale, C)
    return o, S


def gdn2_chunk_head(q, k, v, log_alpha, bgate, wgate, S0, scale, C=64, keep=False):
    """One GDN-2 head: log_alpha, bgate [T,Dk], wgate [T,Dv]."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    inter = [] if keep else None
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V = q[s:e], k[s:e], v[s:e]
        n = e - s
        G = np.cumsum(log_alpha[s:e], axis=0)                  # [n, Dk]
        E = bgate[s:e] * K
        Z = wgate[s:e] * V
        lower_incl = np.tril(np.ones((n, n), dtype=bool))
        diff = np.where(lower_incl[:, :, None], G[:, None, :] - G[None, :, :], -np.inf)
        D = np.exp(diff)                                       # [n, n, Dk]
        A = np.tril(np.einsum("ic,jc,ijc->ij", E, K, D), -1)
        Tm = _tri_inverse(A)
        Gam = np.exp(G)
        U = Tm @ Z
        W = Tm @ (Gam * E)
        Vnew = U - W @ S
        P = np.einsum("ic,jc,ijc->ij", Q, K, D)
        o[s:e] = scale * ((Gam * Q) @ S + P @ Vnew)
        S_in = S
        S = Gam[-1][:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ Vnew
        if keep:
            inter.append(dict(G=G, G2=G * LOG2E, A=A, T=Tm, U=U, W=W, Vnew=Vnew, P=P, S_in=S_in))
    return o, S, inter


def gdn2_chunk_fwd(q, k, v, log_alpha, b, w, h0=None, scale=None, C=64):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    o = np.zeros((B, T, H, Dv))
    S = np.zeros((B, H, Dk, Dv))
    for bb in range(B):
        for h in range(H):
            S0 = np.zeros((Dk, Dv)) if h0 is None else h0[bb, h]
            o[bb, :, h], S[bb, h], _ = gdn2_chunk_head(
                q[bb, :, h], k[bb, :, h], v[bb, :, h], log_alpha[bb, :, h], b[bb, :, h],
                w[bb, :, h], S0, scale, C)
    return o, S
