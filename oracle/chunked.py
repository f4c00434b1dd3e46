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


def gdn_chunk_bwd_head(q, k, v, g, beta, S0, dO, dST, scale, C=64):
    """Backward of gdn_chunk_head for one head (the chunk equations above,
    differentiated in reverse chunk order).  dO [T,Dv], dST [Dk,Dv] or None.
    Returns dq, dk [T,Dk], dv [T,Dv], dg, dbeta [T], dS0 [Dk,Dv].

    Per chunk with entry state S (from a forward pass), D_ij = exp(G_i - G_j)
    for j <= i, Kd_j = k_j exp(G_C - G_j), R = diag(beta) (V - diag(gamma) K S),
    Vnew = T R, O = scale (diag(gamma) Q S + P Vnew), S' = gamma_C S + Kd^T Vnew,
    and dS' the gradient of the state leaving the chunk:
        dVnew = scale P^T dO + Kd dS'        dR = T^T dVnew
        dA    = -strict_lower(dR Vnew^T)     dP = scale lower(dO Vnew^T)
        dS    = gamma_C dS' + scale (diag(gamma) Q)^T dO - (diag(beta gamma) K)^T dR
    then the chain rule through A_ij = beta_i (k_i.k_j) D_ij, P_ij = (q_i.k_j) D_ij,
    R, the state term of O, and Kd gives dq, dk, dv, dbeta and dG; dg is the
    reverse cumulative sum of dG within the chunk."""
    T = q.shape[0]
    Dk, Dv = q.shape[1], v.shape[1]
    # forward: entry states of the chunks
    starts = []
    S = np.array(S0, dtype=np.float64, copy=True)
    for s in range(0, T, C):
        starts.append(S)
        _, S, _ = gdn_chunk_head(q[s:s + C], k[s:s + C], v[s:s + C], g[s:s + C], beta[s:s + C], S, scale, C)
    dq = np.zeros((T, Dk))
    dk = np.zeros((T, Dk))
    dv = np.zeros((T, Dv))
    dg = np.zeros(T)
    db = np.zeros(T)
    dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    for ci in range(len(starts) - 1, -1, -1):
        s = ci * C
        e = min(s + C, T)
        S = starts[ci]
        Q, K, V, gc, bc, dOc = q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], dO[s:e]
        n = e - s
        G = np.cumsum(gc)
        gamma = np.exp(G)
        lower_incl = np.tril(np.ones((n, n), dtype=bool))
        D = np.exp(np.where(lower_incl, G[:, None] - G[None, :], -np.inf))
        KK = K @ K.T
        A = np.tril(bc[:, None] * KK * D, -1)
        Tm = _tri_inverse(A)
        KS = K @ S
        R = bc[:, None] * (V - gamma[:, None] * KS)
        Vn = Tm @ R
        P = (Q @ K.T) * D
        dec = np.exp(G[-1] - G)
        Kd = K * dec[:, None]
        dSp = dS                                          # gradient of the state leaving the chunk
        dVn = scale * P.T @ dOc + Kd @ dSp
        dR = Tm.T @ dVn
        dA = -np.tril(dR @ Vn.T, -1)
        dP = scale * np.tril(dOc @ Vn.T)
        dS = gamma[-1] * dSp + scale * (gamma[:, None] * Q).T @ dOc - ((bc * gamma)[:, None] * K).T @ dR
        dG = np.zeros(n)
        # R = diag(beta) (V - diag(gamma) K S)
        dv[s:e] = bc[:, None] * dR
        db[s:e] += np.sum(dR * (V - gamma[:, None] * KS), axis=1)
        dk[s:e] += -(bc * gamma)[:, None] * (dR @ S.T)
        dG += -bc * gamma * np.sum(dR * KS, axis=1)
        # A_ij = beta_i (k_i.k_j) D_ij, strictly lower
        dAs = dA * D
        db[s:e] += np.sum(dAs * KK, axis=1)
        dk[s:e] += bc[:, None] * (dAs @ K) + dAs.T @ (bc[:, None] * K)
        dAA = dA * A
        dG += np.sum(dAA, axis=1) - np.sum(dAA, axis=0)
        # P_ij = (q_i.k_j) D_ij, lower incl. diagonal
        dPs = dP * D
        dq[s:e] += dPs @ K
        dk[s:e] += dPs.T @ Q
        dPP = dP * P
        dG += np.sum(dPP, axis=1) - np.sum(dPP, axis=0)
        # state term of O: scale diag(gamma) Q S
        QS = Q @ S
        dq[s:e] += scale * gamma[:, None] * (dOc @ S.T)
        dG += scale * gamma * np.sum(dOc * QS, axis=1)
        # S' = gamma_C S + Kd^T Vn
        dG[-1] += gamma[-1] * np.sum(dSp * S)
        dKd = Vn @ dSp.T
        dk[s:e] += dec[:, None] * dKd
        t = np.sum(dKd * Kd, axis=1)
        dG[-1] += np.sum(t)
        dG -= t
        # G_i = sum_{s<=i} g_s within the chunk
        dg[s:e] = np.cumsum(dG[::-1])[::-1]
    return dq, dk, dv, dg, db, dS


def gdn_chunk_bwd(q, k, v, g, beta, h0, dO, dST=None, scale=None, C=64):
    """All heads, [B,T,H,D] layout.  Returns dq, dk, dv, dg, dbeta, dh0."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    dq = np.zeros((B, T, H, Dk)); dk = np.zeros((B, T, H, Dk)); dv = np.zeros((B, T, H, Dv))
    dg = np.zeros((B, T, H)); db = np.zeros((B, T, H)); dh0 = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S0 = np.zeros((Dk, Dv)) if h0 is None else h0[b, h]
            r = gdn_chunk_bwd_head(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], beta[b, :, h], S0, dO[b, :, h],
                                   None if dST is None else dST[b, h], scale, C)
            dq[b, :, h], dk[b, :, h], dv[b, :, h], dg[b, :, h], db[b, :, h], dh0[b, h] = r
    return dq, dk, dv, dg, db, dh0


def gdn2_chunk_bwd_head(q, k, v, log_alpha, bgate, wgate, S0, dO, dST, scale, C=64):
    """Backward of gdn2_chunk_head for one head (the GDN-2 chunk equations,
    differentiated in reverse chunk order).  Returns dq, dk, dv, dlog_alpha,
    db, dw and dS0.

    Per chunk with entry state S, per-channel cumulative log-decay G_i (n x Dk),
    Gam = exp(G), D_ijc = exp(G_ic - G_jc) for j <= i, E = b . k, Z = w . v:
        A_ij = sum_c E_ic K_jc D_ijc (i > j),  T = (I + A)^-1
        Ehat = Gam . E,  R = Z - Ehat S,  Dl = T R
        P_ij = sum_c Q_ic K_jc D_ijc (j <= i),  Qhat = Gam . Q
        O = scale (Qhat S + P Dl)
        Khat_j = K_j . exp(G_last - G_j),  S' = Gam_last . S + Khat^T Dl
    With dS' the gradient of the state leaving the chunk:
        dDl = scale P^T dO + Khat dS'        dR = T^T dDl     dZ = dR
        dEhat = -dR S^T                      dA = -strict_lower(dR Dl^T)
        dP = scale lower(dO Dl^T)            dQhat = scale dO S^T
        dKhat = Dl dS'^T
        dS = Gam_last . dS' + scale Qhat^T dO - Ehat^T dR
    then the chain rule through Ehat, Qhat, A, P, Khat and the Gam_last . S
    term gives dq, dk, dE and dG; db = dE . k, dk += dE . b, dw = dZ . v,
    dv = dZ . w, and dlog_alpha is the reverse cumulative sum of dG within
    the chunk."""
    T = q.shape[0]
    Dk, Dv = q.shape[1], v.shape[1]
    starts = []
    S = np.array(S0, dtype=np.float64, copy=True)
    for s in range(0, T, C):
        starts.append(S)
        _, S, _ = gdn2_chunk_head(q[s:s + C], k[s:s + C], v[s:s + C], log_alpha[s:s + C], bgate[s:s + C],
                                  wgate[s:s + C], S, scale, C)
    dq = np.zeros((T, Dk)); dk = np.zeros((T, Dk)); dla = np.zeros((T, Dk)); db = np.zeros((T, Dk))
    dv = np.zeros((T, Dv)); dw = np.zeros((T, Dv))
    dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    for ci in range(len(starts) - 1, -1, -1):
        s = ci * C
        e = min(s + C, T)
        S = starts[ci]
        Q, K, V, Bg, Wg, dOc = q[s:e], k[s:e], v[s:e], bgate[s:e], wgate[s:e], dO[s:e]
        n = e - s
        G = np.cumsum(log_alpha[s:e], axis=0)
        Gam = np.exp(G)
        E = Bg * K
        Z = Wg * V
        lower_incl = np.tril(np.ones((n, n), dtype=bool))
        D3 = np.exp(np.where(lower_incl[:, :, None], G[:, None, :] - G[None, :, :], -np.inf))
        A = np.tril(np.einsum("ic,jc,ijc->ij", E, K, D3), -1)
        Tm = _tri_inverse(A)
        Eh = Gam * E
        R = Z - Eh @ S
        Dl = Tm @ R
        P = np.einsum("ic,jc,ijc->ij", Q, K, D3)
        Qh = Gam * Q
        dec = np.exp(G[-1][None, :] - G)
        Kh = K * dec
        dSp = dS
        dDl = scale * P.T @ dOc + Kh @ dSp
        dR = Tm.T @ dDl
        dEh = -dR @ S.T
        dA = -np.tril(dR @ Dl.T, -1)
        dP = scale * np.tril(dOc @ Dl.T)
        dQh = scale * dOc @ S.T
        dKh = Dl @ dSp.T
        dS = Gam[-1][:, None] * dSp + scale * Qh.T @ dOc - Eh.T @ dR
        dG = np.zeros((n, Dk))
        dE = np.zeros((n, Dk))
        dKc = np.zeros((n, Dk))
        dQc = np.zeros((n, Dk))
        # Z = w . v
        dw[s:e] = dR * V
        dv[s:e] = dR * Wg
        # Ehat = Gam . E and Qhat = Gam . Q
        dE += Gam * dEh
        dG += Gam * E * dEh
        dQc += Gam * dQh
        dG += Gam * Q * dQh
        # A_ij = sum_c E_ic K_jc D_ijc, strictly lower
        dE += np.einsum("ij,jc,ijc->ic", dA, K, D3)
        dKc += np.einsum("ij,ic,ijc->jc", dA, E, D3)
        tA = dA[:, :, None] * E[:, None, :] * K[None, :, :] * D3
        dG += tA.sum(axis=1) - tA.sum(axis=0)
        # P_ij = sum_c Q_ic K_jc D_ijc, lower incl. diagonal
        dQc += np.einsum("ij,jc,ijc->ic", dP, K, D3)
        dKc += np.einsum("ij,ic,ijc->jc", dP, Q, D3)
        tP = dP[:, :, None] * Q[:, None, :] * K[None, :, :] * D3
        dG += tP.sum(axis=1) - tP.sum(axis=0)
        # Khat_j = K_j exp(G_last - G_j) and the Gam_last . S term of S'
        dKc += dec * dKh
        t = dKh * Kh
        dG -= t
        dG[-1] += t.sum(axis=0) + Gam[-1] * np.sum(dSp * S, axis=1)
        # E = b . k
        db[s:e] = dE * K
        dKc += dE * Bg
        dq[s:e] = dQc
        dk[s:e] = dKc
        dla[s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dv, dla, db, dw, dS


def gdn2_chunk_bwd(q, k, v, log_alpha, b, w, h0, dO, dST=None, scale=None, C=64):
    """All heads, [B,T,H,D] layout.  Returns dq, dk, dv, dlog_alpha, db, dw, dh0."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    out = [np.zeros((B, T, H, d)) for d in (Dk, Dk, Dv, Dk, Dk, Dv)] + [np.zeros((B, H, Dk, Dv))]
    for bb in range(B):
        for h in range(H):
            S0 = np.zeros((Dk, Dv)) if h0 is None else h0[bb, h]
            r = gdn2_chunk_bwd_head(q[bb, :, h], k[bb, :, h], v[bb, :, h], log_alpha[bb, :, h], b[bb, :, h],
                                    w[bb, :, h], S0, dO[bb, :, h], None if dST is None else dST[bb, h], scale, C)
            for i in range(6):
                out[i][bb, :, h] = r[i]
            out[6][bb, h] = r[6]
    return tuple(out)
