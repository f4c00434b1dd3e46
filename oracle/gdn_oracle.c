/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is used by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg; the product path never
 * links, loads or calls it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (per independent (b, h) head, tokens t = 0..T-1):
 *
 *   Gated DeltaNet (GatedDeltaNet walkthrough, yfxerp.com, section "Delta
 *   Rule: predict first, then correct"; the recurrence and the per-token
 *   reference loop there):
 *       S <- exp(g_t) * S                       (gated forgetting of the whole state)
 *       u <- beta_t * (v_t - S^T k_t)           (prediction error, scaled by write strength)
 *       S <- S + k_t u^T                        (write only the correction)
 *       o_t <- scale * S^T q_t                  (read-out with the query, after the update)
 *   S is d_k x d_v (key rows, value columns).  The matrix form on that page,
 *   S_t = (I - beta k k^T) exp(g) S_{t-1} + beta k v^T, is the same map.
 *
 *   Gated DeltaNet-2 (NVIDIA AI lanza Gated DeltaNet-2, 7minutos.es, section
 *   "Regla-2 del Delta cerrado"):
 *       S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T
 *   evaluated as: decay rows by alpha (before the edit), predict with the
 *   erase-gated key, write the write-gated value minus the prediction:
 *       S <- Diag(exp(log_alpha_t)) S
 *       u <- w_t . v_t - S^T (b_t . k_t)
 *       S <- S + k_t u^T ;   o_t <- scale * S^T q_t
 *
 *   Decode steps: the Gated DeltaNet or Gated DeltaNet-2 body above once, with
 *   S given and updated in place (gdn_oracle_step, gdn2_oracle_step).
 *
 * Layouts (row-major, contiguous): q,k [B,T,H,Dk]; v [B,T,H,Dv];
 * g, beta [B,T,H]; log_alpha, b [B,T,H,Dk]; w [B,T,H,Dv];
 * h0, S [B,H,Dk,Dv]; o [B,T,H,Dv].  h0 may be NULL (zero initial state).
 * S_out may be NULL.  Heads run in parallel with OpenMP, one head per
 * iteration; within a head everything is sequential.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* One Gated DeltaNet token on one head's state S[Dk*Dv]. */
static void gdn_token(double *S, const double *q, const double *k, const double *v,
                      double g, double beta, double *u, double *o,
                      int Dk, int Dv, double scale) {
    const double decay = exp(g);
    for (int i = 0; i < Dk * Dv; ++i) S[i] *= decay;
    for (int j = 0; j < Dv; ++j) {
        double pred = 0.0;
        for (int i = 0; i < Dk; ++i) pred += S[i * Dv + j] * k[i];
        u[j] = beta * (v[j] - pred);
    }
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[i * Dv + j] += k[i] * u[j];
    if (o) {
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i) acc += S[i * Dv + j] * q[i];
            o[j] = scale * acc;
        }
    }
}

void gdn_oracle_fwd(const double *q, const double *k, const double *v,
                    const double *g, const double *beta, const double *h0,
                    double *o, double *S_out,
                    int B, int T, int H, int Dk, int Dv, double scale, int nthreads) {
    set_threads(nthreads);
    const long units = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long unit = 0; unit < units; ++unit) {
        const long b = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (h0) memcpy(S, h0 + unit * (long)Dk * Dv, sizeof(double) * (size_t)Dk * Dv);
        else memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        for (long t = 0; t < T; ++t) {
            const long th = (b * T + t) * H + h;        /* token-head index */
            gdn_token(S, q + th * Dk, k + th * Dk, v + th * Dv, g[th], beta[th], u,
                      o + th * Dv, Dk, Dv, scale);
        }
        if (S_out) memcpy(S_out + unit * (long)Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
        free(u);
    }
}

/* One Gated DeltaNet-2 token on a d_k x d_v state (row-major), in place;
 * u [Dv] and e [Dk] are scratch.  o (Dv values) may be NULL. */
static void gdn2_token(double *S, const double *qt, const double *kt, const double *vt,
                       const double *la, const double *bt, const double *wt, double *u, double *e,
                       double *ot, int Dk, int Dv, double scale) {
    /* decay each key row by its own channel rate, before the edit */
    for (int i = 0; i < Dk; ++i) {
        const double a = exp(la[i]);
        for (int j = 0; j < Dv; ++j) S[i * Dv + j] *= a;
        e[i] = bt[i] * kt[i];
    }
    for (int j = 0; j < Dv; ++j) {
        double pred = 0.0;
        for (int i = 0; i < Dk; ++i) pred += S[i * Dv + j] * e[i];
        u[j] = wt[j] * vt[j] - pred;
    }
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[i * Dv + j] += kt[i] * u[j];
    if (ot) {
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i) acc += S[i * Dv + j] * qt[i];
            ot[j] = scale * acc;
        }
    }
}

void gdn2_oracle_fwd(const double *q, const double *k, const double *v,
                     const double *log_alpha, const double *bgate, const double *wgate,
                     const double *h0, double *o, double *S_out,
                     int B, int T, int H, int Dk, int Dv, double scale, int nthreads) {
    set_threads(nthreads);
    const long units = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long unit = 0; unit < units; ++unit) {
        const long b = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (h0) memcpy(S, h0 + unit * (long)Dk * Dv, sizeof(double) * (size_t)Dk * Dv);
        else memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        for (long t = 0; t < T; ++t) {
            const long th = (b * T + t) * H + h;
            gdn2_token(S, q + th * Dk, k + th * Dk, v + th * Dv, log_alpha + th * Dk, bgate + th * Dk,
                       wgate + th * Dv, u, e, o + th * Dv, Dk, Dv, scale);
        }
        if (S_out) memcpy(S_out + unit * (long)Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
        free(u);
        free(e);
    }
}

/* Single-token decode step: q,k [B,H,Dk], v [B,H,Dv], g,beta [B,H], S [B,H,Dk,Dv] in/out. */
void gdn_oracle_step(const double *q, const double *k, const double *v,
                     const double *g, const double *beta, double *S, double *o,
                     int B, int H, int Dk, int Dv, double scale, int nthreads) {
    set_threads(nthreads);
    const long units = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long unit = 0; unit < units; ++unit) {
        double *u = (double *)malloc(sizeof(double) * (size_t)Dv);
        gdn_token(S + unit * (long)Dk * Dv, q + unit * Dk, k + unit * Dk, v + unit * Dv,
                  g[unit], beta[unit], u, o + unit * Dv, Dk, Dv, scale);
        free(u);
    }
}

/* Single-token Gated DeltaNet-2 decode step: q,k,log_alpha,b [B,H,Dk],
 * v,w [B,H,Dv], S [B,H,Dk,Dv] in/out. */
void gdn2_oracle_step(const double *q, const double *k, const double *v,
                      const double *log_alpha, const double *bgate, const double *wgate,
                      double *S, double *o, int B, int H, int Dk, int Dv, double scale, int nthreads) {
    set_threads(nthreads);
    const long units = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long unit = 0; unit < units; ++unit) {
        double *u = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)Dk);
        gdn2_token(S + unit * (long)Dk * Dv, q + unit * Dk, k + unit * Dk, v + unit * Dv, log_alpha + unit * Dk,
                   bgate + unit * Dk, wgate + unit * Dv, u, e, o + unit * Dv, Dk, Dv, scale);
        free(u);
        free(e);
    }
}

/*
 * Backward of the Gated DeltaNet forward: reverse-mode differentiation of the
 * per-token recurrence above for the loss L = sum(dO . o) + sum(dST . S_T).
 * Per token, with S' = exp(g) S_{t-1}, p = S'^T k, u = beta (v - p),
 * S_t = S' + k u^T, o = scale S_t^T q, and D the gradient of L w.r.t. S_t:
 *   D   += scale q do^T          dq    = scale S_t do
 *   dk   = D u                   du    = D^T k
 *   dbeta = du . (v - p)         dv    = beta du
 *   D'   = D - beta k du^T       dk   -= beta S' du
 *   dg    = <D', S'>             D     = exp(g) D'      (gradient w.r.t. S_{t-1})
 * and dh0 = D after the first token.  States are recomputed forward one
 * 64-token segment at a time from stored segment-start states.
 * dO [B,T,H,Dv]; dST [B,H,Dk,Dv] or NULL; outputs dq, dk [B,T,H,Dk],
 * dv [B,T,H,Dv], dg, dbeta [B,T,H], dh0 [B,H,Dk,Dv] or NULL.
 */
void gdn_oracle_bwd(const double *q, const double *k, const double *v, const double *g, const double *beta,
                    const double *h0, const double *dO, const double *dST, double *dq, double *dk, double *dv,
                    double *dg, double *dbeta, double *dh0, int B, int T, int H, int Dk, int Dv, double scale,
                    int nthreads) {
    set_threads(nthreads);
    const long units = (long)B * H;
    const int SEG = 64;
    const int nseg = (T + SEG - 1) / SEG;
    const size_t SS = (size_t)Dk * Dv;
#pragma omp parallel for schedule(static)
    for (long unit = 0; unit < units; ++unit) {
        const long b = unit / H, h = unit % H;
        double *starts = (double *)malloc(sizeof(double) * SS * (size_t)nseg);
        double *Sp = (double *)malloc(sizeof(double) * SS * (size_t)SEG);  /* S' of each token of a segment */
        double *us = (double *)malloc(sizeof(double) * (size_t)Dv * SEG);   /* u of each token */
        double *ps = (double *)malloc(sizeof(double) * (size_t)Dv * SEG);   /* p of each token */
        double *S = (double *)malloc(sizeof(double) * SS);
        double *St = (double *)malloc(sizeof(double) * SS);
        double *D = (double *)malloc(sizeof(double) * SS);
        double *du = (double *)malloc(sizeof(double) * (size_t)Dv);
        /* forward: segment-start states */
        if (h0) memcpy(S, h0 + unit * (long)SS, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (long t = 0; t < T; ++t) {
            if (t % SEG == 0) memcpy(starts + (size_t)(t / SEG) * SS, S, sizeof(double) * SS);
            const long th = (b * T + t) * H + h;
            gdn_token(S, q + th * Dk, k + th * Dk, v + th * Dv, g[th], beta[th], du, NULL, Dk, Dv, scale);
        }
        if (dST) memcpy(D, dST + unit * (long)SS, sizeof(double) * SS);
        else memset(D, 0, sizeof(double) * SS);
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const long t0 = (long)sg * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
            /* recompute S', p, u of the segment */
            memcpy(S, starts + (size_t)sg * SS, sizeof(double) * SS);
            for (long t = t0; t < t1; ++t) {
                const long th = (b * T + t) * H + h, x = t - t0;
                const double *kt = k + th * Dk, *vt = v + th * Dv;
                const double decay = exp(g[th]);
                double *spx = Sp + (size_t)x * SS;
                for (size_t i = 0; i < SS; ++i) spx[i] = S[i] * decay;
                for (int j = 0; j < Dv; ++j) {
                    double p = 0.0;
                    for (int i = 0; i < Dk; ++i) p += spx[i * Dv + j] * kt[i];
                    ps[(size_t)x * Dv + j] = p;
                    us[(size_t)x * Dv + j] = beta[th] * (vt[j] - p);
                }
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < Dv; ++j) S[i * Dv + j] = spx[i * Dv + j] + kt[i] * us[(size_t)x * Dv + j];
            }
            /* reverse through the segment */
            for (long t = t1 - 1; t >= t0; --t) {
                const long th = (b * T + t) * H + h, x = t - t0;
                const double *qt = q + th * Dk, *kt = k + th * Dk, *vt = v + th * Dv, *dot = dO + th * Dv;
                const double *spx = Sp + (size_t)x * SS, *ux = us + (size_t)x * Dv, *px = ps + (size_t)x * Dv;
                const double bt = beta[th];
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < Dv; ++j) St[i * Dv + j] = spx[i * Dv + j] + kt[i] * ux[j];
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < Dv; ++j) D[i * Dv + j] += scale * qt[i] * dot[j];
                double *dqt = dq + th * Dk, *dkt = dk + th * Dk, *dvt = dv + th * Dv;
                for (int i = 0; i < Dk; ++i) {
                    double a = 0.0, c = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        a += St[i * Dv + j] * dot[j];
                        c += D[i * Dv + j] * ux[j];
                    }
                    dqt[i] = scale * a;
                    dkt[i] = c;
                }
                double db = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    double a = 0.0;
                    for (int i = 0; i < Dk; ++i) a += D[i * Dv + j] * kt[i];
                    du[j] = a;
                    db += a * (vt[j] - px[j]);
                    dvt[j] = bt * a;
                }
                dbeta[th] = db;
                for (int i = 0; i < Dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        D[i * Dv + j] -= bt * kt[i] * du[j];
                        a += spx[i * Dv + j] * du[j];
                    }
                    dkt[i] -= bt * a;
                }
                double dgt = 0.0;
                for (size_t i = 0; i < SS; ++i) dgt += D[i] * spx[i];
                dg[th] = dgt;
                const double decay = exp(g[th]);
                for (size_t i = 0; i < SS; ++i) D[i] *= decay;
            }
        }
        if (dh0) memcpy(dh0 + unit * (long)SS, D, sizeof(double) * SS);
        free(starts); free(Sp); free(us); free(ps); free(S); free(St); free(D); free(du);
    }
}

/*
 * Backward of the Gated DeltaNet-2 forward (same loss as gdn_oracle_bwd).
 * Per token, with P = Diag(exp(log_alpha)) S_{t-1}, e = b . k,
 * p = P^T e, u = w . v - p, S_t = P + k u^T, o = scale S_t^T q, and D the
 * gradient of L w.r.t. S_t:
 *   D   += scale q do^T          dq   = scale S_t do
 *   dk   = D u                   du   = D^T k
 *   dw   = du . v                dv   = du . w
 *   de   = -P du                 D'   = D - e du^T   (gradient w.r.t. P)
 *   db   = de . k                dk  += de . b
 *   dlog_alpha_i = sum_j D'_ij P_ij                   D = Diag(exp(log_alpha)) D'
 * and dh0 = D after the first token.  States are recomputed forward one
 * 64-token segment at a time from stored segment-start states.
 * Outputs dq, dk, dla, db [B,T,H,Dk], dv, dw [B,T,H,Dv], dh0 [B,H,Dk,Dv] or NULL.
 */
void gdn2_oracle_bwd(const double *q, const double *k, const double *v, const double *log_alpha,
                     const double *bgate, const double *wgate, const double *h0, const double *dO,
                     const double *dST, double *dq, double *dk, double *dv, double *dla, double *db,
                     double *dw, double *dh0, int B, int T, int H, int Dk, int Dv, double scale, int nthreads) {
    set_threads(nthreads);
    const long units = (long)B * H;
    const int SEG = 64;
    const int nseg = (T + SEG - 1) / SEG;
    const size_t SS = (size_t)Dk * Dv;
#pragma omp parallel for schedule(static)
    for (long unit = 0; unit < units; ++unit) {
        const long b = unit / H, h = unit % H;
        double *starts = (double *)malloc(sizeof(double) * SS * (size_t)nseg);
        double *Ps = (double *)malloc(sizeof(double) * SS * (size_t)SEG);  /* P of each token of a segment */
        double *us = (double *)malloc(sizeof(double) * (size_t)Dv * SEG);  /* u of each token */
        double *S = (double *)malloc(sizeof(double) * SS);
        double *St = (double *)malloc(sizeof(double) * SS);
        double *D = (double *)malloc(sizeof(double) * SS);
        double *du = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *de = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (h0) memcpy(S, h0 + unit * (long)SS, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (long t = 0; t < T; ++t) {
            if (t % SEG == 0) memcpy(starts + (size_t)(t / SEG) * SS, S, sizeof(double) * SS);
            const long th = (b * T + t) * H + h;
            gdn2_token(S, q + th * Dk, k + th * Dk, v + th * Dv, log_alpha + th * Dk, bgate + th * Dk,
                       wgate + th * Dv, du, e, NULL, Dk, Dv, scale);
        }
        if (dST) memcpy(D, dST + unit * (long)SS, sizeof(double) * SS);
        else memset(D, 0, sizeof(double) * SS);
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const long t0 = (long)sg * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
            /* recompute P and u of the segment */
            memcpy(S, starts + (size_t)sg * SS, sizeof(double) * SS);
            for (long t = t0; t < t1; ++t) {
                const long th = (b * T + t) * H + h, x = t - t0;
                const double *kt = k + th * Dk, *vt = v + th * Dv, *la = log_alpha + th * Dk;
                const double *bt = bgate + th * Dk, *wt = wgate + th * Dv;
                double *px = Ps + (size_t)x * SS;
                for (int i = 0; i < Dk; ++i) {
                    const double dec = exp(la[i]);
                    for (int j = 0; j < Dv; ++j) px[i * Dv + j] = S[i * Dv + j] * dec;
                }
                for (int j = 0; j < Dv; ++j) {
                    double p = 0.0;
                    for (int i = 0; i < Dk; ++i) p += px[i * Dv + j] * bt[i] * kt[i];
                    us[(size_t)x * Dv + j] = wt[j] * vt[j] - p;
                }
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < Dv; ++j) S[i * Dv + j] = px[i * Dv + j] + kt[i] * us[(size_t)x * Dv + j];
            }
            /* reverse through the segment */
            for (long t = t1 - 1; t >= t0; --t) {
                const long th = (b * T + t) * H + h, x = t - t0;
                const double *qt = q + th * Dk, *kt = k + th * Dk, *vt = v + th * Dv, *dot = dO + th * Dv;
                const double *la = log_alpha + th * Dk, *bt = bgate + th * Dk, *wt = wgate + th * Dv;
                const double *px = Ps + (size_t)x * SS, *ux = us + (size_t)x * Dv;
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < Dv; ++j) St[i * Dv + j] = px[i * Dv + j] + kt[i] * ux[j];
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < Dv; ++j) D[i * Dv + j] += scale * dot[j] * qt[i];
                double *dqt = dq + th * Dk, *dkt = dk + th * Dk, *dvt = dv + th * Dv;
                double *dlat = dla + th * Dk, *dbt = db + th * Dk, *dwt = dw + th * Dv;
                for (int i = 0; i < Dk; ++i) {
                    double a = 0.0, c = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        a += dot[j] * St[i * Dv + j];
                        c += D[i * Dv + j] * ux[j];
                    }
                    dqt[i] = scale * a;
                    dkt[i] = c;
                }
                for (int j = 0; j < Dv; ++j) {
                    double a = 0.0;
                    for (int i = 0; i < Dk; ++i) a += D[i * Dv + j] * kt[i];
                    du[j] = a;
                    dwt[j] = a * vt[j];
                    dvt[j] = a * wt[j];
                }
                for (int i = 0; i < Dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < Dv; ++j) a += px[i * Dv + j] * du[j];
                    de[i] = -a;
                    dbt[i] = de[i] * kt[i];
                    dkt[i] += de[i] * bt[i];
                }
                for (int i = 0; i < Dk; ++i) {
                    const double ei = bt[i] * kt[i];
                    double a = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        D[i * Dv + j] -= ei * du[j];
                        a += D[i * Dv + j] * px[i * Dv + j];
                    }
                    dlat[i] = a;
                    const double al = exp(la[i]);
                    for (int j = 0; j < Dv; ++j) D[i * Dv + j] *= al;
                }
            }
        }
        if (dh0) memcpy(dh0 + unit * (long)SS, D, sizeof(double) * SS);
        free(starts); free(Ps); free(us); free(S); free(St); free(D); free(du); free(e); free(de);
    }
}
