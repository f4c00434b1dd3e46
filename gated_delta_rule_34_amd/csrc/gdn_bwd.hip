// gdn_bwd.hip -- backward of the chunked Gated DeltaNet forward on gfx950
// (fp32 arithmetic throughout; bf16 inputs are exact in fp32).
//
// Chunk equations (the chunked form of the GatedDeltaNet walkthrough's
// recurrence, section on the chunked Triton kernels): in a chunk with entry
// state S, G the chunk-local cumsum of g, gamma_i = e^{G_i},
// D_ij = e^{G_i - G_j} (j <= i), Kd_j = k_j e^{G_C - G_j},
//   A = strict(diag(beta) K K^T . D),  T = (I + A)^-1,
//   R = diag(beta) (V - diag(gamma) K S),  Vn = T R,
//   P = (Q K^T) . D,  O = scale (diag(gamma) Q S + P Vn),
//   S' = gamma_C S + Kd^T Vn.
// Reverse mode, with dS' the gradient of the state leaving the chunk:
//   dVn = scale P^T dO + Kd dS'        dR = T^T dVn
//   dA  = -strict(dR Vn^T)             dP = scale lower(dO Vn^T)
//   dS  = gamma_C dS' + scale (diag(gamma) Q)^T dO - (diag(beta gamma) K)^T dR
// and the chain rule through A, P, R, the state read of O and Kd gives dq,
// dk, dv = diag(beta) dR, dbeta and dG; dg is the reverse cumulative sum of
// dG within the chunk.
//
// Stages (all chunks of all heads):
//   1. the forward's intra stage: G2 = log2(e) G and T - I per chunk
//   2. the forward walk, writing the entry state of every chunk
//   3. bwd_walk_kernel: dS' chunk by chunk from the last one back (state
//      columns are independent, so one workgroup owns 32 of them), written
//      per chunk; dh0 is the gradient entering the first chunk
//   4. bwd_chunk_kernel: one workgroup per (batch, head, chunk) recomputes
//      the chunk and produces its dq, dk, dv, dbeta, dg, looping over the
//      value columns 16 at a time
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// acc (the 16x16 tile at rows i0, columns j0 of C) += A B over k in [0, K):
// A(i, k) = A[i * sar + k * sac], B(k, j) = B[k * sbr + j * sbc] (LDS, fp32),
// optionally B(k, j) * ks[k].  Lane (g, r) ends with C[i0 + 4g + e][j0 + r].
// K is a compile-time constant so the loop unrolls and the LDS reads of
// successive steps are issued ahead of their MFMAs.
template <int K>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const float *A, int sar, int sac, const float *B, int sbr,
                                          int sbc, const float *ks, int i0, int j0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float *pa = A + (i0 + r) * sar + g * sac;
    const float *pb = B + g * sbr + (j0 + r) * sbc;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
        const float a = pa[k0 * sac];
        float b = pb[k0 * sbr];
        if (ks) b *= ks[k0 + g];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

// Sum over the 16 lanes of a lane group (the columns of a tile row).
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// Chunk inputs common to both backward kernels: Q, K rows (zero past T) and
// the gate tables of chunk c.
template <class Pol, int DK, int LDQ, int NTHR>
__device__ __forceinline__ void load_chunk_qk(float *sQ, float *sK, float *sG2, float *sGam, float *sDec, float *sBeta,
                                              const typename Pol::in_t *q, const typename Pol::in_t *k,
                                              const float *beta, const float *G2ws, long b, int h, int c, long cb,
                                              int T, int H, int tid) {
    const int t0 = c * BT;
    stage_rows<DK, LDQ, NTHR>(sQ, q, b, h, t0, T, H, 0, DK, tid);
    stage_rows<DK, LDQ, NTHR>(sK, k, b, h, t0, T, H, 0, DK, tid);
    if (tid < BT) {
        const int t = t0 + tid;
        const float G2 = G2ws[cb * BT + tid], G2L = G2ws[cb * BT + BT - 1];
        sG2[tid] = G2;
        sGam[tid] = exp2f(G2);
        sDec[tid] = exp2f(G2L - G2);
        sBeta[tid] = (t < T) ? beta[(b * T + t) * H + h] : 0.f;
    }
}

// A 64 x 64 fp32 matrix (T - I of a chunk) into LDS with row stride LD.
template <int LD, int NTHR>
__device__ __forceinline__ void stage_tm(float *dst, const float *src, int tid) {
    constexpr int U = BT * BT / 4 / NTHR;
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = *(const float4 *)(src + 4 * (tid + NTHR * u));
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = 4 * (tid + NTHR * u), row = idx / BT, col = idx % BT;
        dst[row * LD + col] = x[u].x;
        dst[row * LD + col + 1] = x[u].y;
        dst[row * LD + col + 2] = x[u].z;
        dst[row * LD + col + 3] = x[u].w;
    }
}

// --------------------------------------------------------- reverse state walk
template <class Pol, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_walk_kernel(const typename Pol::in_t *__restrict__ q,
                                                       const typename Pol::in_t *__restrict__ k,
                                                       const float *__restrict__ beta, const float *__restrict__ dO,
                                                       const float *__restrict__ dht, const float *__restrict__ G2ws,
                                                       const float *__restrict__ Tws, float *__restrict__ dSck,
                                                       float *__restrict__ dh0, int T, int H, int NT, float scale) {
    constexpr int BV = 32, NTHR = 256, LDQ = DK + 4, LDC = BT + 1, LDB = BV + 1;
    __shared__ float sQ[BT * LDQ], sK[BT * LDQ], sTm[BT * LDC], sP[BT * LDC];
    __shared__ float sdO[BT * LDB], sdVn[BT * LDB], sdR[BT * LDB], sdS[DK * LDB];
    __shared__ float sG2[BT], sGam[BT], sDec[BT], sBeta[BT], sGdO[BT], sBG[BT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    constexpr int NTILE = DV / BV;
    const int vt = blockIdx.x % NTILE;
    const long bh = blockIdx.x / NTILE;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int vcol0 = vt * BV;
    const long sbase = bh * (long)DK * DV;

    for (int idx = tid; idx < DK * BV; idx += NTHR) {
        const int row = idx / BV, col = idx % BV;
        sdS[row * LDB + col] = dht ? dht[sbase + (long)row * DV + vcol0 + col] : 0.f;
    }
    for (int idx = tid; idx < BT * LDC; idx += NTHR) sP[idx] = 0.f;  // upper tiles stay zero
    __syncthreads();

    for (int c = NT - 1; c >= 0; --c) {
        const long cb = bh * NT + c;
        const int t0 = c * BT;
        // gradient of the state leaving chunk c, for the per-chunk stage
#pragma unroll
        for (int u = 0; u < DK * BV / 4 / NTHR; ++u) {
            const int idx = 4 * (tid + NTHR * u), row = idx / BV, col = idx % BV;
            const float *p = &sdS[row * LDB + col];
            *(float4 *)(dSck + cb * DK * DV + (long)row * DV + vcol0 + col) = make_float4(p[0], p[1], p[2], p[3]);
        }
        load_chunk_qk<Pol, DK, LDQ, NTHR>(sQ, sK, sG2, sGam, sDec, sBeta, q, k, beta, G2ws, b, h, c, cb, T, H, tid);
        stage_tm<LDC, NTHR>(sTm, Tws + cb * BT * BT, tid);
        stage_rows<BV, LDB, NTHR>(sdO, dO, b, h, t0, T, H, vcol0, DV, tid);
        __syncthreads();
        if (tid < BT) {
            sGdO[tid] = sGam[tid];               // B-row scale of (gamma Q)^T dO
            sBG[tid] = sBeta[tid] * sGam[tid];   // B-row scale of (beta gamma K)^T dR
        }
        // P = (Q K^T) . D on the 10 lower tiles
        for (int tile = wave; tile < 10; tile += 4) {
            const int I = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J = tile - I * (I + 1) / 2;
            f32x4 acc = tile_mma<DK>(zero4(), sQ, LDQ, 1, sK, 1, LDQ, nullptr, 16 * I, 16 * J, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e, j = 16 * J + r;
                sP[i * LDC + j] = (j <= i) ? acc[e] * exp2f(sG2[i] - sG2[j]) : 0.f;
            }
        }
        __syncthreads();
        // dVn = scale P^T dO + Kd dS' (8 tiles of 64 x 32)
        for (int tile = wave; tile < 8; tile += 4) {
            const int I = tile >> 1, J = tile & 1;
            const f32x4 a1 = tile_mma<BT>(zero4(), sP, 1, LDC, sdO, LDB, 1, nullptr, 16 * I, 16 * J, lane);
            const f32x4 a2 = tile_mma<DK>(zero4(), sK, LDQ, 1, sdS, LDB, 1, nullptr, 16 * I, 16 * J, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                sdVn[i * LDB + 16 * J + r] = scale * a1[e] + sDec[i] * a2[e];
            }
        }
        __syncthreads();
        // dR = dVn + (T - I)^T dVn
        for (int tile = wave; tile < 8; tile += 4) {
            const int I = tile >> 1, J = tile & 1;
            const f32x4 a = tile_mma<BT>(zero4(), sTm, 1, LDC, sdVn, LDB, 1, nullptr, 16 * I, 16 * J, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                sdR[i * LDB + 16 * J + r] = sdVn[i * LDB + 16 * J + r] + a[e];
            }
        }
        __syncthreads();
        // dS = gamma_C dS' + scale (gamma Q)^T dO - (beta gamma K)^T dR  (DK/16 x 2 tiles)
        const float gC = sGam[BT - 1];
        for (int tile = wave; tile < (DK / 16) * 2; tile += 4) {
            const int M = tile >> 1, J = tile & 1;
            const f32x4 a1 = tile_mma<BT>(zero4(), sQ, 1, LDQ, sdO, LDB, 1, sGdO, 16 * M, 16 * J, lane);
            const f32x4 a2 = tile_mma<BT>(zero4(), sK, 1, LDQ, sdR, LDB, 1, sBG, 16 * M, 16 * J, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float *d = &sdS[(16 * M + 4 * g + e) * LDB + 16 * J + r];
                *d = gC * *d + scale * a1[e] - a2[e];
            }
        }
        __syncthreads();
    }
    if (dh0) {
        for (int idx = tid; idx < DK * BV; idx += NTHR) {
            const int row = idx / BV, col = idx % BV;
            dh0[sbase + (long)row * DV + vcol0 + col] = sdS[row * LDB + col];
        }
    }
}

// ----------------------------------------------------- per-chunk gradients
template <int DK>
struct BwdChunkSmem {
    static constexpr int LDQ = DK + 4, LDC = BT + 1, CW = 16, LDW = CW + 1;
    float Q[BT * LDQ], K[BT * LDQ];
    float Tm[BT * LDC];   // T - I; after the column loop: dA . D
    float P[BT * LDC];    // (Q K^T) . D, lower; after the column loop: dP . D
    float S[DK * LDW], dS[DK * LDW];                 // column slice of S and dS'
    float V[BT * LDW], dO[BT * LDW], R[BT * LDW], Vn[BT * LDW], dVn[BT * LDW];
    float G2[BT], Gam[BT], Dec[BT], Beta[BT];
    float dB[BT], dG[BT], colG[4][BT], red[256];
};

template <class Pol, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_chunk_kernel(
    const typename Pol::in_t *__restrict__ q, const typename Pol::in_t *__restrict__ k,
    const typename Pol::in_t *__restrict__ v, const float *__restrict__ beta, const float *__restrict__ dO,
    const float *__restrict__ G2ws, const float *__restrict__ Tws, const float *__restrict__ Sck,
    const float *__restrict__ dSck, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
    float *__restrict__ dg, float *__restrict__ dbeta, int T, int H, int NT, float scale) {
    using SM = BwdChunkSmem<DK>;
    constexpr int LDQ = SM::LDQ, LDC = SM::LDC, CW = SM::CW, LDW = SM::LDW, NTHR = 256, NM = DK / 16;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const long cb = blockIdx.x;
    const int c = (int)(cb % NT);
    const long bh = cb / NT;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int t0 = c * BT;
    const int I = wave;  // this wave's 16-row block of every chunk-row product

    load_chunk_qk<Pol, DK, LDQ, NTHR>(sm.Q, sm.K, sm.G2, sm.Gam, sm.Dec, sm.Beta, q, k, beta, G2ws, b, h, c, cb, T,
                                      H, tid);
    stage_tm<LDC, NTHR>(sm.Tm, Tws + cb * BT * BT, tid);
    if (tid < BT) {
        sm.dB[tid] = 0.f;
        sm.dG[tid] = 0.f;
    }
    __syncthreads();
    // P = (Q K^T) . D, lower with the diagonal (all 16 tiles, upper ones zero)
    for (int tile = wave; tile < 16; tile += 4) {
        const int TI = tile >> 2, TJ = tile & 3;
        const f32x4 acc = tile_mma<DK>(zero4(), sm.Q, LDQ, 1, sm.K, 1, LDQ, nullptr, 16 * TI, 16 * TJ, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * TI + 4 * g + e, j = 16 * TJ + r;
            sm.P[i * LDC + j] = (j <= i) ? acc[e] * exp2f(sm.G2[i] - sm.G2[j]) : 0.f;
        }
    }

    f32x4 dqs[NM], dkR[NM], dKd[NM], dA[4], dP[4];
#pragma unroll
    for (int m = 0; m < NM; ++m) dqs[m] = dkR[m] = dKd[m] = zero4();
#pragma unroll
    for (int j = 0; j < 4; ++j) dA[j] = dP[j] = zero4();
    float dGC = 0.f;  // <dS', S> over the slices this thread loaded

    for (int c0 = 0; c0 < DV; c0 += CW) {
        __syncthreads();  // previous slice fully consumed
        {
            // S and dS' slices: DK x CW fp32, 4 columns per thread and pass
            constexpr int US = DK * CW / 4 / NTHR;
            float4 xs[US], xd[US];
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int idx = 4 * (tid + NTHR * u), row = idx / CW, col = idx % CW;
                const long off = cb * DK * DV + (long)row * DV + c0 + col;
                xs[u] = *(const float4 *)(Sck + off);
                xd[u] = *(const float4 *)(dSck + off);
            }
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int idx = 4 * (tid + NTHR * u), row = idx / CW, col = idx % CW;
                float *ps = &sm.S[row * LDW + col], *pd = &sm.dS[row * LDW + col];
                ps[0] = xs[u].x; ps[1] = xs[u].y; ps[2] = xs[u].z; ps[3] = xs[u].w;
                pd[0] = xd[u].x; pd[1] = xd[u].y; pd[2] = xd[u].z; pd[3] = xd[u].w;
                dGC += xs[u].x * xd[u].x + xs[u].y * xd[u].y + xs[u].z * xd[u].z + xs[u].w * xd[u].w;
            }
        }
        if (tid < BT * CW / 8) stage_rows<CW, LDW, BT * CW / 8>(sm.V, v, b, h, t0, T, H, c0, DV, tid);
        else if (tid < BT * CW / 4) stage_rows<CW, LDW, BT * CW / 8>(sm.dO, dO, b, h, t0, T, H, c0, DV, tid - BT * CW / 8);
        __syncthreads();
        // KS, QS, R for rows of block I
        const f32x4 KS = tile_mma<DK>(zero4(), sm.K, LDQ, 1, sm.S, LDW, 1, nullptr, 16 * I, 0, lane);
        const f32x4 QS = tile_mma<DK>(zero4(), sm.Q, LDQ, 1, sm.S, LDW, 1, nullptr, 16 * I, 0, lane);
        f32x4 Rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            Rr[e] = sm.Beta[i] * (sm.V[i * LDW + r] - sm.Gam[i] * KS[e]);
            sm.R[i * LDW + r] = Rr[e];
        }
        __syncthreads();
        // Vn = R + (T - I) R;  dVn = scale P^T dO + Kd dS'
        {
            const f32x4 a = tile_mma<BT>(zero4(), sm.Tm, LDC, 1, sm.R, LDW, 1, nullptr, 16 * I, 0, lane);
            const f32x4 b1 = tile_mma<BT>(zero4(), sm.P, 1, LDC, sm.dO, LDW, 1, nullptr, 16 * I, 0, lane);
            const f32x4 b2 = tile_mma<DK>(zero4(), sm.K, LDQ, 1, sm.dS, LDW, 1, nullptr, 16 * I, 0, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                sm.Vn[i * LDW + r] = Rr[e] + a[e];
                sm.dVn[i * LDW + r] = scale * b1[e] + sm.Dec[i] * b2[e];
            }
        }
        __syncthreads();
        // dR = dVn + (T - I)^T dVn; dv; the row sums of dbeta and dG
        f32x4 dRr;
        {
            const f32x4 a = tile_mma<BT>(zero4(), sm.Tm, 1, LDC, sm.dVn, LDW, 1, nullptr, 16 * I, 0, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                const int t = t0 + i;
                dRr[e] = sm.dVn[i * LDW + r] + a[e];
                if (t < T) dv[((b * T + t) * H + h) * (long)DV + c0 + r] = sm.Beta[i] * dRr[e];
                const float vb = sm.V[i * LDW + r] - sm.Gam[i] * KS[e];
                const float pb = row16_sum(dRr[e] * vb);
                const float pg = row16_sum(-sm.Beta[i] * sm.Gam[i] * dRr[e] * KS[e] +
                                           scale * sm.Gam[i] * sm.dO[i * LDW + r] * QS[e]);
                if (r == 0) {
                    sm.dB[i] += pb;
                    sm.dG[i] += pg;
                }
            }
        }
        // dR rows of this wave go where R was (R is no longer read)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.R[(16 * I + 4 * g + e) * LDW + r] = dRr[e];
        __syncthreads();
        // accumulate dA, dP (64 x 64) and the DK-wide products for rows of block I
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            // B(k, j) = Vn[j][k]
            const f32x4 x = tile_mma<CW>(zero4(), sm.R, LDW, 1, sm.Vn, 1, LDW, nullptr, 16 * I, 16 * J, lane);
            const f32x4 y = tile_mma<CW>(zero4(), sm.dO, LDW, 1, sm.Vn, 1, LDW, nullptr, 16 * I, 16 * J, lane);
            dA[J] -= x;
            dP[J] += y * scale;
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            // B(k, m) = S[m][k] and dS'[m][k]
            dqs[m] = tile_mma<CW>(dqs[m], sm.dO, LDW, 1, sm.S, 1, LDW, nullptr, 16 * I, 16 * m, lane);
            dkR[m] = tile_mma<CW>(dkR[m], sm.R, LDW, 1, sm.S, 1, LDW, nullptr, 16 * I, 16 * m, lane);
            dKd[m] = tile_mma<CW>(dKd[m], sm.Vn, LDW, 1, sm.dS, 1, LDW, nullptr, 16 * I, 16 * m, lane);
        }
    }
    __syncthreads();  // every wave is done with Tm and P

    // dA, dP on their supports; A, P and the K K^T terms
    float colp[4][4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        const f32x4 KK = tile_mma<DK>(zero4(), sm.K, LDQ, 1, sm.K, 1, LDQ, nullptr, 16 * I, 16 * J, lane);
        const f32x4 QK = tile_mma<DK>(zero4(), sm.Q, LDQ, 1, sm.K, 1, LDQ, nullptr, 16 * I, 16 * J, lane);
        const int j = 16 * J + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            const float D = (j <= i) ? exp2f(sm.G2[i] - sm.G2[j]) : 0.f;
            const float dAv = (j < i) ? dA[J][e] : 0.f;
            const float dPv = (j <= i) ? dP[J][e] : 0.f;
            const float Av = sm.Beta[i] * KK[e] * D, Pv = QK[e] * D;
            const float w = dAv * Av + dPv * Pv;
            const float pb = row16_sum(dAv * D * KK[e]);
            const float pg = row16_sum(w);
            if (r == 0) {
                sm.dB[i] += pb;
                sm.dG[i] += pg;
            }
            colp[J][e] = w;
            sm.Tm[i * LDC + j] = dAv * D;  // dA . D
            sm.P[i * LDC + j] = dPv * D;   // dP . D
        }
    }
    // column sums of dA . A + dP . P: lanes of column j = 16J + r, over the 4 rows e and the 4 row groups g
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        float x = colp[J][0] + colp[J][1] + colp[J][2] + colp[J][3];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (g == 0) sm.colG[wave][16 * J + r] = x;
    }
    __syncthreads();

    // dk = diag(beta) dAs K + dAs^T diag(beta) K + dPs^T Q + diag(dec) dKd - diag(beta gamma) dkR
    // dq = scale diag(gamma) dqs + dPs K
    float tdec[4] = {0.f, 0.f, 0.f, 0.f};  // sum_m dKd_im K_im for the 4 rows of this lane
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const f32x4 t1 = tile_mma<BT>(zero4(), sm.Tm, LDC, 1, sm.K, LDQ, 1, nullptr, 16 * I, 16 * m, lane);
        const f32x4 t2 = tile_mma<BT>(zero4(), sm.Tm, 1, LDC, sm.K, LDQ, 1, sm.Beta, 16 * I, 16 * m, lane);
        const f32x4 t3 = tile_mma<BT>(zero4(), sm.P, 1, LDC, sm.Q, LDQ, 1, nullptr, 16 * I, 16 * m, lane);
        const f32x4 t4 = tile_mma<BT>(zero4(), sm.P, LDC, 1, sm.K, LDQ, 1, nullptr, 16 * I, 16 * m, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e, col = 16 * m + r;
            const int t = t0 + i;
            const float kim = sm.K[i * LDQ + col];
            tdec[e] = fmaf(dKd[m][e], kim, tdec[e]);
            const float dkv = sm.Beta[i] * t1[e] + t2[e] + t3[e] + sm.Dec[i] * dKd[m][e] -
                              sm.Beta[i] * sm.Gam[i] * dkR[m][e];
            const float dqv = scale * sm.Gam[i] * dqs[m][e] + t4[e];
            if (t < T) {
                const long off = ((b * T + t) * H + h) * (long)DK + col;
                dk[off] = dkv;
                dq[off] = dqv;
            }
        }
    }
    // Kd terms of dG: t_j = dec_j (dKd_j . k_j) leaves row j and enters the last row
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * g + e;
        const float tj = row16_sum(tdec[e]) * sm.Dec[i];
        if (r == 0) sm.dG[i] -= tj;
        tdec[e] = (r == 0) ? tj : 0.f;
    }
    sm.red[tid] = tdec[0] + tdec[1] + tdec[2] + tdec[3];
    __syncthreads();
    if (tid == 0) {
        float tsum = 0.f;
        for (int x = 0; x < NTHR; ++x) tsum += sm.red[x];
        sm.dG[BT - 1] += tsum;
    }
    __syncthreads();
    sm.red[tid] = dGC;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int x = 0; x < NTHR; ++x) s += sm.red[x];
        sm.dG[BT - 1] += sm.Gam[BT - 1] * s;
        // dG_j -= column sums; dg = reverse cumulative sum of dG within the chunk
        float acc = 0.f;
        for (int i = BT - 1; i >= 0; --i) {
            const float dGi = sm.dG[i] - (sm.colG[0][i] + sm.colG[1][i] + sm.colG[2][i] + sm.colG[3][i]);
            acc += dGi;
            const int t = t0 + i;
            if (t < T) {
                dg[(b * T + t) * H + h] = acc;
                dbeta[(b * T + t) * H + h] = sm.dB[i];
            }
        }
    }
}

// ----------------------------------------------------------------- launchers
template <class Pol, int DK, int DV>
static hipError_t launch_bwd_t(const void *q, const void *k, const void *v, const float *beta, const float *dO,
                               const float *dht, const float *G2, const float *Tinv, const float *Sck, float *dSck,
                               float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0, int B, int T,
                               int H, float scale, hipStream_t st) {
    using in_t = typename Pol::in_t;
    const int NT = (T + BT - 1) / BT;
    hipLaunchKernelGGL((bwd_walk_kernel<Pol, DK, DV>), dim3((unsigned)((long)B * H * (DV / 32))), dim3(256), 0, st,
                       (const in_t *)q, (const in_t *)k, beta, dO, dht, G2, Tinv, dSck, dh0, T, H, NT, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_chunk_kernel<Pol, DK, DV>), dim3((unsigned)((long)B * H * NT)), dim3(256), 0, st,
                       (const in_t *)q, (const in_t *)k, (const in_t *)v, beta, dO, G2, Tinv, Sck, dSck, dq, dk, dv,
                       dg, dbeta, T, H, NT, scale);
    return hipGetLastError();
}

hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *beta, const float *dO,
                      const float *dht, const float *G2, const float *Tinv, const float *Sck, float *dSck, float *dq,
                      float *dk, float *dv, float *dg, float *dbeta, float *dh0, int B, int T, int H, int Dk, int Dv,
                      bool bf16, float scale, hipStream_t st) {
#define GDN_BWD(P, DKv, DVv)                                                                                       \
    if (Dk == DKv && Dv == DVv)                                                                                    \
    return launch_bwd_t<P, DKv, DVv>(q, k, v, beta, dO, dht, G2, Tinv, Sck, dSck, dq, dk, dv, dg, dbeta, dh0, B, T, \
                                     H, scale, st)
    if (bf16) {
        GDN_BWD(PolBF16, 64, 64);
        GDN_BWD(PolBF16, 64, 128);
        GDN_BWD(PolBF16, 128, 64);
        GDN_BWD(PolBF16, 128, 128);
    } else {
        GDN_BWD(PolF32, 64, 64);
        GDN_BWD(PolF32, 64, 128);
        GDN_BWD(PolF32, 128, 64);
        GDN_BWD(PolF32, 128, 128);
    }
#undef GDN_BWD
    return hipErrorInvalidValue;
}

}  // namespace gdn
