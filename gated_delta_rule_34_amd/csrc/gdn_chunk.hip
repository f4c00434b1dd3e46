// gdn_chunk.hip -- chunked Gated DeltaNet forward on gfx950.
//
// Two kernels per call, both enqueued on the caller's stream:
//
//  intra_kernel  (one workgroup per 64-token chunk of one head; B*H*NT groups)
//    * chunk-local cumsum of g, times log2(e), so every decay below is one
//      exp2 of a non-positive difference (GatedDeltaNet walkthrough,
//      yfxerp.com, chunked-kernel section: cumsum scaled by 1.44269504);
//    * A = strictly-lower( diag(beta) K K^T  .  2^(G2_i - G2_j) ) on MFMA
//      (bf16 MFMA for bf16 keys, whose products are exact);
//    * T = (I + A)^-1: the four 16x16 diagonal blocks by forward
//      substitution (one lane per column), the off-diagonal blocks by
//      block forward substitution T_IJ = -T_II sum_K A_IK T_KJ on fp32 MFMA.
//    Writes G2 and T - I to the workspace.
//
//  walk_kernel   (one workgroup per (b, h, BV-wide slice of value columns))
//    walks the chunks in order with its d_k x BV slice of the state resident
//    in MFMA accumulator registers; per chunk:
//      X = K S, Y = Q S                                (state reads)
//      R = diag(beta) (V - diag(gamma) X)              (fp32)
//      Vnew = R + (T - I) R  = U - W S                 (the WY form: U = T diag(beta) V,
//                                                       W = T diag(beta gamma) K)
//      O = scale (diag(gamma) Y + diag(q.k) Vnew + strict(P) Vnew),
//          P_ij = (q_i . k_j) 2^(G2_i - G2_j)          (causal intra-chunk term)
//      S = gamma_C S + (K . 2^(G2_C - G2))^T Vnew      (carry to the next chunk)
//    The value columns of the state evolve independently, so each wave owns
//    16 columns and runs the whole chain in registers; only the per-chunk
//    inputs (Q, K, decayed K^T, P) are shared through LDS.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8c;

// The 10 lower-triangular 16x16 tiles (I >= J) of a 64x64 chunk matrix.
__constant__ int kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <class Pol, int DK>
__global__ __launch_bounds__(256) void intra_kernel(const typename Pol::in_t *__restrict__ kin,
                                                    const float *__restrict__ gin,
                                                    const float *__restrict__ betain,
                                                    float *__restrict__ G2out, float *__restrict__ Tout,
                                                    double *__restrict__ G2dout, int T, int H, int NT) {
    using mt = typename Pol::mt;
    constexpr int LDK = DK + 8;
    constexpr int LDA = 65;
    __shared__ float sA[BT * LDA];
    // bf16 keys stay raw bf16 rows (their products are exact on bf16 MFMA)
    constexpr bool RAW = std::is_same<typename Pol::in_t, uint16_t>::value && std::is_same<mt, float>::value;
    __shared__ union alignas(16) {
        mt k[BT * LDK];
        uint16_t kraw[BT * LDK];
        float t[BT * LDA];
    } u;
    __shared__ float sBeta[BT];
    // G2 in fp64: its differences G2_i - G2_j are then exact to fp32 however
    // large the chunk's decay (an fp32 G2 of magnitude ~1000 carries an
    // absolute error of ~6e-5 into every decay factor)
    __shared__ double sG2[BT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const long chunk = blockIdx.x;
    const int c = (int)(chunk % NT);
    const long bh = chunk / NT;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int t0 = c * BT;

    if (wave == 0) {
        const int t = t0 + lane;
        float gv = 0.f, bv = 0.f;
        if (t < T) {
            const long idx = (b * T + t) * H + h;
            gv = gin[idx];
            bv = betain[idx];
        }
        double x = gv;  // the scan runs in fp64: G2 is then rounded once
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const double G2 = x * 1.4426950408889634;
        sG2[lane] = G2;
        sBeta[lane] = bv;
        G2out[chunk * BT + lane] = (float)G2;
        if (G2dout) G2dout[chunk * BT + lane] = G2;
    }
    for (int idx = tid; idx < BT * DK / 4; idx += 256) {
        const int row = idx / (DK / 4), col = (idx % (DK / 4)) * 4;
        const int t = t0 + row;
        if constexpr (RAW) {
            uint2 x = make_uint2(0u, 0u);
            if (t < T) x = *(const uint2 *)(kin + ((b * T + t) * H + h) * (long)DK + col);
            *(uint2 *)&u.kraw[row * LDK + col] = x;
        } else {
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            if (t < T) {
                const typename Pol::in_t *p = kin + ((b * T + t) * H + h) * (long)DK + col;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = load_elem(p + e);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) u.k[row * LDK + col + e] = to_mt<mt>(x[e]);
        }
    }
    __syncthreads();

    // A = strictly-lower(diag(beta) K K^T . decay), tile by tile on MFMA.
    for (int tile = wave; tile < 10; tile += 4) {
        const int I = kTileI[tile], J = kTileJ[tile];
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += 32) {
            if constexpr (RAW) {
                // one 16-byte read per operand (lane (g, r): k-slots 8g .. + 7)
                // and one exact bf16 MFMA per 32 k
                const bf16x8c a = *(const bf16x8c *)&u.kraw[(16 * I + r) * LDK + kk + 8 * g];
                const bf16x8c bb = *(const bf16x8c *)&u.kraw[(16 * J + r) * LDK + kk + 8 * g];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc, 0, 0, 0);
            } else {
                mt a[8], bb[8];
                frag_rows(a, u.k, LDK, 16 * I, kk, lane);
                frag_rows(bb, u.k, LDK, 16 * J, kk, lane);
                acc = mma_slab(acc, a, bb);
            }
        }
        const int j = 16 * J + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            float val = 0.f;
            if (i > j) val = acc[e] * sBeta[i] * exp2f((float)(sG2[i] - sG2[j]));
            sA[i * LDA + j] = val;
        }
    }
    __syncthreads();

    // Diagonal 16x16 blocks of T: lane (block bb, column cc) solves its column.
    if (wave == 0) {
        const int bb = lane >> 4, cc = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == cc) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= sA[(16 * bb + i) * LDA + 16 * bb + j] * x[j];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) u.t[(16 * bb + i) * LDA + 16 * bb + cc] = x[i];
    }
    __syncthreads();

    // Off-diagonal blocks, one sub-diagonal at a time.
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int J = wave, I = wave + d;
            f32x4 m = zero4();
            for (int K = J; K < I; ++K) {
                float a[4], bq[4];
                frag_rows4(a, sA, LDA, 16 * I, 16 * K, lane);
                frag_cols4(bq, u.t, LDA, 16 * K, 16 * J, lane);
                m = mma_block_f32(m, a, bq);
            }
            float a[4], bq[4];
            frag_rows4(a, u.t, LDA, 16 * I, 16 * I, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) bq[e] = m[e];
            const f32x4 res = mma_block_f32(zero4(), a, bq);
#pragma unroll
            for (int e = 0; e < 4; ++e) u.t[(16 * I + 4 * g + e) * LDA + 16 * J + r] = -res[e];
        }
        __syncthreads();
    }

    float *Tc = Tout + chunk * (BT * BT);
    for (int idx = tid; idx < BT * BT; idx += 256) {
        const int i = idx >> 6, j = idx & 63;
        Tc[idx] = (i > j) ? u.t[i * LDA + j] : 0.f;
    }
}

// OUT = false: only the state chain (entry states into ck, final state),
// for the backward's recompute; Q, P and the output are skipped.
template <class Pol, int DK, int DV, int BV, bool OUT>
__global__ __launch_bounds__(BV * 4) void walk_kernel(const typename Pol::in_t *__restrict__ q,
                                                      const typename Pol::in_t *__restrict__ k,
                                                      const typename Pol::in_t *__restrict__ v,
                                                      const float *__restrict__ betain,
                                                      const float *__restrict__ G2ws,
                                                      const float *__restrict__ Tws,
                                                      const float *__restrict__ h0, float *__restrict__ o,
                                                      float *__restrict__ ht, float *__restrict__ ck, int T,
                                                      int H, int NT, float scale) {
    using mt = typename Pol::mt;
    using in_t = typename Pol::in_t;
    constexpr int NW = BV / 16;
    constexpr int NTHR = NW * 64;
    constexpr int NKB = DK / 16;
    constexpr int LDQ = DK + 8;
    constexpr int LDKT = BT + 8;
    constexpr int LDP = BT + 8;
    constexpr int LDV = BV + 1;
    __shared__ mt sQ[BT * LDQ], sK[BT * LDQ], sKt[DK * LDKT], sP[BT * LDP], sT[BT * LDP];
    __shared__ float sV[BT * LDV];
    __shared__ float sG2[BT], sBeta[BT], sGam[BT], sDecK[BT], sDiag[BT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    constexpr int NTILE = DV / BV;
    const int vt = blockIdx.x % NTILE;
    const long bh = blockIdx.x / NTILE;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int col = vt * BV + wave * 16 + r;

    // The upper tiles (0,1) and (2,3) of sP are read by the 32-wide slabs of
    // the output product but never written: they hold zeros for the whole walk.
    if constexpr (OUT)
        for (int idx = tid; idx < BT * LDP; idx += NTHR) sP[idx] = to_mt<mt>(0.f);

    f32x4 S[NKB];
    const long sbase = bh * (long)DK * DV;
#pragma unroll
    for (int m = 0; m < NKB; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][e] = h0 ? h0[sbase + (long)(16 * m + 4 * g + e) * DV + col] : 0.f;

    for (int c = 0; c < NT; ++c) {
        const int t0 = c * BT;
        const long cbase = bh * NT + c;
        if (ck) {  // entry state of chunk c, [B, H, NT, DK, DV]
#pragma unroll
            for (int m = 0; m < NKB; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) ck[cbase * DK * DV + (long)(16 * m + 4 * g + e) * DV + col] = S[m][e];
        }
        if (tid < BT) {
            const float G2 = G2ws[cbase * BT + tid];
            const float G2L = G2ws[cbase * BT + BT - 1];
            const int t = t0 + tid;
            sG2[tid] = G2;
            sGam[tid] = exp2f(G2);
            sDecK[tid] = exp2f(G2L - G2);
            sBeta[tid] = (t < T) ? betain[(b * T + t) * H + h] : 0.f;
        }
        // Q, K rows, the value slice and T - I of the chunk into LDS (vector
        // loads, issued ahead of their stores)
        if constexpr (OUT) stage_rows<DK, LDQ, NTHR>(sQ, q, b, h, t0, T, H, 0, DK, tid);
        stage_rows<DK, LDQ, NTHR>(sK, k, b, h, t0, T, H, 0, DK, tid);
        stage_rows<BV, LDV, NTHR>(sV, v, b, h, t0, T, H, vt * BV, DV, tid);
        {
            const float *Tc = Tws + cbase * (BT * BT);
            constexpr int UT = BT * BT / 4 / NTHR;
#pragma unroll
            for (int u0 = 0; u0 < UT; u0 += 4) {
                float4 x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) x[u] = *(const float4 *)(Tc + 4 * (tid + NTHR * (u0 + u)));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int idx = 4 * (tid + NTHR * (u0 + u)), row = idx / BT, cc = idx % BT;
                    mt *d = &sT[row * LDP + cc];
                    d[0] = to_mt<mt>(x[u].x);
                    d[1] = to_mt<mt>(x[u].y);
                    d[2] = to_mt<mt>(x[u].z);
                    d[3] = to_mt<mt>(x[u].w);
                }
            }
        }
        __syncthreads();

        // Decayed keys, transposed: sKt[kc][j] = k_j[kc] * 2^(G2_last - G2_j).
        for (int idx = tid; idx < BT * DK; idx += NTHR) {
            const int j = idx % BT, kc = idx / BT;
            sKt[kc * LDKT + j] = to_mt<mt>((float)sK[j * LDQ + kc] * sDecK[j]);
        }
        // P^T tiles (K_J Q_I^T): lane gets P[16I + r][16J + 4g + e].
        if constexpr (OUT)
        for (int tile = wave; tile < 10; tile += NW) {
            const int I = kTileI[tile], J = kTileJ[tile];
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += 32) {
                mt a[8], bb[8];
                frag_rows(a, sK, LDQ, 16 * J, kk, lane);
                frag_rows(bb, sQ, LDQ, 16 * I, kk, lane);
                acc = mma_slab(acc, a, bb);
            }
            const int i = 16 * I + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * J + 4 * g + e;
                float val = 0.f;
                if (i > j) val = acc[e] * exp2f(sG2[i] - sG2[j]);
                if (i == j) sDiag[i] = acc[e];
                sP[i * LDP + j] = to_mt<mt>(val);
            }
        }
        __syncthreads();

        // X = K S and Y = Q S for the four 16-row blocks of the chunk.
        f32x4 X[4], Y[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) X[I] = Y[I] = zero4();
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            mt sb[8];
            frag_from_acc(sb, S[2 * s], S[2 * s + 1]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                mt a[8];
                frag_rows(a, sK, LDQ, 16 * I, 32 * s, lane);
                X[I] = mma_slab(X[I], a, sb);
                if constexpr (OUT) {
                    frag_rows(a, sQ, LDQ, 16 * I, 32 * s, lane);
                    Y[I] = mma_slab(Y[I], a, sb);
                }
            }
        }
        // R = beta (V - gamma X), fp32.
        f32x4 R[4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                R[I][e] = sBeta[i] * (sV[i * LDV + wave * 16 + r] - sGam[i] * X[I][e]);
            }
        // Vnew = R + (T - I) R; block row I only needs column blocks J <= I.
        mt rf[2][8];
        frag_from_acc(rf[0], R[0], R[1]);
        frag_from_acc(rf[1], R[2], R[3]);
        f32x4 Vn[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            Vn[I] = R[I];
#pragma unroll
            for (int s = 0; s <= (I >> 1); ++s) {
                mt a[8];
                frag_rows(a, sT, LDP, 16 * I, 32 * s, lane);
                Vn[I] = mma_slab(Vn[I], a, rf[s]);
            }
        }
        // Output: inter-chunk read of the entry state plus the causal intra term.
        mt vf[2][8];
        frag_from_acc(vf[0], Vn[0], Vn[1]);
        frag_from_acc(vf[1], Vn[2], Vn[3]);
        if constexpr (OUT)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                acc[e] = sGam[i] * Y[I][e] + sDiag[i] * Vn[I][e];
            }
#pragma unroll
            for (int s = 0; s <= (I >> 1); ++s) {
                mt a[8];
                frag_rows(a, sP, LDP, 16 * I, 32 * s, lane);
                acc = mma_slab(acc, a, vf[s]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 16 * I + 4 * g + e;
                if (o && t < T) o[((b * T + t) * H + h) * (long)DV + col] = scale * acc[e];
            }
        }
        // State carry: S = gamma_C S + Kdecayed^T Vnew.
        const float gl = sGam[BT - 1];
#pragma unroll
        for (int m = 0; m < NKB; ++m) {
            f32x4 acc = S[m] * gl;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                mt a[8];
                frag_rows(a, sKt, LDKT, 16 * m, 32 * s, lane);
                acc = mma_slab(acc, a, vf[s]);
            }
            S[m] = acc;
        }
        __syncthreads();
    }
    if (ht) {
#pragma unroll
        for (int m = 0; m < NKB; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) ht[sbase + (long)(16 * m + 4 * g + e) * DV + col] = S[m][e];
    }
}

// ----------------------------------------------------------------- launchers

template <class Pol, int DK>
static hipError_t launch_intra_t(const void *k, const float *g, const float *beta, float *G2, float *Tinv,
                                 double *G2d, int B, int T, int H, hipStream_t st) {
    const int NT = (T + BT - 1) / BT;
    const long grid = (long)B * H * NT;
    hipLaunchKernelGGL((intra_kernel<Pol, DK>), dim3((unsigned)grid), dim3(256), 0, st,
                       (const typename Pol::in_t *)k, g, beta, G2, Tinv, G2d, T, H, NT);
    return hipGetLastError();
}

hipError_t launch_intra(const void *k, const float *g, const float *beta, float *G2, float *Tinv, int B,
                        int T, int H, int Dk, bool bf16, hipStream_t st, bool exact, double *G2d) {
    if (bf16 && exact) {
        if (Dk == 64) return launch_intra_t<PolBF16F32, 64>(k, g, beta, G2, Tinv, G2d, B, T, H, st);
        return launch_intra_t<PolBF16F32, 128>(k, g, beta, G2, Tinv, G2d, B, T, H, st);
    }
    if (bf16) {
        if (Dk == 64) return launch_intra_t<PolBF16, 64>(k, g, beta, G2, Tinv, G2d, B, T, H, st);
        return launch_intra_t<PolBF16, 128>(k, g, beta, G2, Tinv, G2d, B, T, H, st);
    }
    if (Dk == 64) return launch_intra_t<PolF32, 64>(k, g, beta, G2, Tinv, G2d, B, T, H, st);
    return launch_intra_t<PolF32, 128>(k, g, beta, G2, Tinv, G2d, B, T, H, st);
}

template <class Pol, int DK, int DV>
static hipError_t launch_walk_t(const void *q, const void *k, const void *v, const float *beta,
                                const float *G2, const float *Tinv, const float *h0, float *o, float *ht,
                                float *ck, int B, int T, int H, float scale, hipStream_t st) {
    constexpr int BV = 32;
    const int NT = (T + BT - 1) / BT;
    const long grid = (long)B * H * (DV / BV);
    using in_t = typename Pol::in_t;
    if (o)
        hipLaunchKernelGGL((walk_kernel<Pol, DK, DV, BV, true>), dim3((unsigned)grid), dim3(BV * 4), 0, st,
                           (const in_t *)q, (const in_t *)k, (const in_t *)v, beta, G2, Tinv, h0, o, ht, ck, T, H,
                           NT, scale);
    else
        hipLaunchKernelGGL((walk_kernel<Pol, DK, DV, BV, false>), dim3((unsigned)grid), dim3(BV * 4), 0, st,
                           (const in_t *)q, (const in_t *)k, (const in_t *)v, beta, G2, Tinv, h0, o, ht, ck, T, H,
                           NT, scale);
    return hipGetLastError();
}

hipError_t launch_walk(const void *q, const void *k, const void *v, const float *beta, const float *G2,
                       const float *Tinv, const float *h0, float *o, float *ht, float *ck, int B, int T, int H,
                       int Dk, int Dv, bool bf16, float scale, hipStream_t st, bool exact) {
#define GDN_WALK(P, DKv, DVv) \
    if (Dk == DKv && Dv == DVv) return launch_walk_t<P, DKv, DVv>(q, k, v, beta, G2, Tinv, h0, o, ht, ck, B, T, H, scale, st)
    if (bf16 && exact) {
        GDN_WALK(PolBF16F32, 64, 64);
        GDN_WALK(PolBF16F32, 64, 128);
        GDN_WALK(PolBF16F32, 128, 64);
        GDN_WALK(PolBF16F32, 128, 128);
    } else if (bf16) {
        GDN_WALK(PolBF16, 64, 64);
        GDN_WALK(PolBF16, 64, 128);
        GDN_WALK(PolBF16, 128, 64);
        GDN_WALK(PolBF16, 128, 128);
    } else {
        GDN_WALK(PolF32, 64, 64);
        GDN_WALK(PolF32, 64, 128);
        GDN_WALK(PolF32, 128, 64);
        GDN_WALK(PolF32, 128, 128);
    }
#undef GDN_WALK
    return hipErrorInvalidValue;
}

}  // namespace gdn
