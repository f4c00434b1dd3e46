// gdn2_chunk.hip -- chunked Gated DeltaNet-2 forward on gfx950.
//
// The update (Gated DeltaNet-2 article, 7minutos.es, section "Regla-2 del
// Delta cerrado"):  S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1}
//                         + k_t (w_t . v_t)^T,   o_t = scale S_t^T q_t.
// The decay is per key channel, so it cannot be pulled out of the
// contractions as in Gated DeltaNet; the chunked WY form carries it inside
// both factors of every product (the article: the channel decay is absorbed
// into both factors of each rank-one erase).  With G2[i][c] = log2(e) *
// (chunk-local cumsum of log_alpha), Gamma_i = 2^G2_i, e_i = b_i . k_i,
// z_i = w_i . v_i, chunk entry state S0:
//   A_ij  = sum_c e_ic k_jc 2^(G2_ic - G2_jc)          (i > j)
//   P_ij  = sum_c q_ic k_jc 2^(G2_ic - G2_jc)          (i >= j)
//   T     = (I + A)^-1
//   Vnew  = T (Z - Ehat S0),       Ehat_i = e_i . Gamma_i
//   O_i   = scale ((q_i . Gamma_i)^T S0 + sum_{j<=i} P_ij vnew_j)
//   S_end = Diag(Gamma_C) S0 + Khat^T Vnew,  Khat_j = k_j . Gamma_C / Gamma_j
//
// Two kernels:
//  gdn2_intra_kernel (one workgroup per chunk of one head) computes G2 and
//    writes Ehat, Qhat = q . Gamma, Khat, Gamma_C, T - I, strict P and
//    diag(P).  The off-diagonal 16x16 blocks of A and P run on MFMA with the
//    decay split at an anchor row a (the first row of the block row):
//    2^(G2_i - G2_j) = 2^(G2_i - G2_a) 2^(G2_a - G2_j), both factors <= 1
//    because j < a <= i.  The diagonal 16x16 blocks are anchored at their
//    own first row (one factor at most 1, the other at least 1) while the
//    block's decay stays inside 2^(+-100), and otherwise summed directly in
//    fp32 on the VALU.
//  gdn2_walk_kernel (one workgroup per (b, h, 32 value columns)) walks the
//    chunks with the state slice in MFMA accumulators, like the Gated
//    DeltaNet walk, on the prepared operands.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

__device__ constexpr int t2I(int t) { return t < 1 ? 1 : t < 3 ? 2 : 3; }           // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__device__ constexpr int t2J(int t) { return t < 1 ? 0 : t < 3 ? t - 1 : t - 3; }

template <class Pol, int DK>
struct Gdn2IntraSmem {
    static constexpr int LD = DK + 1;
    static constexpr int LDA = BT + 1;
    union {
        struct {
            float K[BT * LD], E[BT * LD], Q[BT * LD];
        } in;
        float Tm[BT * LDA];
    } u;
    float G2[BT * LD];
    float A[BT * LDA];
};

// Diagonal block (rows and columns a .. a + 15) of A and P, one wave.  The
// factors are anchored at the block's own first row: e_i 2^(G2_i - G2_a) and
// q_i 2^(G2_i - G2_a), at most 1 in size, against k_j 2^(G2_a - G2_j), at
// least 1.  While every channel's decay within the block stays inside
// 2^(+-100) of row a both are fp32 numbers with no overflow or underflow and
// the block is their product on fp32 MFMA; otherwise each entry is summed
// directly with its own exponentials.
template <class Pol, int DK>
__device__ __forceinline__ void gdn2_intra_diag(Gdn2IntraSmem<Pol, DK> &sm, int a, int lane, float *__restrict__ Pc,
                                                float *__restrict__ Dc) {
    using SM = Gdn2IntraSmem<Pol, DK>;
    constexpr int LD = SM::LD, LDA = SM::LDA;
    const int r = lane & 15, g = lane >> 4;
    float span = 0.f;
    for (int c = lane; c < DK; c += 64) {
        const float ga = sm.G2[a * LD + c];
#pragma unroll
        for (int x = 1; x < 16; ++x) span = fmaxf(span, fabsf(sm.G2[(a + x) * LD + c] - ga));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
    if (span < 100.f) {
        f32x4 accA = zero4(), accP = zero4();
        const int i = a + r;  // this lane's A-operand row and B-operand column
#pragma unroll
        for (int kk = 0; kk < DK; kk += 32) {
            float fa[8], fq[8], fb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int cc = kk + (e >> 2) * 16 + 4 * g + (e & 3);
                const float Ga = sm.G2[a * LD + cc], Gi = sm.G2[i * LD + cc];
                const float ri = exp2f(Gi - Ga);
                fa[e] = sm.u.in.E[i * LD + cc] * ri;
                fq[e] = sm.u.in.Q[i * LD + cc] * ri;
                fb[e] = sm.u.in.K[i * LD + cc] * exp2f(Ga - Gi);
            }
            accA = mma_slab(accA, fa, fb);
            accP = mma_slab(accP, fq, fb);
        }
        // lane holds [a + 4g + e][a + r]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ii = 4 * g + e;
            if (r < ii) {
                sm.A[(a + ii) * LDA + a + r] = accA[e];
                Pc[(a + ii) * BT + a + r] = accP[e];
            } else if (r == ii) {
                Dc[a + ii] = accP[e];
            }
        }
    } else {
        for (int pr = lane; pr < 256; pr += 64) {
            const int il = pr >> 4, jl = pr & 15;
            if (jl > il) continue;
            const int i = a + il, j = a + jl;
            float pa = 0.f, pp = 0.f;
            for (int cc = 0; cc < DK; ++cc) {
                const float kd = sm.u.in.K[j * LD + cc] * exp2f(sm.G2[i * LD + cc] - sm.G2[j * LD + cc]);
                pa = fmaf(sm.u.in.E[i * LD + cc], kd, pa);
                pp = fmaf(sm.u.in.Q[i * LD + cc], kd, pp);
            }
            if (jl < il) {
                sm.A[i * LDA + j] = pa;
                Pc[i * BT + j] = pp;
            } else {
                Dc[i] = pp;
            }
        }
    }
}

template <class Pol, int DK>
__global__ __launch_bounds__(512) void gdn2_intra_kernel(
    const typename Pol::in_t *__restrict__ q, const typename Pol::in_t *__restrict__ k,
    const float *__restrict__ la, const typename Pol::in_t *__restrict__ bg,
    typename Pol::mt *__restrict__ Ehat, typename Pol::mt *__restrict__ Qhat, typename Pol::mt *__restrict__ Khat,
    float *__restrict__ GamC, float *__restrict__ Tout, float *__restrict__ Pout, float *__restrict__ Dout,
    int T, int H, int NT) {
    using mt = typename Pol::mt;
    using SM = Gdn2IntraSmem<Pol, DK>;
    constexpr int NTH = 512;  // eight waves
    constexpr int LD = SM::LD, LDA = SM::LDA;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const long chunk = blockIdx.x;
    const int c = (int)(chunk % NT);
    const long bh = chunk / NT;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int t0 = c * BT;

    // 1. load the chunk (rows past T are zero, log-decay 0)
    if constexpr (std::is_same<typename Pol::in_t, uint16_t>::value) {
        // bf16 inputs: every 16-byte piece of the chunk requested before the
        // first LDS store (8 channels of q, k, b and 4 of the log-decay each)
        typedef __attribute__((ext_vector_type(4))) unsigned int u32x4i;
        constexpr int UP = BT * DK / 8 / NTH, UL = BT * DK / 4 / NTH;
        u32x4i xk[UP], xq[UP], xb[UP];
        f32x4 xl[UL];
#pragma unroll
        for (int u = 0; u < UP; ++u) {
            const int p = tid + NTH * u, row = p / (DK / 8), c0 = 8 * (p % (DK / 8));
            const int t = t0 + row;
            const long off = ((b * T + t) * H + h) * (long)DK + c0;
            const bool in = t < T;
            const u32x4i z = {0u, 0u, 0u, 0u};
            xk[u] = in ? *(const u32x4i *)(k + off) : z;
            xq[u] = in ? *(const u32x4i *)(q + off) : z;
            xb[u] = in ? *(const u32x4i *)(bg + off) : z;
        }
#pragma unroll
        for (int u = 0; u < UL; ++u) {
            const int p = tid + NTH * u, row = p / (DK / 4), c0 = 4 * (p % (DK / 4));
            const int t = t0 + row;
            xl[u] = (t < T) ? *(const f32x4 *)(la + ((b * T + t) * H + h) * (long)DK + c0) : zero4();
        }
#pragma unroll
        for (int u = 0; u < UP; ++u) {
            const int p = tid + NTH * u, row = p / (DK / 8), c0 = 8 * (p % (DK / 8));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = 16 * (e & 1);
                const float kv = bf16_to_f32((uint16_t)(xk[u][e >> 1] >> sh));
                sm.u.in.K[row * LD + c0 + e] = kv;
                sm.u.in.Q[row * LD + c0 + e] = bf16_to_f32((uint16_t)(xq[u][e >> 1] >> sh));
                sm.u.in.E[row * LD + c0 + e] = bf16_to_f32((uint16_t)(xb[u][e >> 1] >> sh)) * kv;
            }
        }
#pragma unroll
        for (int u = 0; u < UL; ++u) {
            const int p = tid + NTH * u, row = p / (DK / 4), c0 = 4 * (p % (DK / 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.G2[row * LD + c0 + e] = xl[u][e];
        }
    } else {
        for (int idx = tid; idx < BT * DK; idx += NTH) {
            const int row = idx / DK, col = idx % DK;
            const int t = t0 + row;
            float kv = 0.f, qv = 0.f, bv = 0.f, lv = 0.f;
            if (t < T) {
                const long off = ((b * T + t) * H + h) * (long)DK + col;
                kv = load_elem(k + off);
                qv = load_elem(q + off);
                bv = load_elem(bg + off);
                lv = la[off];
            }
            sm.u.in.K[row * LD + col] = kv;
            sm.u.in.Q[row * LD + col] = qv;
            sm.u.in.E[row * LD + col] = bv * kv;
            sm.G2[row * LD + col] = lv;
        }
    }
    __syncthreads();
    // 2. chunk-local cumsum per channel (fp64 running sum), times log2(e)
    if (tid < DK) {
        double acc = 0.0;
        for (int i = 0; i < BT; ++i) {
            acc += sm.G2[i * LD + tid];
            sm.G2[i * LD + tid] = (float)(acc * 1.4426950408889634);
        }
    }
    __syncthreads();
    // 3. decayed operands for the walk
    const long obase = chunk * (long)BT * DK;
    for (int idx = tid; idx < BT * DK; idx += NTH) {
        const int row = idx / DK, col = idx % DK;
        const float G = sm.G2[row * LD + col], GL = sm.G2[(BT - 1) * LD + col];
        const float gam = exp2f(G);
        Ehat[obase + idx] = to_mt<mt>(sm.u.in.E[row * LD + col] * gam);
        Qhat[obase + idx] = to_mt<mt>(sm.u.in.Q[row * LD + col] * gam);
        Khat[obase + idx] = to_mt<mt>(sm.u.in.K[row * LD + col] * exp2f(GL - G));
        if (row == 0) GamC[chunk * DK + col] = exp2f(GL);
    }
    // 4a. zero the diagonal blocks of A (the diagonal jobs fill their lower part)
    for (int idx = tid; idx < 4 * 256; idx += NTH) {
        const int blk = idx >> 8, i = (idx >> 4) & 15, j = idx & 15;
        sm.A[(16 * blk + i) * LDA + 16 * blk + j] = 0.f;
    }
    float *Pc = Pout + chunk * (BT * BT);
    for (int idx = tid; idx < BT * BT; idx += NTH) Pc[idx] = 0.f;
    __syncthreads();
    // 4b. A and P on fp32 MFMA with anchored decay factors.  Jobs 0 .. 3 are
    // the diagonal blocks (A and P together, gdn2_intra_diag), jobs 4 .. 15
    // the six off-diagonal tiles of A and of P, anchored at the first row a
    // of their block row: 2^(G2_i - G2_j) = 2^(G2_i - G2_a) 2^(G2_a - G2_j),
    // both factors <= 1 because j < a <= i.  Waves w and w + 4 share a SIMD
    // and get equal work (a diagonal block costs about one and a half tiles).
    float *Dc = Dout + chunk * BT;
    for (int job = wave; job < 16; job += 8) {
        if (job < 4) {
            gdn2_intra_diag<Pol, DK>(sm, 16 * job, lane, Pc, Dc);
            continue;
        }
        const int tile = (job - 4) % 6;
        const bool isP = job - 4 >= 6;
        const int I = t2I(tile), J = t2J(tile);
        const int a = 16 * I;  // anchor row
        const float *src = isP ? sm.u.in.Q : sm.u.in.E;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += 32) {
            mt fa[8], fb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int cc = kk + (e >> 2) * 16 + 4 * g + (e & 3);
                const int i = 16 * I + r, j = 16 * J + r;
                const float Ga = sm.G2[a * LD + cc];
                fa[e] = to_mt<mt>(src[i * LD + cc] * exp2f(sm.G2[i * LD + cc] - Ga));
                fb[e] = to_mt<mt>(sm.u.in.K[j * LD + cc] * exp2f(Ga - sm.G2[j * LD + cc]));
            }
            acc = mma_slab(acc, fa, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e, j = 16 * J + r;
            if (isP) Pc[i * BT + j] = acc[e];
            else sm.A[i * LDA + j] = acc[e];
        }
    }
    __syncthreads();
    // 5. T = (I + A)^-1: diagonal blocks by forward substitution, then the
    // off-diagonal blocks one sub-diagonal at a time on fp32 MFMA.
    if (wave == 0) {
        const int bb = lane >> 4, cc = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == cc) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= sm.A[(16 * bb + i) * LDA + 16 * bb + j] * x[j];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.u.Tm[(16 * bb + i) * LDA + 16 * bb + cc] = x[i];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int J = wave, I = wave + d;
            f32x4 m = zero4();
            for (int K = J; K < I; ++K) {
                float fa[4], fb[4];
                frag_rows4(fa, sm.A, LDA, 16 * I, 16 * K, lane);
                frag_cols4(fb, sm.u.Tm, LDA, 16 * K, 16 * J, lane);
                m = mma_block_f32(m, fa, fb);
            }
            float fa[4], fb[4];
            frag_rows4(fa, sm.u.Tm, LDA, 16 * I, 16 * I, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) fb[e] = m[e];
            const f32x4 res = mma_block_f32(zero4(), fa, fb);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.Tm[(16 * I + 4 * g + e) * LDA + 16 * J + r] = -res[e];
        }
        __syncthreads();
    }
    float *Tc = Tout + chunk * (BT * BT);
    for (int idx = tid; idx < BT * BT; idx += NTH) {
        const int i = idx >> 6, j = idx & 63;
        Tc[idx] = (i > j) ? sm.u.Tm[i * LDA + j] : 0.f;
    }
}

// OUT = false: the backward's recompute, which needs only the chunk entry
// states (no Qhat S, no P Vnew, no output).
template <class Pol, int DK, int DV, int BV, bool OUT = true>
__global__ __launch_bounds__(BV * 4) void gdn2_walk_kernel(
    const typename Pol::mt *__restrict__ Ehat, const typename Pol::mt *__restrict__ Qhat,
    const typename Pol::mt *__restrict__ Khat, const float *__restrict__ GamC, const float *__restrict__ Tws,
    const float *__restrict__ Pws, const float *__restrict__ Dws, const typename Pol::in_t *__restrict__ v,
    const typename Pol::in_t *__restrict__ wg, const float *__restrict__ h0, float *__restrict__ o,
    float *__restrict__ ht, float *__restrict__ ck, int T, int H, int NT, float scale) {
    using mt = typename Pol::mt;
    constexpr int NW = BV / 16;
    constexpr int NTHR = NW * 64;
    constexpr int NKB = DK / 16;
    constexpr int LDQ = DK + 8;
    constexpr int LDKT = BT + 8;
    constexpr int LDP = BT + 8;
    constexpr int QN = OUT ? BT * LDQ : 1, PN = OUT ? BT * LDP : 1;
    __shared__ mt sE[BT * LDQ], sQ[QN], sKt[DK * LDKT], sP[PN], sT[BT * LDP];
    __shared__ float sDiag[BT], sGam[DK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    constexpr int NTILE = DV / BV;
    const int vt = blockIdx.x % NTILE;
    const long bh = blockIdx.x / NTILE;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int col = vt * BV + wave * 16 + r;

    for (int idx = tid; idx < PN; idx += NTHR) sP[idx] = to_mt<mt>(0.f);
    f32x4 S[NKB];
    const long sbase = bh * (long)DK * DV;
#pragma unroll
    for (int m = 0; m < NKB; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][e] = h0 ? h0[sbase + (long)(16 * m + 4 * g + e) * DV + col] : 0.f;

    for (int c = 0; c < NT; ++c) {
        const int t0 = c * BT;
        const long cb = bh * NT + c;
        const long ob = cb * (long)BT * DK;
        if (ck) {  // entry state of chunk c (for the backward)
#pragma unroll
            for (int m = 0; m < NKB; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) ck[cb * DK * DV + (long)(16 * m + 4 * g + e) * DV + col] = S[m][e];
        }
        if (OUT) {
            for (int idx = tid; idx < BT * DK; idx += NTHR) {
                const int row = idx / DK, kc = idx % DK;
                sE[row * LDQ + kc] = Ehat[ob + idx];
                sQ[row * LDQ + kc] = Qhat[ob + idx];
                sKt[kc * LDKT + row] = Khat[ob + idx];
            }
            for (int idx = tid; idx < BT * BT; idx += NTHR) {
                const int i = idx >> 6, j = idx & 63;
                sT[i * LDP + j] = to_mt<mt>(Tws[cb * (BT * BT) + idx]);
                if (j < i) sP[i * LDP + j] = to_mt<mt>(Pws[cb * (BT * BT) + idx]);
            }
        } else {
            // fp32 operands only (the recompute): float4 loads, all issued
            // before their LDS stores
            constexpr int UE = BT * DK / 4 / NTHR, UT = BT * BT / 4 / NTHR;
            float4 xe[UE], xk[UE], xt[UT];
#pragma unroll
            for (int u = 0; u < UE; ++u) {
                xe[u] = *(const float4 *)((const float *)Ehat + ob + 4 * (tid + NTHR * u));
                xk[u] = *(const float4 *)((const float *)Khat + ob + 4 * (tid + NTHR * u));
            }
#pragma unroll
            for (int u = 0; u < UT; ++u) xt[u] = *(const float4 *)(Tws + cb * (BT * BT) + 4 * (tid + NTHR * u));
#pragma unroll
            for (int u = 0; u < UE; ++u) {
                const int idx = 4 * (tid + NTHR * u), row = idx / DK, kc = idx % DK;
                float *pe = (float *)&sE[row * LDQ + kc];
                pe[0] = xe[u].x; pe[1] = xe[u].y; pe[2] = xe[u].z; pe[3] = xe[u].w;
                float *pk = (float *)sKt;
                pk[(kc + 0) * LDKT + row] = xk[u].x;
                pk[(kc + 1) * LDKT + row] = xk[u].y;
                pk[(kc + 2) * LDKT + row] = xk[u].z;
                pk[(kc + 3) * LDKT + row] = xk[u].w;
            }
#pragma unroll
            for (int u = 0; u < UT; ++u) {
                const int idx = 4 * (tid + NTHR * u), i = idx >> 6, j = idx & 63;
                float *pt = (float *)&sT[i * LDP + j];
                pt[0] = xt[u].x; pt[1] = xt[u].y; pt[2] = xt[u].z; pt[3] = xt[u].w;
            }
        }
        if (OUT && tid < BT) sDiag[tid] = Dws[cb * BT + tid];
        for (int idx = tid; idx < DK; idx += NTHR) sGam[idx] = GamC[cb * DK + idx];
        __syncthreads();

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
                frag_rows(a, sE, LDQ, 16 * I, 32 * s, lane);
                X[I] = mma_slab(X[I], a, sb);
                if (OUT) {
                    frag_rows(a, sQ, LDQ, 16 * I, 32 * s, lane);
                    Y[I] = mma_slab(Y[I], a, sb);
                }
            }
        }
        // R = w . v - Ehat S
        f32x4 R[4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 16 * I + 4 * g + e;
                float z = 0.f;
                if (t < T) {
                    const long off = ((b * T + t) * H + h) * (long)DV + col;
                    z = load_elem(wg + off) * load_elem(v + off);
                }
                R[I][e] = z - X[I][e];
            }
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
        mt vf[2][8];
        frag_from_acc(vf[0], Vn[0], Vn[1]);
        frag_from_acc(vf[1], Vn[2], Vn[3]);
#pragma unroll
        for (int I = 0; I < (OUT ? 4 : 0); ++I) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = Y[I][e] + sDiag[16 * I + 4 * g + e] * Vn[I][e];
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
        // S = Diag(Gamma_C) S + Khat^T Vnew (the decay scales key rows)
#pragma unroll
        for (int m = 0; m < NKB; ++m) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = S[m][e] * sGam[16 * m + 4 * g + e];
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
static hipError_t launch_gdn2_intra_t(const void *q, const void *k, const float *la, const void *bg, void *Ehat,
                                      void *Qhat, void *Khat, float *GamC, float *Tinv, float *P, float *D, int B,
                                      int T, int H, hipStream_t st) {
    using in_t = typename Pol::in_t;
    using mt = typename Pol::mt;
    const int NT = (T + BT - 1) / BT;
    hipLaunchKernelGGL((gdn2_intra_kernel<Pol, DK>), dim3((unsigned)((long)B * H * NT)), dim3(512), 0, st,
                       (const in_t *)q, (const in_t *)k, la, (const in_t *)bg, (mt *)Ehat, (mt *)Qhat, (mt *)Khat,
                       GamC, Tinv, P, D, T, H, NT);
    return hipGetLastError();
}

hipError_t launch_gdn2_intra(const void *q, const void *k, const float *la, const void *bg, void *Ehat, void *Qhat,
                             void *Khat, float *GamC, float *Tinv, float *P, float *D, int B, int T, int H, int Dk,
                             bool bf16, hipStream_t st) {
    if (bf16) {
        if (Dk == 64) return launch_gdn2_intra_t<PolBF16, 64>(q, k, la, bg, Ehat, Qhat, Khat, GamC, Tinv, P, D, B, T, H, st);
        return launch_gdn2_intra_t<PolBF16, 128>(q, k, la, bg, Ehat, Qhat, Khat, GamC, Tinv, P, D, B, T, H, st);
    }
    if (Dk == 64) return launch_gdn2_intra_t<PolF32, 64>(q, k, la, bg, Ehat, Qhat, Khat, GamC, Tinv, P, D, B, T, H, st);
    return launch_gdn2_intra_t<PolF32, 128>(q, k, la, bg, Ehat, Qhat, Khat, GamC, Tinv, P, D, B, T, H, st);
}

template <class Pol, int DK, int DV>
static hipError_t launch_gdn2_walk_t(const void *Ehat, const void *Qhat, const void *Khat, const float *GamC,
                                     const float *Tinv, const float *P, const float *D, const void *v,
                                     const void *wg, const float *h0, float *o, float *ht, int B, int T, int H,
                                     float scale, hipStream_t st) {
    constexpr int BV = 32;
    using in_t = typename Pol::in_t;
    using mt = typename Pol::mt;
    const int NT = (T + BT - 1) / BT;
    hipLaunchKernelGGL((gdn2_walk_kernel<Pol, DK, DV, BV>), dim3((unsigned)((long)B * H * (DV / BV))),
                       dim3(BV * 4), 0, st, (const mt *)Ehat, (const mt *)Qhat, (const mt *)Khat, GamC, Tinv, P, D,
                       (const in_t *)v, (const in_t *)wg, h0, o, ht, (float *)nullptr, T, H, NT, scale);
    return hipGetLastError();
}

hipError_t launch_gdn2_walk(const void *Ehat, const void *Qhat, const void *Khat, const float *GamC,
                            const float *Tinv, const float *P, const float *D, const void *v, const void *wg,
                            const float *h0, float *o, float *ht, int B, int T, int H, int Dk, int Dv, bool bf16,
                            float scale, hipStream_t st) {
#define GDN2_WALK(P_, DKv, DVv)                                                                                  \
    if (Dk == DKv && Dv == DVv)                                                                                 \
    return launch_gdn2_walk_t<P_, DKv, DVv>(Ehat, Qhat, Khat, GamC, Tinv, P, D, v, wg, h0, o, ht, B, T, H, scale, \
                                            st)
    if (bf16) {
        GDN2_WALK(PolBF16, 64, 64);
        GDN2_WALK(PolBF16, 64, 128);
        GDN2_WALK(PolBF16, 128, 64);
        GDN2_WALK(PolBF16, 128, 128);
    } else {
        GDN2_WALK(PolF32, 64, 64);
        GDN2_WALK(PolF32, 64, 128);
        GDN2_WALK(PolF32, 128, 64);
        GDN2_WALK(PolF32, 128, 128);
    }
#undef GDN2_WALK
    return hipErrorInvalidValue;
}

// The forward recompute of the backward: the intra stage and the walk in fp32
// operands (bf16 inputs are exact in fp32), the walk writing every chunk's
// entry state into ck [B, H, NT, Dk, Dv] and no output.
template <class Pol, int DK, int DV>
static hipError_t launch_gdn2_recompute_t(const void *q, const void *k, const float *la, const void *bg,
                                          const void *v, const void *wg, const float *h0, float *Eh, float *Qh,
                                          float *Kh, float *GamC, float *Tinv, float *P, float *D, float *ck, int B,
                                          int T, int H, hipStream_t st) {
    constexpr int BV = 32;
    static_assert(std::is_same<typename Pol::mt, float>::value, "the recompute runs on fp32 operands");
    using in_t = typename Pol::in_t;
    hipError_t e = launch_gdn2_intra_t<Pol, DK>(q, k, la, bg, Eh, Qh, Kh, GamC, Tinv, P, D, B, T, H, st);
    if (e != hipSuccess) return e;
    if (std::is_same<in_t, uint16_t>::value)
        return launch_gdn2_states_bf16(Eh, Kh, Tinv, GamC, v, wg, h0, ck, B, T, H, DK, DV, st);
    const int NT = (T + BT - 1) / BT;
    hipLaunchKernelGGL((gdn2_walk_kernel<Pol, DK, DV, BV, false>), dim3((unsigned)((long)B * H * (DV / BV))), dim3(BV * 4),
                       0, st, (const float *)Eh, (const float *)Qh, (const float *)Kh, GamC, Tinv, P, D,
                       (const in_t *)v, (const in_t *)wg, h0, (float *)nullptr, (float *)nullptr, ck, T, H, NT, 1.f);
    return hipGetLastError();
}

hipError_t launch_gdn2_recompute(const void *q, const void *k, const float *la, const void *bg, const void *v,
                                 const void *wg, const float *h0, float *Eh, float *Qh, float *Kh, float *GamC,
                                 float *Tinv, float *P, float *D, float *ck, int B, int T, int H, int Dk, int Dv,
                                 bool bf16, hipStream_t st) {
#define GDN2_RC(P_, DKv, DVv)                                                                                  \
    if (Dk == DKv && Dv == DVv)                                                                               \
    return launch_gdn2_recompute_t<P_, DKv, DVv>(q, k, la, bg, v, wg, h0, Eh, Qh, Kh, GamC, Tinv, P, D, ck, B, T, H, st)
    if (bf16) {
        GDN2_RC(PolBF16F32, 64, 64);
        GDN2_RC(PolBF16F32, 64, 128);
        GDN2_RC(PolBF16F32, 128, 64);
        GDN2_RC(PolBF16F32, 128, 128);
    } else {
        GDN2_RC(PolF32, 64, 64);
        GDN2_RC(PolF32, 64, 128);
        GDN2_RC(PolF32, 128, 64);
        GDN2_RC(PolF32, 128, 128);
    }
#undef GDN2_RC
    return hipErrorInvalidValue;
}

}  // namespace gdn
