// gdn2_states.hip -- the state entering every chunk of the chunked Gated
// DeltaNet-2 forward, for its backward with bf16 inputs, on split 16-bit MFMA
// operands.
//
// Per chunk (the chunked-training form in the Gated DeltaNet-2 article,
// section "Regla-2 del Delta cerrado"), from the intra
// stage's fp32 operands Ehat = Gamma . b . k, Khat_j = k_j . Gamma_C / Gamma_j,
// T - I and Gamma_C:
//   X = Ehat S,  R = w . v - X,  Vnew = R + (T - I) R,
//   S' = Diag(Gamma_C) S + Khat^T Vnew.
// Precision: Ehat and Khat enter as bf16 hi + lo parts and so do the state
// (in Ehat S) and Vnew (in Khat^T Vnew); T - I and R enter as fp16 hi + lo
// parts.  Each product is hi.hi + hi.lo + lo.hi, about 16 bits (bf16) and 22
// bits (fp16) of each operand; accumulation and the state are fp32.
//
// One workgroup per (batch, head, 32 value columns), six waves: waves 0 and 1
// carry 16 state columns each in MFMA accumulators, waves 2 .. 5 fetch the
// next chunk into registers, split it and store it into LDS.  Each chunk has
// two phases split by a barrier: in the first the consumers use Ehat, T - I,
// v and w (one LDS copy) while the loaders store the next chunk's Khat (two
// copies); in the second the consumers use Khat while the loaders refill the
// single copy with the next chunk's Ehat, T - I, v and w.
#include "gdn_launch.h"
#include "gdn_tile.h"

namespace gdn {

namespace {

template <int DK>
struct G2sCfg {
    static constexpr int BV = 32;                   // value columns per workgroup
    static constexpr int LDP = BT + 8;              // fp16 rows of T - I (16-byte aligned)
    static constexpr int LDV = BV + 8;              // bf16 rows of the v and w slices
    static constexpr int NLT = 4 * 64;              // loader threads
    static constexpr int UE = BT * DK / 4 / NLT;    // f32x4 of Ehat (and of Khat) per loader thread
    static constexpr int UT = BT * BT / 4 / NLT;    // f32x4 of T - I
    static constexpr int UG = DK / 4;               // f32x4 of Gamma_C (threads below UG)
    static constexpr int NKB = DK / 16;
};

template <int DK>
struct G2sSmem {
    using C = G2sCfg<DK>;
    alignas(16) uint16_t Eh[BT * DK], El[BT * DK];   // bf16 hi / lo of Ehat, paired-group layout
    alignas(16) _Float16 Th[BT * C::LDP], Tl[BT * C::LDP];
    alignas(16) uint16_t V[BT * C::LDV], W[BT * C::LDV];
    alignas(16) uint16_t Kh[2][BT * DK], Kl[2][BT * DK];
    alignas(16) float gam[2][DK];
};

// One chunk's operands in a loader thread's registers.
template <int DK>
struct G2sStage {
    using C = G2sCfg<DK>;
    f32x4 e[C::UE], k[C::UE], t[C::UT], gm;
    u32x4 v, w;
};

struct G2sHead {
    const float *E, *K, *Tm, *G;   // this head's chunk 0 in each intra-stage array
    const uint16_t *v, *w;
    long row0;                     // token-head row of token 0
    int T, H, DV, vcol0;
};

template <int DK>
__device__ __forceinline__ void g2s_fetch(G2sStage<DK> &R, const G2sHead &hd, int c, int lt) {
    using C = G2sCfg<DK>;
    const long eo = (long)c * BT * DK;
#pragma unroll
    for (int u = 0; u < C::UE; ++u) {
        R.e[u] = *(const f32x4 *)(hd.E + eo + 4 * (lt + C::NLT * u));
        R.k[u] = *(const f32x4 *)(hd.K + eo + 4 * (lt + C::NLT * u));
    }
#pragma unroll
    for (int u = 0; u < C::UT; ++u) R.t[u] = *(const f32x4 *)(hd.Tm + (long)c * BT * BT + 4 * (lt + C::NLT * u));
    R.gm = (lt < C::UG) ? *(const f32x4 *)(hd.G + (long)c * DK + 4 * lt) : (f32x4){0.f, 0.f, 0.f, 0.f};
    // v and w: 64 rows x 32 columns of bf16 = one 16-byte piece per thread
    const int row = lt >> 2, c4 = lt & 3;
    const int t = c * BT + row;
    const long off = (hd.row0 + (long)t * hd.H) * hd.DV + hd.vcol0 + 8 * c4;
    const bool in = t < hd.T;
    R.v = in ? *(const u32x4 *)(hd.v + off) : (u32x4){0u, 0u, 0u, 0u};
    R.w = in ? *(const u32x4 *)(hd.w + off) : (u32x4){0u, 0u, 0u, 0u};
}

// Four consecutive fp32 values as hi and lo parts in the 16-bit type of V2.
template <class V2>
__device__ __forceinline__ void split4(uint2 &h, uint2 &l, const f32x4 &x) {
    V2 h0, l0, h1, l1;
    split_pair(h0, l0, x[0], x[1]);
    split_pair(h1, l1, x[2], x[3]);
    h = make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
    l = make_uint2(__builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1));
}

// Rows of a [64][DK] fp32 block (4 columns per piece) as bf16 hi / lo
// paired-group tiles.
template <int DK>
__device__ __forceinline__ void g2s_put_rows(uint16_t *hi, uint16_t *lo, const f32x4 (&x)[G2sCfg<DK>::UE], int lt) {
    using C = G2sCfg<DK>;
#pragma unroll
    for (int u = 0; u < C::UE; ++u) {
        const int idx = 4 * (lt + C::NLT * u), row = idx / DK, col = idx % DK;
        const int o = tile_off_pg<DK>(row, pair_col(col));
        uint2 h, l;
        split4<bf16x2>(h, l, x[u]);
        *(uint2 *)&hi[o] = h;
        *(uint2 *)&lo[o] = l;
    }
}

// Phase one of the loaders: Khat and Gamma_C of the staged chunk into copy b.
template <int DK>
__device__ __forceinline__ void g2s_store_k(G2sSmem<DK> &sm, const G2sStage<DK> &R, int b, int lt) {
    using C = G2sCfg<DK>;
    g2s_put_rows<DK>(sm.Kh[b], sm.Kl[b], R.k, lt);
    if (lt < C::UG) *(f32x4 *)&sm.gam[b][4 * lt] = R.gm;
}

// Phase two: Ehat, T - I, v and w of the staged chunk.
template <int DK>
__device__ __forceinline__ void g2s_store_rest(G2sSmem<DK> &sm, const G2sStage<DK> &R, int lt) {
    using C = G2sCfg<DK>;
    g2s_put_rows<DK>(sm.Eh, sm.El, R.e, lt);
#pragma unroll
    for (int u = 0; u < C::UT; ++u) {
        const int idx = 4 * (lt + C::NLT * u), row = idx / BT, col = idx % BT;
        const f16x4 h = __builtin_convertvector(R.t[u], f16x4);
        const f16x4 l = __builtin_convertvector(R.t[u] - __builtin_convertvector(h, f32x4), f16x4);
        *(f16x4 *)&sm.Th[row * C::LDP + col] = h;
        *(f16x4 *)&sm.Tl[row * C::LDP + col] = l;
    }
    const int row = lt >> 2, c4 = lt & 3;
    *(u32x4 *)&sm.V[row * C::LDV + 8 * c4] = R.v;
    *(u32x4 *)&sm.W[row * C::LDV + 8 * c4] = R.w;
}

// Consumer phase one: Vnew of this wave's 16 columns (rows 16 I + 4 g + e,
// column r) from the state S.
template <int DK>
__device__ __forceinline__ void g2s_vnew(G2sSmem<DK> &sm, const f32x4 (&S)[DK / 16], f32x4 (&Vn)[4], int wave,
                                         int lane) {
    using C = G2sCfg<DK>;
    const int r = lane & 15, g = lane >> 4;
    const int cl = wave * 16 + r;
    f32x4 wv[4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            wv[I][e] = bf16_to_f32(sm.W[i * C::LDV + cl]) * bf16_to_f32(sm.V[i * C::LDV + cl]);
        }
    // X = Ehat S
    f32x4 X[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) X[I] = zero4();
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        uint4 sh, sl;
        hilo_frags<bf16x2>(sh, sl, S[2 * s], S[2 * s + 1]);
        uint4 eh[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            eh[I] = frag_rows_pg<DK>(sm.Eh, 16 * I, 32 * s, lane);
            X[I] = mma_bf16_raw(X[I], eh[I], sh);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) X[I] = mma_bf16_raw(X[I], eh[I], sl);
#pragma unroll
        for (int I = 0; I < 4; ++I) X[I] = mma_bf16_raw(X[I], frag_rows_pg<DK>(sm.El, 16 * I, 32 * s, lane), sh);
    }
    f32x4 R[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) R[I] = wv[I] - X[I];
    // Vnew = R + (T - I) R on fp16 hi + lo parts of both
    _Float16 rh[2][8], rl[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        frag_from_acc(rh[s], R[2 * s], R[2 * s + 1]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rl[s][e] = (_Float16)(R[2 * s][e] - (float)rh[s][e]);
            rl[s][e + 4] = (_Float16)(R[2 * s + 1][e] - (float)rh[s][e + 4]);
        }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        Vn[I] = R[I];
#pragma unroll
        for (int s = 0; s <= (I >> 1); ++s) {
            _Float16 a[8], al[8];
            frag_rows(a, sm.Th, C::LDP, 16 * I, 32 * s, lane);
            frag_rows(al, sm.Tl, C::LDP, 16 * I, 32 * s, lane);
            Vn[I] = mma_slab(Vn[I], a, rh[s]);
            Vn[I] = mma_slab(Vn[I], a, rl[s]);
            Vn[I] = mma_slab(Vn[I], al, rh[s]);
        }
    }
}

// Consumer phase two: S = Diag(Gamma_C) S + Khat^T Vnew with copy b of Khat.
template <int DK>
__device__ __forceinline__ void g2s_update(G2sSmem<DK> &sm, f32x4 (&S)[DK / 16], const f32x4 (&Vn)[4], int b,
                                           int lane) {
    const int g = lane >> 4;
    uint4 vh[2], vl[2];
    hilo_frags<bf16x2>(vh[0], vl[0], Vn[0], Vn[1]);
    hilo_frags<bf16x2>(vh[1], vl[1], Vn[2], Vn[3]);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
        const f32x4 gm = *(const f32x4 *)&sm.gam[b][16 * m + 4 * g];
        f32x4 acc = S[m] * gm;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 kh = frag_T_pg<DK>(sm.Kh[b], 32 * s, 16 * m, lane);
            const uint4 kl = frag_T_pg<DK>(sm.Kl[b], 32 * s, 16 * m, lane);
            acc = mma_bf16_raw(acc, kh, vh[s]);
            acc = mma_bf16_raw(acc, kh, vl[s]);
            acc = mma_bf16_raw(acc, kl, vh[s]);
        }
        S[m] = acc;
    }
}

}  // namespace

// ck[b, h, c] ([DK][DV] fp32) = the state entering chunk c of (b, h).  Eh, Kh:
// fp32 [B, H, NT, 64, DK]; Tws: T - I, fp32 [B, H, NT, 64, 64]; GamC: fp32
// [B, H, NT, DK]; v, w: bf16 [B, T, H, DV]; h0: fp32 [B, H, DK, DV] or null.
template <int DK, int DV>
__global__ __launch_bounds__(384, 1) void gdn2_states_kernel(const float *__restrict__ Eh, const float *__restrict__ Kh,
                                                             const float *__restrict__ Tws,
                                                             const float *__restrict__ GamC,
                                                             const uint16_t *__restrict__ v,
                                                             const uint16_t *__restrict__ w,
                                                             const float *__restrict__ h0, float *__restrict__ ck,
                                                             int T, int H, int NT) {
    static_assert(sizeof(G2sSmem<DK>) <= 160 * 1024, "LDS budget");
    using C = G2sCfg<DK>;
    __shared__ G2sSmem<DK> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    constexpr int NTILE = DV / C::BV;
    const int n = blockIdx.x, nwg = gridDim.x;
    // the column slices of one head get consecutive ids on one XCD (shared L2)
    const int L = (nwg % 8 == 0) ? (n % 8) * (nwg / 8) + n / 8 : n;
    const int vt = L % NTILE;
    const long bh = L / NTILE;
    const long sbase = bh * (long)DK * DV;

    if (wave < 2) {
        f32x4 S[C::NKB];
        const int col = vt * C::BV + wave * 16 + r;
#pragma unroll
        for (int m = 0; m < C::NKB; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = h0 ? h0[sbase + (long)(16 * m + 4 * g + e) * DV + col] : 0.f;
        __syncthreads();
        for (int c = 0; c < NT; ++c) {
            // the state entering chunk c, as 16-byte row pieces after a quad transpose
            float *dst = ck + (bh * NT + c) * (long)DK * DV + vt * C::BV + wave * 16 + 4 * (r >> 2);
#pragma unroll
            for (int m = 0; m < C::NKB; ++m)
                *(f32x4 *)&dst[(long)(16 * m + 4 * g + (r & 3)) * DV] = quad_transpose(S[m], lane);
            f32x4 Vn[4];
            g2s_vnew<DK>(sm, S, Vn, wave, lane);
            __syncthreads();
            g2s_update<DK>(sm, S, Vn, c & 1, lane);
            __syncthreads();
        }
    } else {
        const int lt = tid - 128;
        G2sHead hd;
        hd.E = Eh + bh * NT * (long)BT * DK;
        hd.K = Kh + bh * NT * (long)BT * DK;
        hd.Tm = Tws + bh * NT * (long)BT * BT;
        hd.G = GamC + bh * NT * (long)DK;
        hd.v = v;
        hd.w = w;
        hd.row0 = (bh / H) * (long)T * H + (bh % H);
        hd.T = T;
        hd.H = H;
        hd.DV = DV;
        hd.vcol0 = vt * C::BV;
        G2sStage<DK> R;
        if (NT > 0) {
            g2s_fetch<DK>(R, hd, 0, lt);
            g2s_store_k<DK>(sm, R, 0, lt);
            g2s_store_rest<DK>(sm, R, lt);
            if (NT > 1) g2s_fetch<DK>(R, hd, 1, lt);
        }
        __syncthreads();
        for (int c = 0; c < NT; ++c) {
            if (c + 1 < NT) g2s_store_k<DK>(sm, R, (c + 1) & 1, lt);
            __syncthreads();
            if (c + 1 < NT) {
                g2s_store_rest<DK>(sm, R, lt);
                if (c + 2 < NT) g2s_fetch<DK>(R, hd, c + 2, lt);
            }
            __syncthreads();
        }
    }
}

template <int DK, int DV>
static hipError_t launch_states_t(const float *Eh, const float *Kh, const float *Tws, const float *GamC,
                                  const uint16_t *v, const uint16_t *w, const float *h0, float *ck, int B, int T,
                                  int H, hipStream_t st) {
    const int NT = (T + BT - 1) / BT;
    hipLaunchKernelGGL((gdn2_states_kernel<DK, DV>), dim3((unsigned)((long)B * H * (DV / 32))), dim3(384), 0, st, Eh,
                       Kh, Tws, GamC, v, w, h0, ck, T, H, NT);
    return hipGetLastError();
}

hipError_t launch_gdn2_states_bf16(const float *Eh, const float *Kh, const float *Tws, const float *GamC,
                                   const void *v, const void *w, const float *h0, float *ck, int B, int T, int H,
                                   int Dk, int Dv, hipStream_t st) {
    const uint16_t *vv = (const uint16_t *)v, *ww = (const uint16_t *)w;
    if (Dk == 64 && Dv == 64) return launch_states_t<64, 64>(Eh, Kh, Tws, GamC, vv, ww, h0, ck, B, T, H, st);
    if (Dk == 64 && Dv == 128) return launch_states_t<64, 128>(Eh, Kh, Tws, GamC, vv, ww, h0, ck, B, T, H, st);
    if (Dk == 128 && Dv == 64) return launch_states_t<128, 64>(Eh, Kh, Tws, GamC, vv, ww, h0, ck, B, T, H, st);
    if (Dk == 128 && Dv == 128) return launch_states_t<128, 128>(Eh, Kh, Tws, GamC, vv, ww, h0, ck, B, T, H, st);
    return hipErrorInvalidValue;
}

}  // namespace gdn
