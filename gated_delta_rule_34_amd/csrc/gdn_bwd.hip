// gdn_bwd.hip -- backward of the chunked Gated DeltaNet forward on gfx950.
// fp32 inputs: fp32 arithmetic on fp32 MFMA.  bf16 inputs: fp32 values and
// accumulation, with the products on bf16 MFMA, exact where an operand is a
// bf16 input and otherwise on bf16 parts (hi + lo, or hi + mid + lo where
// the product needs fp32's precision) of the fp32 operands.
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
//   3. bwd_walk_kernel (bf16 inputs: bwd_walk_fused_kernel in
//      gdn_bwd_fused.hip): dS' chunk by chunk from the last one back (state
//      columns are independent, so one workgroup owns 32 of them), written
//      per chunk; dh0 is the gradient entering the first chunk
//   4. bwd_chunk_kernel (bf16 inputs: bwd_chunk2_kernel, eight waves in two
//      groups): one workgroup per (batch, head, chunk) recomputes the chunk
//      and produces its dq, dk, dv, dbeta, dg, looping over the value
//      columns 16 (32) at a time
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8v;
// 16 bytes as a native vector (arrays of HIP's uint4 struct can be demoted to scratch)
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4b;

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

// acc (the 16x16 tile at rows i0, columns j0 of C) += A B^T over k in
// [0, K) for fp32 LDS rows A[i][k] = A[i * lda + k], B[j][k] = B[j * ldb + k]
// whose values are bf16 numbers (bf16 inputs staged in fp32): one bf16 MFMA
// per 32 k instead of eight fp32 ones, the same result up to fp32 summation
// order.  Lane (g, r) gives both operands k-slots 8g .. 8g + 7 of its row.
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}
// a, b rounded to bf16 (nearest even) in the low and high halves
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <int K>
__device__ __forceinline__ f32x4 tile_mma_bf16rows(f32x4 acc, const float *A, int lda, const float *B, int ldb, int i0,
                                                   int j0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float *pa = A + (i0 + r) * lda + 8 * g;
    const float *pb = B + (j0 + r) * ldb + 8 * g;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const float4 a0 = *(const float4 *)(pa + k0), a1 = *(const float4 *)(pa + k0 + 4);
        const float4 b0 = *(const float4 *)(pb + k0), b1 = *(const float4 *)(pb + k0 + 4);
        const uint4 ua = make_uint4(pack_bf16_exact(a0.x, a0.y), pack_bf16_exact(a0.z, a0.w),
                                    pack_bf16_exact(a1.x, a1.y), pack_bf16_exact(a1.z, a1.w));
        const uint4 ub = make_uint4(pack_bf16_exact(b0.x, b0.y), pack_bf16_exact(b0.z, b0.w),
                                    pack_bf16_exact(b1.x, b1.y), pack_bf16_exact(b1.z, b1.w));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, ua), __builtin_bit_cast(bf16x8v, ub),
                                                      acc, 0, 0, 0);
    }
    return acc;
}

// Eight floats as 2 or 3 bf16 parts (hi + lo ~16 bits, hi + mid + lo ~24
// bits), packed in k-slot order for a bf16 MFMA operand.
__device__ __forceinline__ void split_8(u32x4b (&out)[2], const float (&x)[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t h = pack_bf16_rne(x[2 * p], x[2 * p + 1]);
        out[0][p] = h;
        out[1][p] = pack_bf16_rne(x[2 * p] - bf16_lo(h), x[2 * p + 1] - bf16_hi(h));
    }
}
__device__ __forceinline__ void split_8(u32x4b (&out)[3], const float (&x)[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t h = pack_bf16_rne(x[2 * p], x[2 * p + 1]);
        const float r0 = x[2 * p] - bf16_lo(h), r1 = x[2 * p + 1] - bf16_hi(h);
        const uint32_t m = pack_bf16_rne(r0, r1);
        out[0][p] = h;
        out[1][p] = m;
        out[2][p] = pack_bf16_rne(r0 - bf16_lo(m), r1 - bf16_hi(m));
    }
}
__device__ __forceinline__ f32x4 mma_bf16v(f32x4 acc, const u32x4b &a, const u32x4b &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), acc,
                                                   0, 0, 0);
}

// acc += A B over k in [0, K), A = fp32 LDS rows holding bf16 numbers (row
// stride lda), B given as NP bf16 parts per 32-deep block (k-slots
// 32 kb + 8g .. + 7 of this lane's column).
template <int K, int NP>
__device__ __forceinline__ f32x4 mma_rows_parts(f32x4 acc, const float *A, int lda, int i0,
                                                const u32x4b (&bp)[K / 32][NP], int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float *pa = A + (i0 + r) * lda + 8 * g;
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
        const float4 a0 = *(const float4 *)(pa + 32 * kb), a1 = *(const float4 *)(pa + 32 * kb + 4);
        const u32x4b ua = {pack_bf16_exact(a0.x, a0.y), pack_bf16_exact(a0.z, a0.w), pack_bf16_exact(a1.x, a1.y),
                           pack_bf16_exact(a1.z, a1.w)};
#pragma unroll
        for (int q = 0; q < NP; ++q) acc = mma_bf16v(acc, ua, bp[kb][q]);
    }
    return acc;
}

// Column col of a [K][ld] fp32 LDS matrix as NP bf16 parts per 32-deep
// block, k-slots 32 kb + 8g .. + 7.
template <int K, int NP>
__device__ __forceinline__ void col_parts(u32x4b (&bp)[K / 32][NP], const float *M, int ld, int col, int lane) {
    const int g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = M[(32 * kb + 8 * g + e) * ld + col];
        split_8(bp[kb], x);
    }
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
__device__ __forceinline__ void load_chunk_qk(float *sQ, float *sK, double *sG2, float *sGam, float *sDec, float *sBeta,
                                              const typename Pol::in_t *q, const typename Pol::in_t *k,
                                              const float *beta, const double *G2ws, long b, int h, int c, long cb,
                                              int T, int H, int tid) {
    const int t0 = c * BT;
    stage_rows<DK, LDQ, NTHR>(sQ, q, b, h, t0, T, H, 0, DK, tid);
    stage_rows<DK, LDQ, NTHR>(sK, k, b, h, t0, T, H, 0, DK, tid);
    if (tid < BT) {
        const int t = t0 + tid;
        // fp64 gate sums (see the intra stage): their differences are exact to fp32
        const double G2 = G2ws[cb * BT + tid], G2L = G2ws[cb * BT + BT - 1];
        sG2[tid] = G2;
        sGam[tid] = exp2f((float)G2);
        sDec[tid] = exp2f((float)(G2L - G2));
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

// The raw inputs of one chunk of the reverse walk, held in registers from
// the iteration before the one that stages them (their loads then have a
// whole iteration to arrive).  Rows past T read the last token and are
// zeroed when staged.
template <class In, int DK, int BV, int NTHR>
struct WalkRegs {
    static constexpr int W = sizeof(In) / 2;          // 16-byte pieces per 8 inputs
    static constexpr int UQ = BT * DK / 8 / NTHR;     // 8-input groups per thread (Q, K rows)
    static constexpr int UT = BT * BT / 4 / NTHR;     // float4 per thread (T - I)
    static constexpr int UD = BT * BV / 8 / NTHR;     // 8-float groups per thread (dO)
    u32x4b q[UQ][W], k[UQ][W];
    float4 t[UT];
    float4 d[UD][2];
    double g2, g2L;
    float beta;
};

template <class In, int DK, int BV, int NTHR>
__device__ __forceinline__ void walk_fetch(WalkRegs<In, DK, BV, NTHR> &R, const In *q, const In *k, const float *beta,
                                           const float *dO, const double *G2ws, const float *Tws, long b, int h,
                                           int c, long cb, int T, int H, int vcol0, int DV, int tid) {
    using WR = WalkRegs<In, DK, BV, NTHR>;
    const int t0 = c * BT;
#pragma unroll
    for (int u = 0; u < WR::UQ; ++u) {
        const int idx = tid + NTHR * u, row = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        const long off = ((b * T + min(t0 + row, T - 1)) * H + h) * (long)DK + c8;
#pragma unroll
        for (int w = 0; w < WR::W; ++w) {
            R.q[u][w] = *(const u32x4b *)((const char *)(q + off) + 16 * w);
            R.k[u][w] = *(const u32x4b *)((const char *)(k + off) + 16 * w);
        }
    }
#pragma unroll
    for (int u = 0; u < WR::UT; ++u) R.t[u] = *(const float4 *)(Tws + cb * BT * BT + 4 * (tid + NTHR * u));
#pragma unroll
    for (int u = 0; u < WR::UD; ++u) {
        const int idx = tid + NTHR * u, row = idx / (BV / 8), c8 = 8 * (idx % (BV / 8));
        const float *p = dO + ((b * T + min(t0 + row, T - 1)) * H + h) * (long)DV + vcol0 + c8;
        R.d[u][0] = *(const float4 *)p;
        R.d[u][1] = *(const float4 *)(p + 4);
    }
    if (tid < BT) {
        R.g2 = G2ws[cb * BT + tid];
        R.g2L = G2ws[cb * BT + BT - 1];
        R.beta = beta[(b * T + min(t0 + tid, T - 1)) * H + h];
    }
}

// Eight inputs of a 16-byte piece (bf16) or two (fp32) as floats.
__device__ __forceinline__ void raw8(float (&x)[8], const u32x4b (&u)[1]) {
    const uint32_t w[4] = {u[0][0], u[0][1], u[0][2], u[0][3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void raw8(float (&x)[8], const u32x4b (&u)[2]) {
    const uint32_t w[8] = {u[0][0], u[0][1], u[0][2], u[0][3], u[1][0], u[1][1], u[1][2], u[1][3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(w[e]);
}

template <class In, int DK, int BV, int NTHR, int LDQ, int LDC, int LDB>
__device__ __forceinline__ void walk_stage(const WalkRegs<In, DK, BV, NTHR> &R, float *sQ, float *sK, float *sTm,
                                           float *sdO, double *sG2, float *sGam, float *sDec, float *sBeta, int c,
                                           int T, int tid) {
    using WR = WalkRegs<In, DK, BV, NTHR>;
    const int t0 = c * BT;
#pragma unroll
    for (int u = 0; u < WR::UQ; ++u) {
        const int idx = tid + NTHR * u, row = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        const bool in = t0 + row < T;
        float xq[8], xk[8];
        raw8(xq, R.q[u]);
        raw8(xk, R.k[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sQ[row * LDQ + c8 + e] = in ? xq[e] : 0.f;
            sK[row * LDQ + c8 + e] = in ? xk[e] : 0.f;
        }
    }
#pragma unroll
    for (int u = 0; u < WR::UT; ++u) {
        const int idx = 4 * (tid + NTHR * u), row = idx / BT, col = idx % BT;
        sTm[row * LDC + col] = R.t[u].x;
        sTm[row * LDC + col + 1] = R.t[u].y;
        sTm[row * LDC + col + 2] = R.t[u].z;
        sTm[row * LDC + col + 3] = R.t[u].w;
    }
#pragma unroll
    for (int u = 0; u < WR::UD; ++u) {
        const int idx = tid + NTHR * u, row = idx / (BV / 8), c8 = 8 * (idx % (BV / 8));
        const bool in = t0 + row < T;
        const float x[8] = {R.d[u][0].x, R.d[u][0].y, R.d[u][0].z, R.d[u][0].w,
                            R.d[u][1].x, R.d[u][1].y, R.d[u][1].z, R.d[u][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) sdO[row * LDB + c8 + e] = in ? x[e] : 0.f;
    }
    if (tid < BT) {
        // fp64 gate sums (see the intra stage): their differences are exact to fp32
        sG2[tid] = R.g2;
        sGam[tid] = exp2f((float)R.g2);
        sDec[tid] = exp2f((float)(R.g2L - R.g2));
        sBeta[tid] = (t0 + tid < T) ? R.beta : 0.f;
    }
}

// --------------------------------------------------------- reverse state walk
template <class Pol, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_walk_kernel(const typename Pol::in_t *__restrict__ q,
                                                       const typename Pol::in_t *__restrict__ k,
                                                       const float *__restrict__ beta, const float *__restrict__ dO,
                                                       const float *__restrict__ dht, const double *__restrict__ G2ws,
                                                       const float *__restrict__ Tws, float *__restrict__ dSck,
                                                       float *__restrict__ dh0, int T, int H, int NT, float scale) {
    constexpr int BV = 32, NTHR = 256, LDQ = DK + 4, LDC = BT + 1, LDB = BV + 1;
    __shared__ float sQ[BT * LDQ], sK[BT * LDQ], sTm[BT * LDC], sP[BT * LDC];
    __shared__ float sdO[BT * LDB], sdVn[BT * LDB], sdR[BT * LDB], sdS[DK * LDB];
    __shared__ double sG2[BT];
    __shared__ float sGam[BT], sDec[BT], sBeta[BT], sGdO[BT], sBG[BT];
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
    using In = typename Pol::in_t;
    WalkRegs<In, DK, BV, NTHR> R;
    walk_fetch<In, DK, BV, NTHR>(R, q, k, beta, dO, G2ws, Tws, b, h, NT - 1, bh * NT + NT - 1, T, H, vcol0, DV, tid);
    __syncthreads();

    for (int c = NT - 1; c >= 0; --c) {
        const long cb = bh * NT + c;
        // gradient of the state leaving chunk c, for the per-chunk stage
#pragma unroll
        for (int u = 0; u < DK * BV / 4 / NTHR; ++u) {
            const int idx = 4 * (tid + NTHR * u), row = idx / BV, col = idx % BV;
            const float *p = &sdS[row * LDB + col];
            *(float4 *)(dSck + cb * DK * DV + (long)row * DV + vcol0 + col) = make_float4(p[0], p[1], p[2], p[3]);
        }
        // this chunk's inputs arrived during the previous iteration; the next
        // chunk's (c - 1) are requested now
        walk_stage<In, DK, BV, NTHR, LDQ, LDC, LDB>(R, sQ, sK, sTm, sdO, sG2, sGam, sDec, sBeta, c, T, tid);
        if (c > 0) walk_fetch<In, DK, BV, NTHR>(R, q, k, beta, dO, G2ws, Tws, b, h, c - 1, cb - 1, T, H, vcol0, DV, tid);
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
                sP[i * LDC + j] = (j <= i) ? acc[e] * exp2f((float)(sG2[i] - sG2[j])) : 0.f;
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
    double G2[BT];
    float Gam[BT], Dec[BT], Beta[BT];
    float dB[BT], dG[BT], colG[4][BT], red[256];
};

template <class Pol, int DK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_chunk_kernel(
    const typename Pol::in_t *__restrict__ q, const typename Pol::in_t *__restrict__ k,
    const typename Pol::in_t *__restrict__ v, const float *__restrict__ beta, const float *__restrict__ dO,
    const double *__restrict__ G2ws, const float *__restrict__ Tws, const float *__restrict__ Sck,
    const float *__restrict__ dSck, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
    float *__restrict__ dg, float *__restrict__ dbeta, int T, int H, int NT, float scale) {
    using SM = BwdChunkSmem<DK>;
    constexpr int LDQ = SM::LDQ, LDC = SM::LDC, CW = SM::CW, LDW = SM::LDW, NTHR = 256, NM = DK / 16;
    // bf16 inputs: Q and K hold bf16 numbers, so their products run on bf16 MFMA
    constexpr bool kExact = std::is_same<typename Pol::in_t, uint16_t>::value;
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
        f32x4 acc;
        if constexpr (kExact) acc = tile_mma_bf16rows<DK>(zero4(), sm.Q, LDQ, sm.K, LDQ, 16 * TI, 16 * TJ, lane);
        else acc = tile_mma<DK>(zero4(), sm.Q, LDQ, 1, sm.K, 1, LDQ, nullptr, 16 * TI, 16 * TJ, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * TI + 4 * g + e, j = 16 * TJ + r;
            sm.P[i * LDC + j] = (j <= i) ? acc[e] * exp2f((float)(sm.G2[i] - sm.G2[j])) : 0.f;
        }
    }

    f32x4 dqs[NM], dkR[NM], dKd[NM], dA[4], dP[4];
#pragma unroll
    for (int m = 0; m < NM; ++m) dqs[m] = dkR[m] = dKd[m] = zero4();
#pragma unroll
    for (int j = 0; j < 4; ++j) dA[j] = dP[j] = zero4();
    float dGC = 0.f;  // <dS', S> over the slices this thread loaded

    // The next slice's S, dS', V and dO are requested into registers while
    // the current one is worked on, then staged after the barrier.
    using In = typename Pol::in_t;
    constexpr int US = DK * CW / 4 / NTHR;   // float4 of S (and of dS') per thread
    constexpr int WV = sizeof(In) / 2;       // 16-byte pieces per 8 values of v
    static_assert(BT * CW / 8 == NTHR / 2, "one 8-value piece of v or dO per thread");
    float4 xs[US], xd[US], xo[2];
    u32x4b xv[WV];
    const int prow = (tid & (NTHR / 2 - 1)) / (CW / 8), pc8 = 8 * (tid % (CW / 8));  // this thread's v/dO piece
    const int pt = min(t0 + prow, T - 1);
    auto fetch_slice = [&](int cc) {
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int idx = 4 * (tid + NTHR * u), row = idx / CW, col = idx % CW;
            const long off = cb * DK * DV + (long)row * DV + cc + col;
            xs[u] = *(const float4 *)(Sck + off);
            xd[u] = *(const float4 *)(dSck + off);
        }
        if (tid < NTHR / 2) {
            const In *pv = v + ((b * T + pt) * H + h) * (long)DV + cc + pc8;
#pragma unroll
            for (int w = 0; w < WV; ++w) xv[w] = *(const u32x4b *)((const char *)pv + 16 * w);
        } else {
            const float *po = dO + ((b * T + pt) * H + h) * (long)DV + cc + pc8;
            xo[0] = *(const float4 *)po;
            xo[1] = *(const float4 *)(po + 4);
        }
    };
    // (fp32 inputs fetch each slice just before staging it: the prefetch's
    // registers would not fit beside theirs)
    if constexpr (kExact) fetch_slice(0);

    for (int c0 = 0; c0 < DV; c0 += CW) {
        __syncthreads();  // previous slice fully consumed
        if constexpr (!kExact) fetch_slice(c0);
        {
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int idx = 4 * (tid + NTHR * u), row = idx / CW, col = idx % CW;
                float *ps = &sm.S[row * LDW + col], *pd = &sm.dS[row * LDW + col];
                ps[0] = xs[u].x; ps[1] = xs[u].y; ps[2] = xs[u].z; ps[3] = xs[u].w;
                pd[0] = xd[u].x; pd[1] = xd[u].y; pd[2] = xd[u].z; pd[3] = xd[u].w;
                dGC += xs[u].x * xd[u].x + xs[u].y * xd[u].y + xs[u].z * xd[u].z + xs[u].w * xd[u].w;
            }
            const bool in = t0 + prow < T;  // rows past T are zero
            float x8[8];
            if (tid < NTHR / 2) {
                raw8(x8, xv);
            } else {
                x8[0] = xo[0].x; x8[1] = xo[0].y; x8[2] = xo[0].z; x8[3] = xo[0].w;
                x8[4] = xo[1].x; x8[5] = xo[1].y; x8[6] = xo[1].z; x8[7] = xo[1].w;
            }
            float *dst = (tid < NTHR / 2 ? sm.V : sm.dO) + prow * LDW + pc8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = in ? x8[e] : 0.f;
        }
        if (kExact && c0 + CW < DV) fetch_slice(c0 + CW);
        __syncthreads();
        // KS, QS, R for rows of block I
        f32x4 KS, QS;
        if constexpr (kExact) {
            // K, Q exact in bf16; the S slice as bf16 hi + lo
            u32x4b sp[DK / 32][2];
            col_parts<DK, 2>(sp, sm.S, LDW, r, lane);
            KS = mma_rows_parts<DK, 2>(zero4(), sm.K, LDQ, 16 * I, sp, lane);
            QS = mma_rows_parts<DK, 2>(zero4(), sm.Q, LDQ, 16 * I, sp, lane);
        } else {
            KS = tile_mma<DK>(zero4(), sm.K, LDQ, 1, sm.S, LDW, 1, nullptr, 16 * I, 0, lane);
            QS = tile_mma<DK>(zero4(), sm.Q, LDQ, 1, sm.S, LDW, 1, nullptr, 16 * I, 0, lane);
        }
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
            f32x4 b2;
            if constexpr (kExact) {
                // K exact; dS' as three bf16 parts (K dS' carries the state gradient)
                u32x4b dp[DK / 32][3];
                col_parts<DK, 3>(dp, sm.dS, LDW, r, lane);
                b2 = mma_rows_parts<DK, 3>(zero4(), sm.K, LDQ, 16 * I, dp, lane);
            } else {
                b2 = tile_mma<DK>(zero4(), sm.K, LDQ, 1, sm.dS, LDW, 1, nullptr, 16 * I, 0, lane);
            }
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
        f32x4 KK, QK;
        if constexpr (kExact) {
            KK = tile_mma_bf16rows<DK>(zero4(), sm.K, LDQ, sm.K, LDQ, 16 * I, 16 * J, lane);
            QK = tile_mma_bf16rows<DK>(zero4(), sm.Q, LDQ, sm.K, LDQ, 16 * I, 16 * J, lane);
        } else {
            KK = tile_mma<DK>(zero4(), sm.K, LDQ, 1, sm.K, 1, LDQ, nullptr, 16 * I, 16 * J, lane);
            QK = tile_mma<DK>(zero4(), sm.Q, LDQ, 1, sm.K, 1, LDQ, nullptr, 16 * I, 16 * J, lane);
        }
        const int j = 16 * J + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            const float D = (j <= i) ? exp2f((float)(sm.G2[i] - sm.G2[j])) : 0.f;
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
    // bf16 inputs: the four products on bf16 MFMA.  Their left operands (dA.D,
    // its transpose with beta, dP.D transposed and not) are split once into
    // bf16 parts (three for dP.D, which feeds dq, two for the others); K and Q
    // are bf16 numbers.  Lane (g, r): row 16I + r, k-slots 32 kb + 8g .. + 7.
    u32x4b a1[2][2], a2[2][2], a3[2][2], a4[2][3];
    if constexpr (kExact) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float x1[8], x2[8], x3[8], x4[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = 16 * I + r, j = 32 * kb + 8 * g + e;
                x1[e] = sm.Tm[i * LDC + j];
                x2[e] = sm.Tm[j * LDC + i] * sm.Beta[j];
                x3[e] = sm.P[j * LDC + i];
                x4[e] = sm.P[i * LDC + j];
            }
            split_8(a1[kb], x1);
            split_8(a2[kb], x2);
            split_8(a3[kb], x3);
            split_8(a4[kb], x4);
        }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        f32x4 t1, t2, t3, t4;
        if constexpr (kExact) {
            t1 = t2 = t3 = t4 = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float xk[8], xq[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * kb + 8 * g + e;
                    xk[e] = sm.K[j * LDQ + 16 * m + r];
                    xq[e] = sm.Q[j * LDQ + 16 * m + r];
                }
                const u32x4b bk = {pack_bf16_exact(xk[0], xk[1]), pack_bf16_exact(xk[2], xk[3]),
                                   pack_bf16_exact(xk[4], xk[5]), pack_bf16_exact(xk[6], xk[7])};
                const u32x4b bq = {pack_bf16_exact(xq[0], xq[1]), pack_bf16_exact(xq[2], xq[3]),
                                   pack_bf16_exact(xq[4], xq[5]), pack_bf16_exact(xq[6], xq[7])};
                t1 = mma_bf16v(mma_bf16v(t1, a1[kb][0], bk), a1[kb][1], bk);
                t2 = mma_bf16v(mma_bf16v(t2, a2[kb][0], bk), a2[kb][1], bk);
                t3 = mma_bf16v(mma_bf16v(t3, a3[kb][0], bq), a3[kb][1], bq);
                t4 = mma_bf16v(mma_bf16v(mma_bf16v(t4, a4[kb][0], bk), a4[kb][1], bk), a4[kb][2], bk);
            }
        } else {
            t1 = tile_mma<BT>(zero4(), sm.Tm, LDC, 1, sm.K, LDQ, 1, nullptr, 16 * I, 16 * m, lane);
            t2 = tile_mma<BT>(zero4(), sm.Tm, 1, LDC, sm.K, LDQ, 1, sm.Beta, 16 * I, 16 * m, lane);
            t3 = tile_mma<BT>(zero4(), sm.P, 1, LDC, sm.Q, LDQ, 1, nullptr, 16 * I, 16 * m, lane);
            t4 = tile_mma<BT>(zero4(), sm.P, LDC, 1, sm.K, LDQ, 1, nullptr, 16 * I, 16 * m, lane);
        }
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
    // the Kd terms' total and sum_v dS' . S (both enter the last row's dG):
    // wave sums on shuffles, then the four waves' partials
    float tv = tdec[0] + tdec[1] + tdec[2] + tdec[3], sv = dGC;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        tv += __shfl_xor(tv, off, 64);
        sv += __shfl_xor(sv, off, 64);
    }
    if (lane == 0) {
        sm.red[wave] = tv;
        sm.red[4 + wave] = sv;
    }
    __syncthreads();
    if (wave == 0) {
        // dG_j -= column sums; dg = reverse cumulative sum of dG within the
        // chunk, one row per lane (a suffix scan on shuffles)
        const int i = lane;
        float x = sm.dG[i] - (sm.colG[0][i] + sm.colG[1][i] + sm.colG[2][i] + sm.colG[3][i]);
        if (i == BT - 1)
            x += (sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3]) +
                 sm.Gam[BT - 1] * (sm.red[4] + sm.red[5] + sm.red[6] + sm.red[7]);
#pragma unroll
        for (int off = 1; off < BT; off <<= 1) {
            const float y = __shfl_down(x, off, 64);
            if (i + off < BT) x += y;
        }
        const int t = t0 + i;
        if (t < T) {
            dg[(b * T + t) * H + h] = x;
            dbeta[(b * T + t) * H + h] = sm.dB[i];
        }
    }
}

// ------------------------------------------- per-chunk gradients, bf16 inputs
// The same chunk equations as bwd_chunk_kernel on eight waves in two groups
// of four, so every SIMD runs two waves: each 32-column step of the value
// columns gives the groups 16 columns each for the per-column products (R,
// Vnew, dVnew, dR), and then each group accumulates half of the output tiles
// (dA and dP for two of the four column blocks, dq, dk and dKd terms for
// half of the key blocks) over all 32 columns, reading both groups' slice
// buffers.  The epilogue is split the same way.  Q and K are kept as raw
// bf16 rows (they are bf16 numbers), which makes room for the two groups'
// slice buffers.
template <int DK>
struct BwdChunk2Smem {
    static constexpr int LDQ = DK + 8, LDC = BT + 1, CW = 16, LDW = CW + 1;
    alignas(16) uint16_t Q[BT * LDQ], K[BT * LDQ];   // raw bf16 rows
    // T - I as two bf16 parts and P = (Q K^T) . D (lower) as three, 64 x 64
    // planes in the layout of plane_off; after the column loop the same bytes
    // hold dA . D and dP . D in fp32
    union {
        struct {
            alignas(16) uint16_t T[2][BT * BT];
            alignas(16) uint16_t P[3][BT * BT];
        } pl;
        struct {
            float Tm[BT * LDC];
            float P[BT * LDC];
        } ep;
    } tp;
    struct Slices {
        float S[DK * LDW], dS[DK * LDW];
        float V[BT * LDW], dO[BT * LDW], R[BT * LDW], Vn[BT * LDW], dVn[BT * LDW];
    };
    Slices sl[2];  // one per group
    double G2[BT];
    float Gam[BT], Dec[BT], Beta[BT];
    float dB[2][BT], dG[2][BT], colG[4][BT], red[16];
};

// acc += A B^T over k in [0, K) for raw bf16 rows A[i][k], B[j][k]: one
// 16-byte read per operand and 32 k (lane (g, r): row r, k-slots 8g .. + 7).
template <int K>
__device__ __forceinline__ f32x4 tile_mma_raw(f32x4 acc, const uint16_t *A, int lda, const uint16_t *B, int ldb,
                                              int i0, int j0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const uint16_t *pa = A + (i0 + r) * lda + 8 * g, *pb = B + (j0 + r) * ldb + 8 * g;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32)
        acc = mma_bf16v(acc, *(const u32x4b *)(pa + k0), *(const u32x4b *)(pb + k0));
    return acc;
}

// acc += A B over k in [0, K), A = raw bf16 rows, B as NP bf16 parts per 32 k.
template <int K, int NP>
__device__ __forceinline__ f32x4 mma_raw_parts(f32x4 acc, const uint16_t *A, int lda, int i0,
                                               const u32x4b (&bp)[K / 32][NP], int lane) {
    const int r = lane & 15, g = lane >> 4;
    const uint16_t *pa = A + (i0 + r) * lda + 8 * g;
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
        const u32x4b ua = *(const u32x4b *)(pa + 32 * kb);
#pragma unroll
        for (int q = 0; q < NP; ++q) acc = mma_bf16v(acc, ua, bp[kb][q]);
    }
    return acc;
}

// acc += A B^T for A and B given as bf16 parts of one 32-deep block (the
// first parts the largest): the products of total order at most one
// (a0 b0, a0 b1, a1 b0) or two (also a0 b2, a1 b1, a2 b0), smallest first.
__device__ __forceinline__ f32x4 mma_parts2(f32x4 acc, const u32x4b *a, const u32x4b *b) {
    acc = mma_bf16v(acc, a[1], b[0]);
    acc = mma_bf16v(acc, a[0], b[1]);
    return mma_bf16v(acc, a[0], b[0]);
}
__device__ __forceinline__ f32x4 mma_parts3(f32x4 acc, const u32x4b *a, const u32x4b *b) {
    acc = mma_bf16v(acc, a[2], b[0]);
    acc = mma_bf16v(acc, a[1], b[1]);
    acc = mma_bf16v(acc, a[0], b[2]);
    return mma_parts2(acc, a, b);
}

// Element (row, col) of a 64 x 64 bf16 plane: 16-byte units XOR-swizzled by
// the row's low three bits, so that 16 lanes reading one unit of 16 rows, or
// a transpose load's 4 rows x 4 chunks, spread over the banks.
__device__ __forceinline__ int plane_off(int row, int col) {
    return row * BT + ((((col >> 3) ^ (row & 7)) << 3) | (col & 7));
}

// acc += A B for row block i0 of a product over the 64 rows of a chunk: A
// given as NP bf16 planes, B an fp32 LDS slice (row stride LDW, column r of
// the lane) split into NP parts on the fly, over the 32-deep blocks
// kb0 .. kb1 - 1 (uniform over the wave; the others are zero for the
// triangular A).  TRANS: A(i, k) = plane[k][i], read with the gfx950 LDS
// transpose load, which hands lane (g, r) rows 4g + e and 16 + 4g + e of
// the block (e = 0..3) of column i0 + r; otherwise A(i, k) = plane[i][k],
// k-slots 8g .. 8g + 7 in one 16-byte read.
template <int NP, bool TRANS, int LDW>
__device__ __forceinline__ f32x4 mma_planes(f32x4 acc, const uint16_t (*pl)[BT * BT], const float *B, int i0, int kb0,
                                            int kb1, int lane) {
    const int r = lane & 15, g = lane >> 4;
    typedef __attribute__((ext_vector_type(4))) short s16x4b;
    typedef __attribute__((address_space(3))) s16x4b lds_s16x4b;
    typedef __attribute__((address_space(3))) const uint16_t lds_u16c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb < kb0 || kb >= kb1) continue;
        u32x4b pa[NP], pb[NP];
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = TRANS ? 32 * kb + (e >> 2) * 16 + 4 * g + (e & 3) : 32 * kb + 8 * g + e;
            xb[e] = B[k * LDW + r];
        }
        split_8(pb, xb);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (TRANS) {
                lds_u16c *m3 = (lds_u16c *)pl[p];
                const int rr = 32 * kb + 4 * g + (r >> 2), cc = i0 + 4 * (r & 3);
                const s16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4b *)(m3 + plane_off(rr, cc)));
                const s16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4b *)(m3 + plane_off(rr + 16, cc)));
                const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
                pa[p] = (u32x4b){ulo.x, ulo.y, uhi.x, uhi.y};
            } else {
                pa[p] = *(const u32x4b *)&pl[p][plane_off(i0 + r, 32 * kb + 8 * g)];
            }
        }
        acc = NP == 2 ? mma_parts2(acc, pa, pb) : mma_parts3(acc, pa, pb);
    }
    return acc;
}

// Two LDS transpose loads (at p and p + step elements) of 16-bit rows as one
// 8-element MFMA operand.
__device__ __forceinline__ u32x4b tr_rows16(const uint16_t *p, int step) {
    typedef __attribute__((ext_vector_type(4))) short s16x4c;
    typedef __attribute__((address_space(3))) s16x4c lds_s16x4c;
    typedef __attribute__((address_space(3))) const uint16_t lds_u16d;
    lds_u16d *m3 = (lds_u16d *)p;
    const s16x4c lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4c *)m3);
    const s16x4c hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4c *)(m3 + step));
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return (u32x4b){ulo.x, ulo.y, uhi.x, uhi.y};
}

template <int DK, int DV>
__global__ __launch_bounds__(512, 1) void bwd_chunk2_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ beta, const float *__restrict__ dO, const double *__restrict__ G2ws,
    const float *__restrict__ Tws, const float *__restrict__ Sck, const float *__restrict__ dSck,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta, int T, int H, int NT, float scale) {
    using SM = BwdChunk2Smem<DK>;
    constexpr int LDQ = SM::LDQ, LDC = SM::LDC, CW = SM::CW, LDW = SM::LDW, NTHR = 512, GT = 256, NM = DK / 16;
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int gi = wave >> 2, gt = tid & (GT - 1);  // group and thread within the group
    const long cb = blockIdx.x;
    const int c = (int)(cb % NT);
    const long bh = cb / NT;
    const int h = (int)(bh % H);
    const long b = bh / H;
    const int t0 = c * BT;
    const int I = wave & 3;  // this wave's 16-row block of every chunk-row product
    typename SM::Slices &sl = sm.sl[gi];

    // Q and K raw rows (zero past T), gate tables, T - I
    {
        constexpr int U = BT * DK / 8 / NTHR;
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const int idx = tid + NTHR * x, row = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
            const int t = min(t0 + row, T - 1);
            const long off = ((b * T + t) * H + h) * (long)DK + c8;
            const bool in = t0 + row < T;
            const u32x4b z = {0u, 0u, 0u, 0u};
            const u32x4b xq = *(const u32x4b *)(q + off), xk = *(const u32x4b *)(k + off);
            *(u32x4b *)&sm.Q[row * LDQ + c8] = in ? xq : z;
            *(u32x4b *)&sm.K[row * LDQ + c8] = in ? xk : z;
        }
    }
    if (tid < BT) {
        const int t = t0 + tid;
        const double G2 = G2ws[cb * BT + tid], G2L = G2ws[cb * BT + BT - 1];
        sm.G2[tid] = G2;
        sm.Gam[tid] = exp2f((float)G2);
        sm.Dec[tid] = exp2f((float)(G2L - G2));
        sm.Beta[tid] = (t < T) ? beta[(b * T + t) * H + h] : 0.f;
    }
    {
        // T - I (strictly lower, fp32) as two bf16 parts
        constexpr int U = BT * BT / 4 / NTHR;
        const float *src = Tws + cb * BT * BT;
        f32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = *(const f32x4 *)(src + 4 * (tid + NTHR * u));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = 4 * (tid + NTHR * u), row = idx / BT, col = idx % BT;
            const uint32_t h0 = pack_bf16_rne(x[u][0], x[u][1]), h1 = pack_bf16_rne(x[u][2], x[u][3]);
            const uint32_t l0 = pack_bf16_rne(x[u][0] - bf16_lo(h0), x[u][1] - bf16_hi(h0));
            const uint32_t l1 = pack_bf16_rne(x[u][2] - bf16_lo(h1), x[u][3] - bf16_hi(h1));
            *(uint2 *)&sm.tp.pl.T[0][plane_off(row, col)] = make_uint2(h0, h1);
            *(uint2 *)&sm.tp.pl.T[1][plane_off(row, col)] = make_uint2(l0, l1);
        }
    }
    if (tid < 2 * BT) {
        sm.dB[tid / BT][tid % BT] = 0.f;
        sm.dG[tid / BT][tid % BT] = 0.f;
    }
    __syncthreads();
    // P = (Q K^T) . D, lower with the diagonal (all 16 tiles, upper ones zero)
    for (int tile = wave; tile < 16; tile += 8) {
        const int TI = tile >> 2, TJ = tile & 3;
        const f32x4 acc = tile_mma_raw<DK>(zero4(), sm.Q, LDQ, sm.K, LDQ, 16 * TI, 16 * TJ, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * TI + 4 * g + e, j = 16 * TJ + r;
            const float pv = (j <= i) ? acc[e] * exp2f((float)(sm.G2[i] - sm.G2[j])) : 0.f;
            // three bf16 parts (the low halves of packed conversions)
            const uint32_t h = pack_bf16_rne(pv, 0.f);
            const float r1 = pv - bf16_lo(h);
            const uint32_t m = pack_bf16_rne(r1, 0.f);
            const uint32_t l = pack_bf16_rne(r1 - bf16_lo(m), 0.f);
            const int o = plane_off(i, j);
            sm.tp.pl.P[0][o] = (uint16_t)h;
            sm.tp.pl.P[1][o] = (uint16_t)m;
            sm.tp.pl.P[2][o] = (uint16_t)l;
        }
    }

    // this group's output tiles: column blocks J = 2 gi + jj of dA and dP,
    // key blocks m = MH gi + mm of the DK-wide products
    constexpr int MH = NM / 2;
    f32x4 dqs[MH], dkR[MH], dKd[MH], dA[2], dP[2];
#pragma unroll
    for (int m = 0; m < MH; ++m) dqs[m] = dkR[m] = dKd[m] = zero4();
#pragma unroll
    for (int j = 0; j < 2; ++j) dA[j] = dP[j] = zero4();
    float dGC = 0.f;  // <dS', S> over the slices this thread loaded

    // the group's 16 columns of S, dS', V and dO (fetched at the top of each
    // step: with two waves per SIMD the other wave hides the latency, and a
    // prefetch's registers would spill)
    constexpr int US = DK * CW / 4 / GT;
    static_assert(BT * CW / 8 == GT / 2, "one 8-value piece of v or dO per thread");
    f32x4 xs[US], xd[US], xo[2];
    u32x4b xv;
    const int prow = (gt & (GT / 2 - 1)) / (CW / 8), pc8 = 8 * (gt % (CW / 8));
    const int pt = min(t0 + prow, T - 1);
    auto fetch_slice = [&](int cc) {
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int idx = 4 * (gt + GT * u), row = idx / CW, col = idx % CW;
            const long off = cb * DK * DV + (long)row * DV + cc + col;
            xs[u] = *(const f32x4 *)(Sck + off);
            xd[u] = *(const f32x4 *)(dSck + off);
        }
        if (gt < GT / 2) {
            xv = *(const u32x4b *)(v + ((b * T + pt) * H + h) * (long)DV + cc + pc8);
        } else {
            const float *po = dO + ((b * T + pt) * H + h) * (long)DV + cc + pc8;
            xo[0] = *(const f32x4 *)po;
            xo[1] = *(const f32x4 *)(po + 4);
        }
    };
    for (int c0 = 0; c0 < DV; c0 += 2 * CW) {
        const int cg = c0 + CW * gi;  // this group's first column
        fetch_slice(cg);
        __syncthreads();  // previous slice fully consumed
        {
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int idx = 4 * (gt + GT * u), row = idx / CW, col = idx % CW;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sl.S[row * LDW + col + e] = xs[u][e];
                    sl.dS[row * LDW + col + e] = xd[u][e];
                    dGC += xs[u][e] * xd[u][e];
                }
            }
            const bool in = t0 + prow < T;  // rows past T are zero
            float x8[8];
            if (gt < GT / 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x8[2 * e] = __uint_as_float(xv[e] << 16);
                    x8[2 * e + 1] = __uint_as_float(xv[e] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x8[e] = xo[0][e];
                    x8[e + 4] = xo[1][e];
                }
            }
            float *dst = (gt < GT / 2 ? sl.V : sl.dO) + prow * LDW + pc8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = in ? x8[e] : 0.f;
        }
        __syncthreads();
        // KS, QS, R for rows of block I: K, Q exact in bf16; the S slice as bf16 hi + lo
        f32x4 KS, QS;
        {
            u32x4b sp[DK / 32][2];
            col_parts<DK, 2>(sp, sl.S, LDW, r, lane);
            KS = mma_raw_parts<DK, 2>(zero4(), sm.K, LDQ, 16 * I, sp, lane);
            QS = mma_raw_parts<DK, 2>(zero4(), sm.Q, LDQ, 16 * I, sp, lane);
        }
        f32x4 Rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            Rr[e] = sm.Beta[i] * (sl.V[i * LDW + r] - sm.Gam[i] * KS[e]);
            sl.R[i * LDW + r] = Rr[e];
        }
        __syncthreads();
        // Vn = R + (T - I) R;  dVn = scale P^T dO + Kd dS' (K exact; dS' as three bf16 parts)
        {
            // (T - I) R on two bf16 parts per side, P^T dO on three; row block I of
            // the strictly lower T - I reaches k < 32 only for I < 2, and of the
            // upper P^T k >= 32 only for I >= 2
            const f32x4 a = mma_planes<2, false, LDW>(zero4(), sm.tp.pl.T, sl.R, 16 * I, 0, I < 2 ? 1 : 2, lane);
            const f32x4 b1 = mma_planes<3, true, LDW>(zero4(), sm.tp.pl.P, sl.dO, 16 * I, I < 2 ? 0 : 1, 2, lane);
            u32x4b dp[DK / 32][3];
            col_parts<DK, 3>(dp, sl.dS, LDW, r, lane);
            const f32x4 b2 = mma_raw_parts<DK, 3>(zero4(), sm.K, LDQ, 16 * I, dp, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                sl.Vn[i * LDW + r] = Rr[e] + a[e];
                sl.dVn[i * LDW + r] = scale * b1[e] + sm.Dec[i] * b2[e];
            }
        }
        __syncthreads();
        // dR = dVn + (T - I)^T dVn; dv; the row sums of dbeta and dG (per group)
        f32x4 dRr;
        {
            const f32x4 a = mma_planes<2, true, LDW>(zero4(), sm.tp.pl.T, sl.dVn, 16 * I, I < 2 ? 0 : 1, 2, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                const int t = t0 + i;
                dRr[e] = sl.dVn[i * LDW + r] + a[e];
                if (t < T) dv[((b * T + t) * H + h) * (long)DV + cg + r] = sm.Beta[i] * dRr[e];
                const float vb = sl.V[i * LDW + r] - sm.Gam[i] * KS[e];
                const float pb = row16_sum(dRr[e] * vb);
                const float pg = row16_sum(-sm.Beta[i] * sm.Gam[i] * dRr[e] * KS[e] +
                                           scale * sm.Gam[i] * sl.dO[i * LDW + r] * QS[e]);
                if (r == 0) {
                    sm.dB[gi][i] += pb;
                    sm.dG[gi][i] += pg;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sl.R[(16 * I + 4 * g + e) * LDW + r] = dRr[e];
        __syncthreads();
        // accumulate this group's tiles of dA, dP (64 x 64) and the DK-wide
        // products for rows of block I over both groups' 16 columns, as one
        // 32-deep bf16 MFMA block: lane (g, r) takes k-slots 8g .. 8g + 7,
        // columns 8 (g & 1) .. + 7 of group g >> 1's slice.  The fp32
        // operands enter as bf16 parts: two on each side of dR Vn^T and
        // dR S^T, three on each side of dO Vn^T, dO S^T and Vn dS'^T, keeping
        // the part products of total order at most one (two parts) or two
        // (three).
        {
            const typename SM::Slices &o = sm.sl[g >> 1];
            const int kc = 8 * (g & 1);
            auto parts_of_row = [&](auto &out, const float *M, int row) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = M[row * LDW + kc + e];
                split_8(out, x);
            };
            u32x4b ar[2], ao[3], av[3];
            parts_of_row(ar, o.R, 16 * I + r);
            parts_of_row(ao, o.dO, 16 * I + r);
            parts_of_row(av, o.Vn, 16 * I + r);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                u32x4b bv[3];
                parts_of_row(bv, o.Vn, 16 * (2 * gi + jj) + r);
                dA[jj] -= mma_parts2(zero4(), ar, bv);
                dP[jj] += mma_parts3(zero4(), ao, bv) * scale;
            }
#pragma unroll
            for (int mm = 0; mm < MH; ++mm) {
                const int m = MH * gi + mm;
                u32x4b bs[3], bd[3];
                parts_of_row(bs, o.S, 16 * m + r);
                parts_of_row(bd, o.dS, 16 * m + r);
                dqs[mm] = mma_parts3(dqs[mm], ao, bs);
                dkR[mm] = mma_parts2(dkR[mm], ar, bs);
                dKd[mm] = mma_parts3(dKd[mm], av, bd);
            }
        }
    }
    __syncthreads();  // every wave is done with Tm, P and the slices

    float tdec[4] = {0.f, 0.f, 0.f, 0.f};  // sum over this group's m of dKd_im K_im for the 4 rows of this lane
    {
        // dA, dP on their supports (this group's column blocks); A, P and the K K^T terms
        float colp[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int J = 2 * gi + jj;
            const f32x4 KK = tile_mma_raw<DK>(zero4(), sm.K, LDQ, sm.K, LDQ, 16 * I, 16 * J, lane);
            const f32x4 QK = tile_mma_raw<DK>(zero4(), sm.Q, LDQ, sm.K, LDQ, 16 * I, 16 * J, lane);
            const int j = 16 * J + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e;
                const float D = (j <= i) ? exp2f((float)(sm.G2[i] - sm.G2[j])) : 0.f;
                const float dAv = (j < i) ? dA[jj][e] : 0.f;
                const float dPv = (j <= i) ? dP[jj][e] : 0.f;
                const float Av = sm.Beta[i] * KK[e] * D, Pv = QK[e] * D;
                const float w = dAv * Av + dPv * Pv;
                const float pb = row16_sum(dAv * D * KK[e]);
                const float pg = row16_sum(w);
                if (r == 0) {
                    sm.dB[gi][i] += pb;
                    sm.dG[gi][i] += pg;
                }
                colp[jj][e] = w;
                sm.tp.ep.Tm[i * LDC + j] = dAv * D;  // dA . D
                sm.tp.ep.P[i * LDC + j] = dPv * D;   // dP . D
            }
        }
        // column sums of dA . A + dP . P: lanes of column j = 16J + r
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            float x = colp[jj][0] + colp[jj][1] + colp[jj][2] + colp[jj][3];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (g == 0) sm.colG[I][16 * (2 * gi + jj) + r] = x;
        }
    }
    __syncthreads();
    {
        // dk = diag(beta) dAs K + dAs^T diag(beta) K + dPs^T Q + diag(dec) dKd - diag(beta gamma) dkR
        // dq = scale diag(gamma) dqs + dPs K, on bf16 MFMA: the left operands
        // split once into bf16 parts (three for dP.D, two for the others)
        // k-slots of lane (g, r) in each 32-deep block: rows 4g + e and
        // 16 + 4g + e (e = 0..3), the order in which the LDS transpose load
        // hands out the K and Q columns below
        u32x4b a1[2][2], a2[2][2], a3[2][2], a4[2][3];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float x1[8], x2[8], x3[8], x4[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = 16 * I + r, j = 32 * kb + (e >> 2) * 16 + 4 * g + (e & 3);
                x1[e] = sm.tp.ep.Tm[i * LDC + j];
                x2[e] = sm.tp.ep.Tm[j * LDC + i] * sm.Beta[j];
                x3[e] = sm.tp.ep.P[j * LDC + i];
                x4[e] = sm.tp.ep.P[i * LDC + j];
            }
            split_8(a1[kb], x1);
            split_8(a2[kb], x2);
            split_8(a3[kb], x3);
            split_8(a4[kb], x4);
        }
#pragma unroll
        for (int mm = 0; mm < MH; ++mm) {
            const int m = MH * gi + mm;
            f32x4 t1 = zero4(), t2 = zero4(), t3 = zero4(), t4 = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                // columns 16m .. 16m + 15 of K and Q by transpose loads: lane (g, r)
                // addresses row 32kb + 4g + r/4 (+ 16), columns 16m + 4(r % 4) .. + 3,
                // and receives column 16m + r of rows 4g + e (+ 16) of the block
                const int jr = 32 * kb + 4 * g + (r >> 2), jc = 16 * m + 4 * (r & 3);
                const u32x4b bk = tr_rows16(sm.K + jr * LDQ + jc, 16 * LDQ);
                const u32x4b bq = tr_rows16(sm.Q + jr * LDQ + jc, 16 * LDQ);
                t1 = mma_bf16v(mma_bf16v(t1, a1[kb][0], bk), a1[kb][1], bk);
                t2 = mma_bf16v(mma_bf16v(t2, a2[kb][0], bk), a2[kb][1], bk);
                t3 = mma_bf16v(mma_bf16v(t3, a3[kb][0], bq), a3[kb][1], bq);
                t4 = mma_bf16v(mma_bf16v(mma_bf16v(t4, a4[kb][0], bk), a4[kb][1], bk), a4[kb][2], bk);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * g + e, col = 16 * m + r;
                const int t = t0 + i;
                const float kim = bf16_to_f32(sm.K[i * LDQ + col]);
                tdec[e] = fmaf(dKd[mm][e], kim, tdec[e]);
                const float dkv = sm.Beta[i] * t1[e] + t2[e] + t3[e] + sm.Dec[i] * dKd[mm][e] -
                                  sm.Beta[i] * sm.Gam[i] * dkR[mm][e];
                const float dqv = scale * sm.Gam[i] * dqs[mm][e] + t4[e];
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
            if (r == 0) sm.dG[gi][i] -= tj;
            tdec[e] = (r == 0) ? tj : 0.f;
        }
    }
    // the Kd terms' total and sum_v dS' . S (both enter the last row's dG):
    // wave sums on shuffles, then the eight waves' partials
    float tv = tdec[0] + tdec[1] + tdec[2] + tdec[3], sv = dGC;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        tv += __shfl_xor(tv, off, 64);
        sv += __shfl_xor(sv, off, 64);
    }
    if (lane == 0) {
        sm.red[wave] = tv;
        sm.red[8 + wave] = sv;
    }
    __syncthreads();
    if (wave == 0) {
        // dG_j -= column sums; dg = reverse cumulative sum of dG within the
        // chunk, one row per lane (a suffix scan on shuffles)
        const int i = lane;
        float x = sm.dG[0][i] + sm.dG[1][i] - (sm.colG[0][i] + sm.colG[1][i] + sm.colG[2][i] + sm.colG[3][i]);
        if (i == BT - 1) {
            float ts = 0.f, ss = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                ts += sm.red[w];
                ss += sm.red[8 + w];
            }
            x += ts + sm.Gam[BT - 1] * ss;
        }
#pragma unroll
        for (int off = 1; off < BT; off <<= 1) {
            const float y = __shfl_down(x, off, 64);
            if (i + off < BT) x += y;
        }
        const int t = t0 + i;
        if (t < T) {
            dg[(b * T + t) * H + h] = x;
            dbeta[(b * T + t) * H + h] = sm.dB[0][i] + sm.dB[1][i];
        }
    }
}

// ----------------------------------------------------------------- launchers
template <class Pol, int DK, int DV>
static hipError_t launch_bwd_t(const void *q, const void *k, const void *v, const float *beta, const float *dO,
                               const float *dht, const double *G2, const float *Tinv, const float *Sck, float *dSck,
                               float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0, int B, int T,
                               int H, float scale, hipStream_t st) {
    using in_t = typename Pol::in_t;
    const int NT = (T + BT - 1) / BT;
    hipError_t e;
    if constexpr (std::is_same<in_t, uint16_t>::value) {
        // bf16 inputs: the fused reverse walk (gdn_bwd_fused.hip)
        e = launch_bwd_walk_fused(q, k, beta, dO, dht, G2, Tinv, dSck, dh0, B, T, H, DK, DV, scale, st);
    } else {
        hipLaunchKernelGGL((bwd_walk_kernel<Pol, DK, DV>), dim3((unsigned)((long)B * H * (DV / 32))), dim3(256), 0,
                           st, (const in_t *)q, (const in_t *)k, beta, dO, dht, G2, Tinv, dSck, dh0, T, H, NT, scale);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if constexpr (std::is_same<in_t, uint16_t>::value)
        hipLaunchKernelGGL((bwd_chunk2_kernel<DK, DV>), dim3((unsigned)((long)B * H * NT)), dim3(512), 0, st,
                           (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, beta, dO, G2, Tinv, Sck,
                           dSck, dq, dk, dv, dg, dbeta, T, H, NT, scale);
    else
        hipLaunchKernelGGL((bwd_chunk_kernel<Pol, DK, DV>), dim3((unsigned)((long)B * H * NT)), dim3(256), 0, st,
                           (const in_t *)q, (const in_t *)k, (const in_t *)v, beta, dO, G2, Tinv, Sck, dSck, dq, dk,
                           dv, dg, dbeta, T, H, NT, scale);
    return hipGetLastError();
}

hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *beta, const float *dO,
                      const float *dht, const double *G2, const float *Tinv, const float *Sck, float *dSck, float *dq,
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
