// gdn_bwd_fused.hip -- the reverse state walk of the chunked GDN backward for
// bf16 inputs, in one kernel along the lines of the fused forward.
//
// Reverse mode through a chunk (the chunk equations of the GatedDeltaNet
// walkthrough's chunked section; D_ij = 2^(G2_i - G2_j) for j <= i,
// gamma_i = 2^(G2_i), dec_j = 2^(G2_last - G2_j), dO' = scale dO):
//   dVn = P^T dO' + diag(dec) K dS'          (P = (Q K^T) . D, lower)
//   dR  = dVn + (T - I)^T dVn
//   dS  = gamma_C dS' + Q^T (diag(gamma) dO') - K^T (diag(beta gamma) dR)
// with dS' the gradient of the state leaving the chunk; dS is the one
// entering it.  Columns of the state gradient are independent, so one
// workgroup carries 32 of them through the chunks, last to first:
//   waves 1, 2: 16 columns each of dS' in registers (MFMA accumulator tiles);
//   wave 3:     P of the next chunk from its raw Q and K rows in registers,
//               stored as bf16 hi + lo planes, and the rows for the consumers;
//   wave 0:     T - I of the next chunk (from the intra stage) as bf16 hi + lo
//               planes, dO' transposed, and the gate tables.
// Precision: products that carry dS' (K dS', Q^T (gamma dO') and
// K^T (beta gamma dR)) take K or Q exactly in bf16 and the other operand as
// three bf16 parts (~24 bits, fp32's floor); P^T dO' and (T - I)^T dVn take
// both operands as bf16 hi + lo (hi.hi + hi.lo + lo.hi); accumulation fp32.
// Every decay factor comes from fp64 gate sums (their differences are exact
// to fp32).  The walk stores dS' of every chunk for the per-chunk stage and
// the gradient entering the first chunk (dh0).
#include "gdn_launch.h"
#include "gdn_tile.h"

namespace gdn {

namespace {

constexpr int kRwThreads = 320;  // five waves

template <int DK>
struct RwCfg {
    static constexpr int NS = DK / 32;   // 32-deep slabs of the key dimension
    static constexpr int NKB = DK / 16;  // 16-row blocks of the state gradient
    static constexpr int LDT = BT + 8;   // bf16 row stride of the T - I and P planes
    static constexpr int LDO = BT + 4;   // fp32 row stride of dO' transposed (one row per value column)
};

template <int DK>
struct RwSmem {
    using C = RwCfg<DK>;
    alignas(16) uint16_t K[2][BT * DK];           // raw bf16 rows, paired-group layout (tile_off_pg)
    alignas(16) uint16_t Q[2][BT * DK];
    alignas(16) uint16_t Tp[2][2][BT * C::LDT];   // T - I, bf16 hi and lo planes, [i][j]
    alignas(16) uint16_t Pp[2][2][BT * C::LDT];   // P, bf16 hi and lo planes, [i][j]
    alignas(16) float dOT[2][32 * C::LDO];        // dO' of the workgroup's 32 columns, [column][token]
    alignas(16) float gam[2][BT];                 // gamma_i
    alignas(16) float bgam[2][BT];                // -beta_i gamma_i
    alignas(16) float dec[2][BT];                 // 2^(G2_last - G2_i)
    alignas(16) double G2P[BT];                   // gate sums of the chunk the P producer prepares
};

// One workgroup's head and columns.
struct RwHead {
    long b, bh;
    int h, vcol0;
};

__device__ __forceinline__ RwHead rw_head(int DV) {
    const int n = blockIdx.x, nwg = gridDim.x;
    // the column slices of one head get consecutive ids on one XCD (shared L2)
    const int L = (nwg % 8 == 0) ? (n % 8) * (nwg / 8) + n / 8 : n;
    const int ntile = DV / 32;
    RwHead hd;
    hd.bh = L / ntile;
    hd.vcol0 = (L % ntile) * 32;
    return hd;
}

// 3 bf16 parts of a pair: h + m + l carries ~24 bits of each value.
__device__ __forceinline__ void split3_pair(bf16x2 &h, bf16x2 &m, bf16x2 &l, float a, float b) {
    const f32x2 x = {a, b};
    h = __builtin_convertvector(x, bf16x2);
    const f32x2 r1 = x - __builtin_convertvector(h, f32x2);
    m = __builtin_convertvector(r1, bf16x2);
    l = __builtin_convertvector(r1 - __builtin_convertvector(m, f32x2), bf16x2);
}

// Slots e and e + 4 of a B fragment from t0[e] and t1[e], as 3 bf16 parts.
__device__ __forceinline__ void split3_frags(u32x4 &h, u32x4 &m, u32x4 &l, const f32x4 &t0, const f32x4 &t1) {
    bf16x2 hh[4], mm[4], ll[4];
    split3_pair(hh[0], mm[0], ll[0], t0[0], t0[1]);
    split3_pair(hh[1], mm[1], ll[1], t0[2], t0[3]);
    split3_pair(hh[2], mm[2], ll[2], t1[0], t1[1]);
    split3_pair(hh[3], mm[3], ll[3], t1[2], t1[3]);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        h[x] = __builtin_bit_cast(uint32_t, hh[x]);
        m[x] = __builtin_bit_cast(uint32_t, mm[x]);
        l[x] = __builtin_bit_cast(uint32_t, ll[x]);
    }
}

__device__ __forceinline__ void split2_frags(u32x4 &h, u32x4 &l, const f32x4 &t0, const f32x4 &t1) {
    uint4 a, b;
    hilo_frags<bf16x2>(a, b, t0, t1);
    h = u32x4{a.x, a.y, a.z, a.w};
    l = u32x4{b.x, b.y, b.z, b.w};
}

__device__ __forceinline__ u32x4 as_u32x4(const uint4 &a) { return u32x4{a.x, a.y, a.z, a.w}; }

// A fragment of M^T from a row-major bf16 plane M (row stride LD): rows
// col0 .. col0 + 15 of M^T, the 32-deep slab of M rows row0 .. row0 + 31.
// The gfx950 LDS transpose load gives lane (g, r) M[row0 + 4g + e][col0 + r].
template <int LD>
__device__ __forceinline__ u32x4 planeT_frag(const uint16_t *M, int row0, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    typedef __attribute__((ext_vector_type(4))) short s16x4_t;
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    const uint16_t *p = &M[(row0 + 4 * g + (r >> 2)) * LD + col0 + 4 * (r & 3)];
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p);
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p + 16 * LD));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return u32x4{a.x, a.y, b.x, b.y};
}

// Rows of a chunk held by a lane: row 16I + r, columns 32s + 8g .. + 7 (the
// MFMA fragment order of both operands of Q K^T).
template <int DK>
struct RowRegs {
    u32x4 v[4][DK / 32];
};

template <int DK>
__device__ __forceinline__ void rw_load_rows(RowRegs<DK> &R, const uint16_t *__restrict__ src, long b, int h, int t0,
                                             int T, int H, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const int t = min(t0 + 16 * I + r, T - 1);
        const uint16_t *p = src + ((b * T + t) * H + h) * (long)DK + 8 * g;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) R.v[I][s] = *(const u32x4 *)(p + 32 * s);
    }
}

// Rows past T are zero.
template <int DK>
__device__ __forceinline__ void rw_mask_rows(RowRegs<DK> &R, int t0, int T, int lane) {
    const int r = lane & 15;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const bool in = t0 + 16 * I + r < T;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
            if (!in) R.v[I][s] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Rows into a tile in the paired-group layout.
template <int DK>
__device__ __forceinline__ void rw_write_rows(uint16_t *dst, const RowRegs<DK> &R, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const int row = 16 * I + r, c0 = 32 * s + 8 * g;
            *(uint2 *)&dst[tile_off_pg<DK>(row, pair_col(c0))] = make_uint2(R.v[I][s][0], R.v[I][s][1]);
            *(uint2 *)&dst[tile_off_pg<DK>(row, pair_col(c0 + 4))] = make_uint2(R.v[I][s][2], R.v[I][s][3]);
        }
}

// ------------------------------------------------------------ P producer
// Chunk c into LDS half p: its raw K and Q rows (held in registers since the
// previous iteration) and P = (Q K^T) . D as bf16 hi + lo planes; then the
// rows and gate sums of chunk cn are requested.
template <int DK>
__device__ __forceinline__ void rw_prepare_P(RwSmem<DK> &sm, RowRegs<DK> &Rq, RowRegs<DK> &Rk, double &g2, int c,
                                             int cn, int p, const uint16_t *q, const uint16_t *k,
                                             const double *G2ws, long bh, long b, int h, int T, int H, int NT,
                                             int lane) {
    using C = RwCfg<DK>;
    const int r = lane & 15, g = lane >> 4;
    const int t0 = c * BT;
    rw_mask_rows(Rq, t0, T, lane);
    rw_mask_rows(Rk, t0, T, lane);
    rw_write_rows<DK>(sm.K[p], Rk, lane);
    rw_write_rows<DK>(sm.Q[p], Rq, lane);
    sm.G2P[lane] = g2;
    // Q K^T on the 10 tiles I >= J: lane gets (Q K^T)[16I + 4g + e][16J + r]
    f32x4 acc[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = zero4();
#pragma unroll
    for (int s = 0; s < C::NS; ++s)
#pragma unroll
        for (int t = 0; t < 10; ++t) acc[t] = mma_bf16_raw(acc[t], Rq.v[tileI(t)][s], Rk.v[tileJ(t)][s]);
    // the next chunk's rows overwrite the operands once the products have read them
    if (cn >= 0) {
        rw_load_rows<DK>(Rq, q, b, h, cn * BT, T, H, lane);
        rw_load_rows<DK>(Rk, k, b, h, cn * BT, T, H, lane);
        g2 = G2ws[(bh * NT + cn) * BT + lane];
    }
    // D from fp64 gate sums; the tile then leaves as 4 adjacent columns of one
    // row per lane (quad transpose) in bf16 hi and lo planes
#pragma unroll
    for (int t = 0; t < 10; ++t) {
        const int I = tileI(t), J = tileJ(t);
        const int j = 16 * J + r;
        const double gj = sm.G2P[j];
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            const float d = __builtin_amdgcn_exp2f((float)(sm.G2P[i] - gj));
            v[e] = (I > J || i >= j) ? acc[t][e] * d : 0.f;
        }
        v = quad_transpose(v, lane);
        const int row = 16 * I + 4 * g + (r & 3), col = 16 * J + 4 * (r >> 2);
        bf16x2 h0, l0, h1, l1;
        split_pair(h0, l0, v[0], v[1]);
        split_pair(h1, l1, v[2], v[3]);
        *(uint2 *)&sm.Pp[p][0][row * C::LDT + col] =
            make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
        *(uint2 *)&sm.Pp[p][1][row * C::LDT + col] =
            make_uint2(__builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1));
    }
}

// ---------------------------------------------------------------- loader
// T - I, dO' and the gate tables of one chunk, held in registers between
// their request and their store.
struct RwLoadRegs {
    f32x4 t[16];   // T - I: 16-byte piece u = lane + 64 x of the [64][64] matrix
    f32x4 d[8];    // dO: rows (lane + 64 x) / 8, columns 4 ((lane + 64 x) % 8) .. + 3 of the 32
    double g2, g2L;
    float beta;
};

__device__ __forceinline__ void rw_fetch(RwLoadRegs &R, const float *Tws, const float *dO, const double *G2ws,
                                         const float *beta, long bh, long b, int h, int c, int T, int H, int NT,
                                         int DV, int vcol0, int lane) {
    const long cb = bh * NT + c;
    const int t0 = c * BT;
#pragma unroll
    for (int x = 0; x < 16; ++x) R.t[x] = *(const f32x4 *)(Tws + cb * BT * BT + 4 * (lane + 64 * x));
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int u = lane + 64 * x, row = u >> 3, c4 = 4 * (u & 7);
        R.d[x] = *(const f32x4 *)(dO + ((b * T + min(t0 + row, T - 1)) * H + h) * (long)DV + vcol0 + c4);
    }
    R.g2 = G2ws[cb * BT + lane];
    R.g2L = G2ws[cb * BT + BT - 1];
    R.beta = beta[(b * T + min(t0 + lane, T - 1)) * H + h];
}

template <int DK>
__device__ __forceinline__ void rw_store(RwSmem<DK> &sm, const RwLoadRegs &R, int p, int c, int T, float scale,
                                         int lane) {
    using C = RwCfg<DK>;
    const int t0 = c * BT;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        const int idx = 4 * (lane + 64 * x), row = idx / BT, col = idx % BT;
        bf16x2 h0, l0, h1, l1;
        split_pair(h0, l0, R.t[x][0], R.t[x][1]);
        split_pair(h1, l1, R.t[x][2], R.t[x][3]);
        *(uint2 *)&sm.Tp[p][0][row * C::LDT + col] =
            make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
        *(uint2 *)&sm.Tp[p][1][row * C::LDT + col] =
            make_uint2(__builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1));
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int u = lane + 64 * x, row = u >> 3, c4 = 4 * (u & 7);
        const float m = (t0 + row < T) ? scale : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.dOT[p][(c4 + e) * C::LDO + row] = m * R.d[x][e];
    }
    const bool in = t0 + lane < T;
    const float gm = __builtin_amdgcn_exp2f((float)R.g2);
    sm.gam[p][lane] = gm;
    sm.bgam[p][lane] = in ? -R.beta * gm : 0.f;
    sm.dec[p][lane] = __builtin_amdgcn_exp2f((float)(R.g2L - R.g2));
}

// -------------------------------------------------------------- consumer
// Chunk c (LDS half p) on the 16 columns of wave cw: S holds dS' (rows
// 16m + 4g + e, column r) on entry and dS on return.
template <int DK>
__device__ __forceinline__ void rw_consume(RwSmem<DK> &sm, f32x4 (&S)[DK / 16], int p, int cw, int lane) {
    using C = RwCfg<DK>;
    const int r = lane & 15, g = lane >> 4;
    // X = K dS': K exact in bf16, dS' as three bf16 parts
    f32x4 X[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) X[I] = zero4();
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        u32x4 bh, bm, bl;
        split3_frags(bh, bm, bl, S[2 * s], S[2 * s + 1]);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const u32x4 a = as_u32x4(frag_rows_pg<DK>(sm.K[p], 16 * I, 32 * s, lane));
            X[I] = mma_bf16_raw(X[I], a, bh);
            X[I] = mma_bf16_raw(X[I], a, bm);
            X[I] = mma_bf16_raw(X[I], a, bl);
        }
    }
    // dO' of this wave's columns for slabs 0 and 1 (tokens 32s + 4g + e and
    // 32s + 16 + 4g + e), and the gate tables
    const float *dcol = &sm.dOT[p][(16 * cw + r) * C::LDO];
    f32x4 dlo[2], dhi[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        dlo[s] = *(const f32x4 *)&dcol[32 * s + 4 * g];
        dhi[s] = *(const f32x4 *)&dcol[32 * s + 16 + 4 * g];
    }
    // dVn = P^T dO' + diag(dec) X; P^T nonzero where token i >= j, so row
    // block I takes the slabs s with 32 s + 31 >= 16 I
    f32x4 dVn[4];
    {
        u32x4 oh[2], ol[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) split2_frags(oh[s], ol[s], dlo[s], dhi[s]);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 u = zero4();
#pragma unroll
            for (int s = I >> 1; s < 2; ++s) {
                const u32x4 ah = planeT_frag<C::LDT>(sm.Pp[p][0], 32 * s, 16 * I, lane);
                const u32x4 al = planeT_frag<C::LDT>(sm.Pp[p][1], 32 * s, 16 * I, lane);
                u = mma_bf16_raw(u, ah, oh[s]);
                u = mma_bf16_raw(u, ah, ol[s]);
                u = mma_bf16_raw(u, al, oh[s]);
            }
            const f32x4 dc = *(const f32x4 *)&sm.dec[p][16 * I + 4 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e) dVn[I][e] = u[e] + dc[e] * X[I][e];
        }
    }
    // dR = dVn + (T - I)^T dVn; (T - I)^T is nonzero where token k > i
    f32x4 dR[4];
    {
        u32x4 vh[2], vl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) split2_frags(vh[s], vl[s], dVn[2 * s], dVn[2 * s + 1]);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 u = dVn[I];
#pragma unroll
            for (int s = I >> 1; s < 2; ++s) {
                const u32x4 ah = planeT_frag<C::LDT>(sm.Tp[p][0], 32 * s, 16 * I, lane);
                const u32x4 al = planeT_frag<C::LDT>(sm.Tp[p][1], 32 * s, 16 * I, lane);
                u = mma_bf16_raw(u, ah, vh[s]);
                u = mma_bf16_raw(u, ah, vl[s]);
                u = mma_bf16_raw(u, al, vh[s]);
            }
            dR[I] = u;
        }
    }
    // dS = gamma_C dS' + Q^T (diag(gamma) dO') + K^T (diag(-beta gamma) dR)
    u32x4 gh[2], gm[2], gl[2], rh[2], rm[2], rl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const f32x4 ga = *(const f32x4 *)&sm.gam[p][32 * s + 4 * g];
        const f32x4 gb = *(const f32x4 *)&sm.gam[p][32 * s + 16 + 4 * g];
        split3_frags(gh[s], gm[s], gl[s], ga * dlo[s], gb * dhi[s]);
        const f32x4 ba = *(const f32x4 *)&sm.bgam[p][32 * s + 4 * g];
        const f32x4 bb = *(const f32x4 *)&sm.bgam[p][32 * s + 16 + 4 * g];
        split3_frags(rh[s], rm[s], rl[s], ba * dR[2 * s], bb * dR[2 * s + 1]);
    }
    const float gC = sm.gam[p][BT - 1];
#pragma unroll
    for (int m = 0; m < C::NKB; ++m) {
        f32x4 acc = S[m] * gC;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const u32x4 aq = as_u32x4(frag_T_pg<DK>(sm.Q[p], 32 * s, 16 * m, lane));
            const u32x4 ak = as_u32x4(frag_T_pg<DK>(sm.K[p], 32 * s, 16 * m, lane));
            acc = mma_bf16_raw(acc, aq, gh[s]);
            acc = mma_bf16_raw(acc, ak, rh[s]);
            acc = mma_bf16_raw(acc, aq, gm[s]);
            acc = mma_bf16_raw(acc, ak, rm[s]);
            acc = mma_bf16_raw(acc, aq, gl[s]);
            acc = mma_bf16_raw(acc, ak, rl[s]);
        }
        S[m] = acc;
    }
}

// dS' (rows 16m + 4g + e, column r of the wave's 16) into a [DK][DV] matrix,
// 16-byte row pieces after a quad transpose.
template <int DK, int DV>
__device__ __forceinline__ void rw_store_state(float *dst, const f32x4 (&S)[DK / 16], int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    float *d = dst + col0 + 4 * (r >> 2);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
        *(f32x4 *)&d[(long)(16 * m + 4 * g + (r & 3)) * DV] = quad_transpose(S[m], lane);
}

template <int DK, int DV>
__global__ __launch_bounds__(kRwThreads, 1) void bwd_walk_fused_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ beta,
    const float *__restrict__ dO, const float *__restrict__ dht, const double *__restrict__ G2ws,
    const float *__restrict__ Tws, float *__restrict__ dSck, float *__restrict__ dh0, int T, int H, int NT,
    float scale) {
    using C = RwCfg<DK>;
    static_assert(sizeof(RwSmem<DK>) <= 160 * 1024, "LDS budget");
    __shared__ RwSmem<DK> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    RwHead hd = rw_head(DV);
    hd.h = (int)(hd.bh % H);
    hd.b = hd.bh / H;
    // the upper tiles of the P planes (16-column block above the row's 16-row
    // block) are never written by the producer: zero them once
    for (int idx = tid; idx < 2 * 2 * BT * BT; idx += kRwThreads) {
        const int row = (idx / BT) % BT, col = idx % BT, plane = idx / (BT * BT);
        if (col / 16 > row / 16) (&sm.Pp[0][0][0])[plane * BT * C::LDT + row * C::LDT + col] = 0;
    }
    // iteration it walks chunk NT - 1 - it in LDS half it & 1; the producers
    // prepare the chunk after it (NT - 2 - it) in the other half
    if (wave == 1 || wave == 2) {
        const int cw = wave - 1, col = hd.vcol0 + 16 * cw + r;
        const long sbase = hd.bh * (long)DK * DV;
        f32x4 S[C::NKB];
#pragma unroll
        for (int m = 0; m < C::NKB; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = dht ? dht[sbase + (long)(16 * m + 4 * g + e) * DV + col] : 0.f;
        __syncthreads();
        for (int it = 0; it < NT; ++it) {
            const int c = NT - 1 - it;
            rw_store_state<DK, DV>(dSck + (hd.bh * NT + c) * (long)DK * DV, S, hd.vcol0 + 16 * cw, lane);
            rw_consume<DK>(sm, S, it & 1, cw, lane);
            __syncthreads();
        }
        if (dh0) rw_store_state<DK, DV>(dh0 + sbase, S, hd.vcol0 + 16 * cw, lane);
    } else if (wave == 3) {
        RowRegs<DK> Rq, Rk;
        double g2 = 0.0;
        if (NT > 0) {
            rw_load_rows<DK>(Rq, q, hd.b, hd.h, (NT - 1) * BT, T, H, lane);
            rw_load_rows<DK>(Rk, k, hd.b, hd.h, (NT - 1) * BT, T, H, lane);
            g2 = G2ws[(hd.bh * NT + NT - 1) * BT + lane];
            rw_prepare_P<DK>(sm, Rq, Rk, g2, NT - 1, NT - 2, 0, q, k, G2ws, hd.bh, hd.b, hd.h, T, H, NT, lane);
        }
        __syncthreads();
        for (int it = 0; it < NT; ++it) {
            const int c = NT - 2 - it;
            if (c >= 0)
                rw_prepare_P<DK>(sm, Rq, Rk, g2, c, c - 1, (it + 1) & 1, q, k, G2ws, hd.bh, hd.b, hd.h, T, H, NT,
                                 lane);
            __syncthreads();
        }
    } else if (wave == 0) {
        RwLoadRegs R;
        if (NT > 0) {
            rw_fetch(R, Tws, dO, G2ws, beta, hd.bh, hd.b, hd.h, NT - 1, T, H, NT, DV, hd.vcol0, lane);
            rw_store<DK>(sm, R, 0, NT - 1, T, scale, lane);
            if (NT > 1) rw_fetch(R, Tws, dO, G2ws, beta, hd.bh, hd.b, hd.h, NT - 2, T, H, NT, DV, hd.vcol0, lane);
        }
        __syncthreads();
        for (int it = 0; it < NT; ++it) {
            const int c = NT - 2 - it;
            if (c >= 0) {
                rw_store<DK>(sm, R, (it + 1) & 1, c, T, scale, lane);
                if (c > 0) rw_fetch(R, Tws, dO, G2ws, beta, hd.bh, hd.b, hd.h, c - 1, T, H, NT, DV, hd.vcol0, lane);
            }
            __syncthreads();
        }
    } else {
        __syncthreads();
        for (int it = 0; it < NT; ++it) __syncthreads();
    }
}

}  // namespace

hipError_t launch_bwd_walk_fused(const void *q, const void *k, const float *beta, const float *dO, const float *dht,
                                 const double *G2, const float *Tinv, float *dSck, float *dh0, int B, int T, int H,
                                 int Dk, int Dv, float scale, hipStream_t st) {
    const int NT = (T + BT - 1) / BT;
#define GDN_RW(DKv, DVv)                                                                                         \
    if (Dk == DKv && Dv == DVv) {                                                                                \
        hipLaunchKernelGGL((bwd_walk_fused_kernel<DKv, DVv>), dim3((unsigned)((long)B * H * (DVv / 32))),        \
                           dim3(kRwThreads), 0, st, (const uint16_t *)q, (const uint16_t *)k, beta, dO, dht, G2,   \
                           Tinv, dSck, dh0, T, H, NT, scale);                                                    \
        return hipGetLastError();                                                                                \
    }
    GDN_RW(64, 64);
    GDN_RW(64, 128);
    GDN_RW(128, 64);
    GDN_RW(128, 128);
#undef GDN_RW
    return hipErrorInvalidValue;
}

}  // namespace gdn
