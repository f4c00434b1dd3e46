// gdn_fused.hip -- single-kernel chunked Gated DeltaNet forward for bf16
// inputs on gfx950.
//
// One workgroup owns (batch b, head h, a 32-wide slice of value columns) and
// walks the 64-token chunks of that head in order.  Its five waves run
// concurrently, each in a role of its own:
//
//   consumers (waves 1, 2; 16 value columns each) -- the state chain of
//     chunk c, with their d_k x 16 slice of the state S resident in MFMA
//     accumulators:
//       X = K S, Y = Q S
//       R = diag(beta) (V - diag(gamma) X)
//       Vnew = R + (T - I) R           (= U - W S of the WY form)
//       O = scale (diag(gamma) Y + diag(q.k) Vnew + strict(P) Vnew)
//       S = gamma_C S + (K . 2^(G2_C - G2))^T Vnew
//   producers -- everything that does not depend on the state, written to
//     the other half of double-buffered LDS:
//       wave 4 (chunk c + 2): the chunk-local cumsum G2 = log2(e) cumsum(g)
//         (so each decay is one exp2 of a non-positive difference) and
//         A = strictly-lower(diag(beta) K K^T . 2^(G2_i - G2_j)) on bf16 MFMA
//         straight from raw K rows it loads into registers;
//       wave 0 (chunk c + 1): T = (I + A)^-1 by block doubling
//         (unit_lower_inverse);
//       wave 3 (chunk c + 1): P = (Q K^T) . 2^(G2_i - G2_j) (causal, diagonal
//         kept apart in fp32), the decay of each key to the chunk end, V,
//         gamma, beta, and the raw Q rows of chunk c + 2 (the A producer
//         stores the raw K rows of its chunk).
//   Producers that load keep the raw inputs of their next chunk in
//   registers, loaded an iteration before they are used.  With waves placed
//   on SIMDs in turn, the A producer shares a SIMD with the inverse, whose
//   time is mostly LDS and MFMA latency.
//
// Per chunk the workgroup synchronises once, at the end of the iteration.
// Buffers written in an iteration are never the ones read in it.
//
// Precision: products of exact bf16 inputs (K K^T, Q K^T) run on bf16 MFMA;
// the state reads K S and Q S run on bf16 MFMA with the fp32 state split
// into bf16 hi + lo parts (two products, ~16 significant bits); the other
// products with intermediate operands (new values, decayed keys, T - I, P)
// use fp16 operands; every accumulation, the state, the diagonal terms
// beta_i v_i and (q_i.k_i) vnew_i, and the output are fp32.
#include "gdn_launch.h"
#include "gdn_tile.h"

namespace gdn {

constexpr int kFusedThreads = 320;  // five waves

template <int DK, int DV>
struct FusedCfg {
    static constexpr int BV = 32;
    static constexpr int NS = DK / 32;   // 32-wide k slabs
    static constexpr int NKB = DK / 16;  // 16-row blocks of the state
    static constexpr int LDK = DK;       // row stride of the raw K and Q tiles (paired-group layout)
    static constexpr int LDP = BT + 4;   // fp16 row stride of sP, sT, sA
    static constexpr int LDV = BV + 8;   // bf16 row stride of sV
};

// The raw K and Q rows of chunk c sit in buffer c % 3: they are written two
// iterations ahead (chunk c + 2 in iteration c, K by the A producer, Q by the
// P producer), read by the P producer one
// iteration ahead and by the consumers in iteration c.  A of chunk c is
// written in iteration c - 2 and inverted in iteration c - 1 (index = chunk
// parity).  Everything else the consumers read for a chunk is
// double-buffered (index = chunk parity).  One barrier per iteration
// separates every write from its reads.
template <int DK, int DV>
struct FusedSmem {
    using C = FusedCfg<DK, DV>;
    alignas(16) uint16_t K[3][BT * C::LDK];   // raw bf16 rows, paired-group layout (tile_off_pg)
    alignas(16) uint16_t Q[3][BT * C::LDK];
    alignas(16) _Float16 P[2][BT * C::LDP];
    alignas(16) _Float16 Tm[2][BT * C::LDP];
    alignas(16) uint16_t V[2][BT * C::LDV];
    alignas(16) float gam[2][BT];
    alignas(16) float beta[2][BT];
    alignas(16) float diag[2][BT];             // scale * (q_i . k_i)
    alignas(16) float dk[2][BT];              // 2^(G2_last - G2_j): decay of key j to the chunk end
    alignas(16) _Float16 A[2][BT * C::LDP];
    alignas(16) float g2A[BT], betaA[BT];  // gate tables private to the A producer
    alignas(16) float decA[BT];            // ... 2^(g2_j) = 2^(G2_j - G2_(j-1)), the decay of one token
    alignas(16) float g2P[BT];             // ... and to the P producer
};

// Raw inputs of one chunk held by a producer lane (lane = (g, r)):
// k/q rows 16I + r, columns 32s + 8g .. +7 as 8 bf16 in 16 bytes.
template <int NS>
struct ChunkRegs {
    u32x4 k[4][NS];
    u32x4 q[4][NS];
    u32x4 v[4];   // V tile rows 16p + lane/4, 8 columns at (lane%4)*8
    float g, beta;
};

// One workgroup's sequence: token t of it is token-head row (tok0 + t) * H + h
// of the [., H, D] tensors (tok0 = b T for a dense batch, the sequence start
// for packed variable-length input).
struct HeadArgs {
    const uint16_t *q, *k, *v;
    const float *g, *beta;
    long tok0;
    int h, T, H, vcol0;
    bool zero_v;  // walk with all values zero (a segment's transfer matrix)
};

// A long sequence in segments (chunk-parallel state scan).  Segment s of
// sequence b holds chunks [s L, min((s + 1) L, NT)).  Per chunk the state map
// is affine, S' = M_c S + N_c, so a segment's end state is M_s S_in + E_s, with
// E_s its end state from a zero start and M_s the product of its M_c.
//   walk launch (fused_walk_kernel): for segment 0 its end state from h0, for
//     every middle segment 1 .. NS - 2 the output-free walks that give E_s and
//     M_s (the identity columns walked with zero values); E_s goes to
//     Hin[b NS + s + 1], M_s to M[b NS + s];
//   scan (seg_scan_kernel): Hin[b NS] = h0, and Hin[b NS + s + 1] =
//     M_s Hin[b NS + s] + E_s for s = 1 .. NS - 2, so Hin[b NS + s] is the true
//     entry state of segment s; it also writes the segment offsets cu;
//   then the ordinary single kernel runs the B NS segments as packed
//     sequences (cu, initial states Hin, final states Hout) and the final
//     state of each sequence is Hout[b NS + NS - 1].
// Hin, Hout: [B NS, H, Dk, Dk] fp32; M: [B NS, H, Dk, Dk] fp32 (Dv = Dk here).
struct SegArgs {
    int L, NS;
    float *Hin, *M;
};

// What one workgroup computes: the rows of its sequence, its initial state
// (h0 rows of this head, or null for zeros; or the identity), where its final
// state goes (or null), and its output (or null for a walk without output).
struct WgJob {
    HeadArgs ha;
    const float *h0;
    float *ht;
    float *o;
    bool ident;
};

// The loaders are branch-free, so the compiler can count the loads in
// flight and wait only for the ones it needs.  Rows past the end of the
// sequence read its last row (a.T >= 1 is the caller's guarantee): with
// beta = g = 0 there (load_gates zeroes them) such rows add nothing to A,
// T - I, the new values or the state, and their outputs are not stored.
template <int DK>
__device__ __forceinline__ void load_rows(u32x4 (&dst)[4][DK / 32], const uint16_t *__restrict__ src,
                                          const HeadArgs &a, int chunk, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const int t = min(chunk * BT + 16 * I + r, a.T - 1);
        const uint16_t *p = src + ((a.tok0 + t) * a.H + a.h) * (long)DK + 8 * g;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) dst[I][s] = *(const u32x4 *)(p + 32 * s);
    }
}

template <int DV>
__device__ __forceinline__ void load_v(u32x4 (&dst)[4], const HeadArgs &a, int chunk, int lane) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int t = min(chunk * BT + 16 * p + (lane >> 2), a.T - 1);
        dst[p] = __builtin_nontemporal_load((const u32x4 *)(a.v + ((a.tok0 + t) * a.H + a.h) * (long)DV + a.vcol0 + (lane & 3) * 8));
    }
}

// Raw gates of the chunk's token `lane`; finish_gates zeroes them past the
// end of the sequence once they have arrived.
__device__ __forceinline__ void load_gates(float &gv, float &bv, const HeadArgs &a, int chunk, int lane) {
    const long idx = (a.tok0 + min(chunk * BT + lane, a.T - 1)) * a.H + a.h;
    gv = a.g[idx];
    bv = a.beta[idx];
}

__device__ __forceinline__ void finish_gates(float &gv, float &bv, const HeadArgs &a, int chunk, int lane) {
    const bool in = chunk * BT + lane < a.T;
    gv = in ? gv : 0.f;
    bv = in ? bv : 0.f;
}

// Raw rows held in registers (k or q of ChunkRegs) into a kq-buffer tile in
// the paired-group layout (the two 4-column halves of a register go to
// their stored groups).
template <int DK>
__device__ __forceinline__ void write_rows(uint16_t *dst, const u32x4 (&src)[4][DK / 32], int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const int row = 16 * I + r, c0 = 32 * s + 8 * g;
            *(uint2 *)&dst[tile_off_pg<DK>(row, pair_col(c0))] = make_uint2(src[I][s][0], src[I][s][1]);
            *(uint2 *)&dst[tile_off_pg<DK>(row, pair_col(c0 + 4))] = make_uint2(src[I][s][2], src[I][s][3]);
        }
}

// The 10 lower 16x16 tiles of X_J Y_I^T (tile t: I = tileI(t), J = tileJ(t))
// from two paired-group tiles in LDS: this lane gets row 16J + 4g + e and
// column 16I + r of tile t in acc[t][e].
template <int DK>
__device__ __forceinline__ void lower_tiles(f32x4 (&acc)[10], const uint16_t *X, const uint16_t *Y, int lane) {
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = zero4();
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        uint4 xf[4], yf[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            xf[I] = frag_rows_pg<DK>(X, 16 * I, 32 * s, lane);
            yf[I] = (X == Y) ? xf[I] : frag_rows_pg<DK>(Y, 16 * I, 32 * s, lane);
        }
#pragma unroll
        for (int t = 0; t < 10; ++t) acc[t] = mma_bf16_raw(acc[t], xf[tileJ(t)], yf[tileI(t)]);
    }
}

// ------------------------------------------------------------ producer: A
// Chunk c2 into A of LDS half c2 & 1, from the raw K rows and gates of
// chunk c2 held in R, which also go to kq-buffer c2 % 3 for the P producer
// and the consumers; R then receives those of chunk c2 + 1.  Both MFMA
// operands are the same register fragments (row 16I + r, columns 32s + 8g
// .. + 7), so K_J K_I^T needs no particular k-slot order.
template <int DK, int DV>
__device__ __forceinline__ void produce_A(FusedSmem<DK, DV> &sm, ChunkRegs<DK / 32> &R, int c2, int kb, int NT,
                                          const HeadArgs &ha, int lane) {
    using C = FusedCfg<DK, DV>;
    const int r = lane & 15, g = lane >> 4;
    write_rows<DK>(sm.K[kb], R.k, lane);
    finish_gates(R.g, R.beta, ha, c2, lane);
    sm.g2A[lane] = chunk_g2(R.g);
    sm.betaA[lane] = R.beta;
    sm.decA[lane] = __builtin_amdgcn_exp2f(R.g * LOG2E);
    load_gates(R.g, R.beta, ha, min(c2 + 1, NT - 1), lane);
    // K_J K_I^T: this lane gets row i = 16I + r and columns j = 16J + 4g + e
    // of every tile, stored as 4 adjacent halves
    f32x4 acc[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = zero4();
#pragma unroll
    for (int s = 0; s < C::NS; ++s)
#pragma unroll
        for (int t = 0; t < 10; ++t) acc[t] = mma_bf16_raw(acc[t], R.k[tileJ(t)][s], R.k[tileI(t)][s]);
    // beta_i 2^(G2_i - G2_j) = 2^(G2_i + log2(beta_i) - G2_j): beta enters the
    // row's exponent (beta = 0 gives 2^-inf = 0)
    float rowG2[4];
    f32x4 colG2[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        rowG2[I] = sm.g2A[16 * I + r] + __builtin_amdgcn_logf(sm.betaA[16 * I + r]);
        colG2[I] = *(const f32x4 *)&sm.g2A[16 * I + 4 * g];
    }
    // The next chunk's rows overwrite the MFMA operands, so they are requested
    // once those products have had time to read them.
    load_rows<DK>(R.k, ha.k, ha, min(c2 + 1, NT - 1), lane);
    // A = strictly-lower(diag(beta) K K^T . 2^(G2_i - G2_j))
    _Float16 *A = sm.A[c2 & 1];
#pragma unroll
    for (int tile = 0; tile < 10; ++tile) {
        const int I = tileI(tile), J = tileJ(tile);
        const int i = 16 * I + r;
        f16x4 hv;
        if (I > J) {
            // below the diagonal blocks (i > j always): one exp2 for the nearest
            // of the 4 columns, then one token's decay per step to the left,
            // 2^(G2_i - G2_(j-1)) = 2^(G2_i - G2_j) 2^(g2_j), all factors <= 1
            const f32x4 dc = *(const f32x4 *)&sm.decA[16 * J + 4 * g];
            float d = __builtin_amdgcn_exp2f(rowG2[I] - colG2[J][3]);
            hv[3] = (_Float16)(acc[tile][3] * d);
#pragma unroll
            for (int e = 2; e >= 0; --e) {
                d *= dc[e + 1];
                hv[e] = (_Float16)(acc[tile][e] * d);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * J + 4 * g + e;
                const float val = acc[tile][e] * __builtin_amdgcn_exp2f(rowG2[I] - colG2[J][e]);
                hv[e] = (_Float16)((i > j) ? val : 0.f);
            }
        }
        *(f16x4 *)&A[i * C::LDP + 16 * J + 4 * g] = hv;
    }
}

// ------------------------------------------- producer: P and consumer inputs
// Chunk c1: V, gate tables and P into LDS half c1 & 1 (P from the K and Q
// rows in kq-buffer c1 % 3).  R holds V and the gates of chunk c1 and the raw
// Q rows of chunk c1 + 1; those rows go to kq-buffer (c1 + 1) % 3 and R
// receives the rows of chunk c1 + 2, a full iteration before they are stored.
template <int DK, int DV, bool OUT, bool ZV>
__device__ __forceinline__ void produce_P(FusedSmem<DK, DV> &sm, ChunkRegs<DK / 32> &R, int c1, int kb, int NT,
                                          const HeadArgs &ha, float scale, int lane) {
    using C = FusedCfg<DK, DV>;
    const int r = lane & 15, g = lane >> 4;
    const int buf = c1 & 1;
    // first store everything that arrived during the previous iteration: the
    // V tile, the gates and the raw Q rows of chunk c1 + 1 (when it is past
    // the end, its buffer is written but never read).  A walk with zero
    // values (ZV) keeps the zeroed V buffers and loads no values.
    if constexpr (!ZV) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = 16 * p + (lane >> 2), c0 = (lane & 3) * 8;
            *(u32x4 *)&sm.V[buf][row * C::LDV + c0] = R.v[p];
        }
    }
    finish_gates(R.g, R.beta, ha, c1, lane);
    const float G2 = chunk_g2(R.g);
    sm.g2P[lane] = G2;
    const float gmv = __builtin_amdgcn_exp2f(G2);
    sm.gam[buf][lane] = gmv;
    sm.beta[buf][lane] = R.beta;
    if constexpr (OUT) write_rows<DK>(sm.Q[(kb + 1) % 3], R.q, lane);
    // then fetch the next ones together (indices clamped to the last chunk)
    if constexpr (!ZV) load_v<DV>(R.v, ha, min(c1 + 1, NT - 1), lane);
    load_gates(R.g, R.beta, ha, min(c1 + 1, NT - 1), lane);
    if constexpr (OUT) load_rows<DK>(R.q, ha.q, ha, min(c1 + 2, NT - 1), lane);
    const float G2L = sm.g2P[BT - 1];
    sm.dk[buf][lane] = __builtin_amdgcn_exp2f(G2L - G2);
    if constexpr (!OUT) return;  // a walk without output needs no P
    // P tiles: lane gets P[16I + r][16J + 4g + e] = scale (q_i . k_j) 2^(G2_i - G2_j)
    f32x4 acc[10];
    lower_tiles<DK>(acc, sm.K[kb], sm.Q[kb], lane);
    // scale 2^(G2_i - G2_j) = 2^(G2_i + log2(scale) - G2_j)
    const float lscale = __builtin_amdgcn_logf(scale);
    f32x4 colG2[4];
    float rowG2[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        colG2[I] = *(const f32x4 *)&sm.g2P[16 * I + 4 * g];
        rowG2[I] = sm.g2P[16 * I + r] + lscale;
    }
    _Float16 *P = sm.P[buf];
#pragma unroll
    for (int tile = 0; tile < 10; ++tile) {
        const int I = tileI(tile), J = tileJ(tile);
        const int i = 16 * I + r;
        f16x4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 16 * J + 4 * g + e;
            const float val = acc[tile][e] * __builtin_amdgcn_exp2f(rowG2[I] - colG2[J][e]);
            // below the diagonal blocks i > j always holds; only they are masked
            hv[e] = (_Float16)((I > J || i > j) ? val : 0.f);
            if (I == J && i == j) sm.diag[buf][i] = scale * acc[tile][e];
        }
        *(f16x4 *)&P[i * C::LDP + 16 * J + 4 * g] = hv;
    }
}

// ---------------------------------------------------------------- consumers
template <int DK, int DV, bool OUT, bool TLO = false>
__device__ __forceinline__ void consume(FusedSmem<DK, DV> &sm, f32x4 (&S)[DK / 16], int buf, int kb,
                                        float *__restrict__ o, const HeadArgs &ha, int chunk, int cw, float scale,
                                        int lane) {
    using C = FusedCfg<DK, DV>;
    const int r = lane & 15, g = lane >> 4;
    // X = K S and Y = Q S on bf16 MFMA: exact bf16 K, Q against the state
    // split into bf16 hi + lo parts.
    f32x4 X[4], Y[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) X[I] = Y[I] = zero4();
    // The gate tables and this wave's V columns (transpose loads of the
    // row-major V tile: V[16I + 4g + e][column r]) are read first, so their
    // latency hides under the products below.
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    f32x4 gmv[4], betv[4];
    s16x4 vtv[4];
    {
        const int cl0 = cw * 16 + 4 * (r & 3);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            gmv[I] = *(const f32x4 *)&sm.gam[buf][16 * I + 4 * g];
            betv[I] = *(const f32x4 *)&sm.beta[buf][16 * I + 4 * g];
            vtv[I] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)&sm.V[buf][(16 * I + 4 * g + (r >> 2)) * C::LDV + cl0]);
        }
    }
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        uint4 uhi, ulo;
        hilo_frags<bf16x2>(uhi, ulo, S[2 * s], S[2 * s + 1]);
        const bf16x8 shi = __builtin_bit_cast(bf16x8, uhi), slo = __builtin_bit_cast(bf16x8, ulo);
        // all hi-part products, then all lo-part products: an accumulator's
        // two updates are eight MFMAs apart
        bf16x8 kf[4], qf[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            kf[I] = __builtin_bit_cast(bf16x8, frag_rows_pg<DK>(sm.K[kb], 16 * I, 32 * s, lane));
            X[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[I], shi, X[I], 0, 0, 0);
            if constexpr (OUT) {
                qf[I] = __builtin_bit_cast(bf16x8, frag_rows_pg<DK>(sm.Q[kb], 16 * I, 32 * s, lane));
                Y[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[I], shi, Y[I], 0, 0, 0);
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            X[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[I], slo, X[I], 0, 0, 0);
            if constexpr (OUT) Y[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[I], slo, Y[I], 0, 0, 0);
        }
    }
    // R = beta (V - gamma X)
    f32x4 Rr[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const f32x4 gm = gmv[I], bet = betv[I];
        const s16x4 vt = vtv[I];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float vv = __uint_as_float(((uint32_t)(uint16_t)vt[e]) << 16);
            Rr[I][e] = bet[e] * (vv - gm[e] * X[I][e]);
        }
    }
    // Vnew = R + (T - I) R.  TLO: T - I arrives as fp16 hi (Tm) + lo (the P
    // buffer, free without output) parts and R enters as fp16 hi + lo parts,
    // so the product keeps about 22 bits (hi.hi + hi.lo + lo.hi)
    _Float16 rf[2][8], rl[2][8];
    frag_from_acc(rf[0], Rr[0], Rr[1]);
    frag_from_acc(rf[1], Rr[2], Rr[3]);
    if constexpr (TLO) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rl[s][e] = (_Float16)(Rr[2 * s][e] - (float)rf[s][e]);
                rl[s][e + 4] = (_Float16)(Rr[2 * s + 1][e] - (float)rf[s][e + 4]);
            }
    }
    f32x4 Vn[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        Vn[I] = Rr[I];
#pragma unroll
        for (int s = 0; s <= (I >> 1); ++s) {
            _Float16 a[8];
            frag_rows(a, sm.Tm[buf], C::LDP, 16 * I, 32 * s, lane);
            Vn[I] = mma_slab(Vn[I], a, rf[s]);
            if constexpr (TLO) {
                _Float16 al[8];
                frag_rows(al, sm.P[buf], C::LDP, 16 * I, 32 * s, lane);
                Vn[I] = mma_slab(Vn[I], a, rl[s]);
                Vn[I] = mma_slab(Vn[I], al, rf[s]);
            }
        }
    }
    // The state carry comes first: it is what the next chunk waits for, and
    // the output work below overlaps its MFMAs.
    // S = gamma_C S + (K . d)^T Vnew = gamma_C S + K^T (d . Vnew), d_j =
    // 2^(G2_last - G2_j) <= 1: the decay scales the new values, K^T comes
    // straight from the raw K tile by transpose loads, and d . Vnew enters as
    // bf16 hi + lo parts.
    uint4 dvh[2], dvl[2];
    {
        f32x4 dv[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const f32x4 dd = *(const f32x4 *)&sm.dk[buf][16 * I + 4 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[I][e] = dd[e] * Vn[I][e];
        }
        hilo_frags<bf16x2>(dvh[0], dvl[0], dv[0], dv[1]);
        hilo_frags<bf16x2>(dvh[1], dvl[1], dv[2], dv[3]);
    }
    const float gl = sm.gam[buf][BT - 1];
#pragma unroll
    for (int m = 0; m < C::NKB; ++m) {
        f32x4 acc = S[m] * gl;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 a = frag_T_pg<DK>(sm.K[kb], 32 * s, 16 * m, lane);
            acc = mma_bf16_raw(acc, a, dvh[s]);
            acc = mma_bf16_raw(acc, a, dvl[s]);
        }
        S[m] = acc;
    }
    if constexpr (!OUT) return;  // a walk without output ends with the carry
    // O = scale (gamma Y + diag(q.k) Vnew + strict(P) Vnew), with scale folded
    // into the diag and P tables
    _Float16 vf[2][8];
    frag_from_acc(vf[0], Vn[0], Vn[1]);
    frag_from_acc(vf[1], Vn[2], Vn[3]);
    const int t0 = chunk * BT;
    const bool full = t0 + BT <= ha.T;
    const long ostride = (long)ha.H * DV;
    f32x4 O[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const f32x4 gm = *(const f32x4 *)&sm.gam[buf][16 * I + 4 * g];
        const f32x4 dg = *(const f32x4 *)&sm.diag[buf][16 * I + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) O[I][e] = (scale * gm[e]) * Y[I][e] + dg[e] * Vn[I][e];
#pragma unroll
        for (int s = 0; s <= (I >> 1); ++s) {
            _Float16 a[8];
            frag_rows(a, sm.P[buf], C::LDP, 16 * I, 32 * s, lane);
            O[I] = mma_slab(O[I], a, vf[s]);
        }
    }
    // Stores: a 4 x 4 transpose within each quad of lanes (DPP quad
    // permutations) gives lane (g, 4a + b) row 16I + 4g + b and columns
    // 4a .. 4a + 3 of this wave's 16, so each row block is one 16-byte store
    // per lane (four store instructions per chunk instead of sixteen).
    const int qb = r & 3;
    float *ob = o + ((ha.tok0 + t0 + 4 * g + qb) * ha.H + ha.h) * (long)DV + ha.vcol0 + cw * 16 + 4 * (r >> 2);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const f32x4 v = quad_transpose(O[I], lane);
        if (full || t0 + 16 * I + 4 * g + qb < ha.T) *(f32x4 *)&ob[16 * I * ostride] = v;
    }
}

// Consumer role: the state slice of this wave from the job's initial state (or
// the identity columns of a transfer-matrix walk), the chunks in order, and
// the final state to the job's destination.
template <int DK, int DV, bool OUT, bool ST = false, bool TLO = false>
__device__ __forceinline__ void run_consumer(FusedSmem<DK, DV> &sm, const WgJob &job, int NT, int cw, float scale,
                                             int lane, float *states = nullptr) {
    using C = FusedCfg<DK, DV>;
    const int r = lane & 15, g = lane >> 4;
    const HeadArgs &ha = job.ha;
    f32x4 S[C::NKB];
    const int col = ha.vcol0 + cw * 16 + r;
    // ST: the state entering chunk c goes to states + c DK DV ([DK][DV], this
    // wave's 16 columns), after a quad transpose as 16-byte row pieces
    auto store_state = [&](int c) {
        if constexpr (ST) {
            float *dst = states + (long)c * DK * DV + ha.vcol0 + cw * 16 + 4 * (r >> 2);
#pragma unroll
            for (int m = 0; m < C::NKB; ++m)
                *(f32x4 *)&dst[(long)(16 * m + 4 * g + (r & 3)) * DV] = quad_transpose(S[m], lane);
        }
    };
#pragma unroll
    for (int m = 0; m < C::NKB; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * m + 4 * g + e;
            S[m][e] = job.ident ? (row == col ? 1.f : 0.f) : (job.h0 ? job.h0[(long)row * DV + col] : 0.f);
        }
    __syncthreads();
    __syncthreads();  // iteration -1: the producers fill chunk 0 and 1
    // Unrolled by the period of the kq-buffers, so that buffer c % 3 is a
    // constant in each copy and its fragment addresses stay in registers
    // across chunks; one barrier per chunk as in the other roles.
    for (int c = 0; c < NT; c += 3) {
        store_state(c);
        consume<DK, DV, OUT, TLO>(sm, S, c & 1, 0, job.o, ha, c, cw, scale, lane);
        __syncthreads();
        if (c + 1 < NT) {
            store_state(c + 1);
            consume<DK, DV, OUT, TLO>(sm, S, (c + 1) & 1, 1, job.o, ha, c + 1, cw, scale, lane);
            __syncthreads();
        }
        if (c + 2 < NT) {
            store_state(c + 2);
            consume<DK, DV, OUT, TLO>(sm, S, c & 1, 2, job.o, ha, c + 2, cw, scale, lane);
            __syncthreads();
        }
    }
    if (job.ht) {
#pragma unroll
        for (int m = 0; m < C::NKB; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) job.ht[(long)(16 * m + 4 * g + e) * DV + col] = S[m][e];
    }
}

// P-producer role (see produce_P).
template <int DK, int DV, bool OUT, bool ZV>
__device__ __forceinline__ void run_p_producer(FusedSmem<DK, DV> &sm, const HeadArgs &ha, int NT, float scale,
                                               int lane) {
    using C = FusedCfg<DK, DV>;
    ChunkRegs<C::NS> R;
    // chunk 0's raw Q rows go to kq-buffer 0 before the first barrier;
    // chunk 1's wait in registers (an empty sequence loads nothing)
    if (NT > 0) {
        if constexpr (!ZV) load_v<DV>(R.v, ha, 0, lane);
        load_gates(R.g, R.beta, ha, 0, lane);
        if constexpr (OUT) {
            load_rows<DK>(R.q, ha.q, ha, 0, lane);
            write_rows<DK>(sm.Q[0], R.q, lane);
            load_rows<DK>(R.q, ha.q, ha, min(1, NT - 1), lane);
        }
    }
    __syncthreads();
    // iteration c = c1 - 1 prepares chunk c1; unrolled like the A producer
    for (int c1 = 0; c1 <= NT; c1 += 3) {
        if (c1 < NT) produce_P<DK, DV, OUT, ZV>(sm, R, c1, 0, NT, ha, scale, lane);
        __syncthreads();
        if (c1 + 1 <= NT) {
            if (c1 + 1 < NT) produce_P<DK, DV, OUT, ZV>(sm, R, c1 + 1, 1, NT, ha, scale, lane);
            __syncthreads();
        }
        if (c1 + 2 <= NT) {
            if (c1 + 2 < NT) produce_P<DK, DV, OUT, ZV>(sm, R, c1 + 2, 2, NT, ha, scale, lane);
            __syncthreads();
        }
    }
}

// What one workgroup computes.  Dense batch: (batch b, head h, 32 value
// columns) over the whole sequence.  Packed sequences: the same for sequence
// n of cu_seqlens.  Segmented (a long sequence split into segments whose
// entry states come from a scan, see SegArgs): one segment of one head, either
// in full (output and final state) or as an output-free walk that records the
// segment's end state from a zero start (E) or its transfer matrix (M: zero
// values, the identity as initial state).
template <int DK, int DV, bool SEG>
__device__ __forceinline__ WgJob decode_job(int L, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                            const float *gin, const float *betain, const float *h0, float *o,
                                            float *ht, const int *cu_seqlens, int T, int H, const SegArgs &sg) {
    using C = FusedCfg<DK, DV>;
    constexpr int W = DV / C::BV;  // column slices per head
    WgJob job;
    HeadArgs &ha = job.ha;
    ha.q = q; ha.k = k; ha.v = v; ha.g = gin; ha.beta = betain;
    ha.H = H;
    ha.zero_v = false;
    job.ident = false;
    job.o = o;
    if constexpr (!SEG) {
        const int vt = L % W;
        const long bh = L / W;
        ha.h = (int)(bh % H);
        ha.vcol0 = vt * C::BV;
        if (cu_seqlens) {
            // packed sequences: T is the total token count; the bounds are clamped
            // into [0, T] so that malformed offsets can never address out of range
            const long n_seq = bh / H;
            const int s0 = min(max(cu_seqlens[n_seq], 0), T);
            const int s1 = min(max(cu_seqlens[n_seq + 1], s0), T);
            ha.tok0 = s0;
            ha.T = s1 - s0;
        } else {
            ha.tok0 = (bh / H) * (long)T;
            ha.T = T;
        }
        const long sbase = bh * (long)DK * DV;
        job.h0 = h0 ? h0 + sbase : nullptr;
        job.ht = ht ? ht + sbase : nullptr;
    } else {
        // walk launch: per head, W workgroups for segment 0's end state, then
        // 2 W per middle segment (W for E_s, W for M_s)
        const int per_head = W + 2 * W * (sg.NS - 2);
        const long bh = L / per_head;
        const int j = L % per_head;
        const long b = bh / H;
        ha.h = (int)(bh % H);
        job.o = nullptr;
        job.h0 = nullptr;
        int seg, slice;
        if (j < W) {
            seg = 0;
            slice = j;
            job.h0 = h0 ? h0 + bh * (long)DK * DV : nullptr;
        } else {
            const int kk = j - W;
            seg = 1 + kk / (2 * W);
            slice = kk % (2 * W);
            if (slice >= W) {
                slice -= W;
                job.ident = true;
                ha.zero_v = true;
            }
        }
        job.ht = job.ident ? sg.M + ((b * sg.NS + seg) * H + ha.h) * (long)DK * DV
                           : sg.Hin + ((b * sg.NS + seg + 1) * H + ha.h) * (long)DK * DV;
        ha.vcol0 = slice * C::BV;
        const int c0 = seg * sg.L;
        ha.tok0 = b * (long)T + (long)c0 * BT;
        ha.T = min(T, (c0 + sg.L) * BT) - c0 * BT;
    }
    return job;
}

template <int DK, int DV>
__global__ __global__ __launch_bounds__(kFusedThreads, 1) void fused_kernel(const uint16_t *__restrict__ q,
                                                       const uint16_t *__restrict__ k,
                                                       const uint16_t *__restrict__ v,
                                                       const float *__restrict__ gin,
                                                       const float *__restrict__ betain,
                                                       const float *__restrict__ h0, float *__restrict__ o,
                                                       float *__restrict__ ht, const int *__restrict__ cu_seqlens,
                                                       int T, int H, float scale) {
    using C = FusedCfg<DK, DV>;
    static_assert(sizeof(FusedSmem<DK, DV>) <= 160 * 1024, "LDS budget");
    __shared__ FusedSmem<DK, DV> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    constexpr int NTILE = DV / C::BV;
    // Workgroup n runs on XCD n % 8; give the slices of one head consecutive
    // ids on one XCD so they share its L2 for K and Q.
    const int n = blockIdx.x, nwg = gridDim.x;
    const int L = (nwg % 8 == 0) ? (n % 8) * (nwg / 8) + n / 8 : n;
    const int vt = L % NTILE;
    const long bh = L / NTILE;
    HeadArgs ha;
    ha.q = q; ha.k = k; ha.v = v; ha.g = gin; ha.beta = betain;
    ha.h = (int)(bh % H);
    ha.H = H;
    ha.vcol0 = vt * C::BV;
    ha.zero_v = false;
    if (cu_seqlens) {
        // packed sequences: T is the total token count; the bounds are clamped
        // into [0, T] so that malformed offsets can never address out of range
        const long n_seq = bh / H;
        const int s0 = min(max(cu_seqlens[n_seq], 0), T);
        const int s1 = min(max(cu_seqlens[n_seq + 1], s0), T);
        ha.tok0 = s0;
        ha.T = s1 - s0;
    } else {
        ha.tok0 = (bh / H) * (long)T;
        ha.T = T;
    }
    const int NT = (ha.T + BT - 1) / BT;  // this workgroup's chunks

    // The upper tiles (0,1) and (2,3) of P and T - I are read by the 32-wide
    // slabs of the consumers but never written: zero them once.
    for (int idx = tid; idx < 2 * BT * C::LDP; idx += kFusedThreads) {
        (&sm.P[0][0])[idx] = (_Float16)0.f;
        (&sm.Tm[0][0])[idx] = (_Float16)0.f;
    }

    const long sbase = bh * (long)DK * DV;
    // Each role runs its own loop with the same barrier count (one per
    // iteration), so the registers of one role are never live in another.
    // Iteration c: consumers walk chunk c (LDS half c & 1, kq-buffer c % 3);
    // the inverse and the P producer prepare chunk c + 1, the P producer also
    // stores the raw rows of chunk c + 2 and fetches chunk c + 3; the A
    // producer prepares chunk c + 2.
    if (wave == 1 || wave == 2) {
        const int cw = wave - 1;
        f32x4 S[C::NKB];
        const int col = ha.vcol0 + cw * 16 + r;
#pragma unroll
        for (int m = 0; m < C::NKB; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = h0 ? h0[sbase + (long)(16 * m + 4 * g + e) * DV + col] : 0.f;
        __syncthreads();
        __syncthreads();  // iteration -1: the producers fill chunk 0 and 1
        // Unrolled by the period of the kq-buffers, so that buffer c % 3 is a
        // constant in each copy and its fragment addresses stay in registers
        // across chunks; one barrier per chunk as in the other roles.
        for (int c = 0; c < NT; c += 3) {
            consume<DK, DV, true>(sm, S, c & 1, 0, o, ha, c, cw, scale, lane);
            __syncthreads();
            if (c + 1 < NT) {
                consume<DK, DV, true>(sm, S, (c + 1) & 1, 1, o, ha, c + 1, cw, scale, lane);
                __syncthreads();
            }
            if (c + 2 < NT) {
                consume<DK, DV, true>(sm, S, c & 1, 2, o, ha, c + 2, cw, scale, lane);
                __syncthreads();
            }
        }
        if (ht) {
#pragma unroll
            for (int m = 0; m < C::NKB; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) ht[sbase + (long)(16 * m + 4 * g + e) * DV + col] = S[m][e];
        }
    } else if (wave == 0) {
        __syncthreads();
        for (int c = -1; c < NT; ++c) {
            if (c + 1 < NT) unit_lower_inverse<C::LDP>(sm.A[(c + 1) & 1], sm.Tm[(c + 1) & 1], lane);
            __syncthreads();
        }
    } else if (wave == 4) {
        // A of chunk 0 before the first barrier; then chunk c + 2 in iteration c
        ChunkRegs<C::NS> R;
        if (NT > 0) {
            load_gates(R.g, R.beta, ha, 0, lane);
            load_rows<DK>(R.k, k, ha, 0, lane);
            produce_A(sm, R, 0, 0, NT, ha, lane);
        }
        __syncthreads();
        // iteration c = c2 - 2 prepares chunk c2; unrolled by the kq-buffer
        // period (c2 % 3 constant in each copy), one barrier per iteration
        for (int c2 = 1; c2 <= NT + 1; c2 += 3) {
            if (c2 < NT) produce_A(sm, R, c2, 1, NT, ha, lane);
            __syncthreads();
            if (c2 + 1 <= NT + 1) {
                if (c2 + 1 < NT) produce_A(sm, R, c2 + 1, 2, NT, ha, lane);
                __syncthreads();
            }
            if (c2 + 2 <= NT + 1) {
                if (c2 + 2 < NT) produce_A(sm, R, c2 + 2, 0, NT, ha, lane);
                __syncthreads();
            }
        }
    } else {
        ChunkRegs<C::NS> R;
        // chunk 0's raw Q rows go to kq-buffer 0 before the first barrier;
        // chunk 1's wait in registers (an empty sequence loads nothing)
        if (NT > 0) {
            load_rows<DK>(R.q, q, ha, 0, lane);
            load_v<DV>(R.v, ha, 0, lane);
            load_gates(R.g, R.beta, ha, 0, lane);
            write_rows<DK>(sm.Q[0], R.q, lane);
            load_rows<DK>(R.q, q, ha, min(1, NT - 1), lane);
        }
        __syncthreads();
        // iteration c = c1 - 1 prepares chunk c1; unrolled like the A producer
        for (int c1 = 0; c1 <= NT; c1 += 3) {
            if (c1 < NT) produce_P<DK, DV, true, false>(sm, R, c1, 0, NT, ha, scale, lane);
            __syncthreads();
            if (c1 + 1 <= NT) {
                if (c1 + 1 < NT) produce_P<DK, DV, true, false>(sm, R, c1 + 1, 1, NT, ha, scale, lane);
                __syncthreads();
            }
            if (c1 + 2 <= NT) {
                if (c1 + 2 < NT) produce_P<DK, DV, true, false>(sm, R, c1 + 2, 2, NT, ha, scale, lane);
                __syncthreads();
            }
        }
    }
}


// Producer role of the walk kernel: the A producer's work for chunk c + 2
// (its K rows to the kq-buffer, A) and the output-free P producer's work for
// chunk c + 1 (V unless the values are zero, the gate tables), in one wave.
template <int DK, int DV, bool ZV>
__device__ __forceinline__ void run_walk_producer(FusedSmem<DK, DV> &sm, const HeadArgs &ha, int NT, float scale,
                                                  int lane) {
    using C = FusedCfg<DK, DV>;
    ChunkRegs<C::NS> RA, RP;
    if (NT > 0) {
        load_gates(RA.g, RA.beta, ha, 0, lane);
        load_rows<DK>(RA.k, ha.k, ha, 0, lane);
        if constexpr (!ZV) load_v<DV>(RP.v, ha, 0, lane);
        load_gates(RP.g, RP.beta, ha, 0, lane);
        produce_A(sm, RA, 0, 0, NT, ha, lane);
    }
    __syncthreads();
    // iteration c = c2 - 2 (A of chunk c2, tables of chunk c2 - 1); unrolled
    // by the kq-buffer period, one barrier per iteration
    for (int c2 = 1; c2 <= NT + 1; c2 += 3) {
        if (c2 < NT) produce_A(sm, RA, c2, 1, NT, ha, lane);
        if (c2 - 1 < NT) produce_P<DK, DV, false, ZV>(sm, RP, c2 - 1, 0, NT, ha, scale, lane);
        __syncthreads();
        if (c2 + 1 <= NT + 1) {
            if (c2 + 1 < NT) produce_A(sm, RA, c2 + 1, 2, NT, ha, lane);
            if (c2 < NT) produce_P<DK, DV, false, ZV>(sm, RP, c2, 1, NT, ha, scale, lane);
            __syncthreads();
        }
        if (c2 + 2 <= NT + 1) {
            if (c2 + 2 < NT) produce_A(sm, RA, c2 + 2, 0, NT, ha, lane);
            if (c2 + 1 < NT) produce_P<DK, DV, false, ZV>(sm, RP, c2 + 1, 2, NT, ha, scale, lane);
            __syncthreads();
        }
    }
}

constexpr int kWalkThreads = 256;  // four waves

// Output-free walks of the chunk-parallel scan (SegArgs): the consumers carry
// the state (or the identity columns of a transfer matrix) through the
// segment and store it at its end.  Four waves, one per SIMD: the inverse,
// two consumers, and one producer for A and the gate tables.
template <int DK, int DV>
__global__ __launch_bounds__(kWalkThreads, 1) void fused_walk_kernel(const uint16_t *__restrict__ q,
                                                       const uint16_t *__restrict__ k,
                                                       const uint16_t *__restrict__ v,
                                                       const float *__restrict__ gin,
                                                       const float *__restrict__ betain,
                                                       const float *__restrict__ h0, float *__restrict__ o,
                                                       float *__restrict__ ht, int T, int H, float scale,
                                                       SegArgs sg) {
    using C = FusedCfg<DK, DV>;
    static_assert(sizeof(FusedSmem<DK, DV>) <= 160 * 1024, "LDS budget");
    __shared__ FusedSmem<DK, DV> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Workgroup n runs on XCD n % 8; give the slices of one head consecutive
    // ids on one XCD so they share its L2 for K.
    const int n = blockIdx.x, nwg = gridDim.x;
    const int L = (nwg % 8 == 0) ? (n % 8) * (nwg / 8) + n / 8 : n;
    // Every role decodes the job itself, so that no part of it stays live
    // across the role branch.
#define GDN_JOB decode_job<DK, DV, true>(L, q, k, v, gin, betain, h0, o, ht, nullptr, T, H, sg)
    {
        const WgJob job = GDN_JOB;
        // the upper tiles of T - I are read by the consumers but never written;
        // a walk with zero values never stores V
        for (int idx = tid; idx < 2 * BT * C::LDP; idx += kWalkThreads) (&sm.Tm[0][0])[idx] = (_Float16)0.f;
        if (job.ha.zero_v)
            for (int idx = tid; idx < 2 * BT * C::LDV; idx += kWalkThreads) (&sm.V[0][0])[idx] = 0;
    }
    if (wave == 1 || wave == 2) {
        const WgJob job = GDN_JOB;
        const int NT = (job.ha.T + BT - 1) / BT;
        run_consumer<DK, DV, false>(sm, job, NT, wave - 1, scale, lane);
    } else if (wave == 0) {
        const WgJob job = GDN_JOB;
        const int NT = (job.ha.T + BT - 1) / BT;
        __syncthreads();
        for (int c = -1; c < NT; ++c) {
            if (c + 1 < NT) unit_lower_inverse<C::LDP>(sm.A[(c + 1) & 1], sm.Tm[(c + 1) & 1], lane);
            __syncthreads();
        }
    } else {
        const WgJob job = GDN_JOB;
        const HeadArgs &ha = job.ha;
        const int NT = (ha.T + BT - 1) / BT;
        if (ha.zero_v) run_walk_producer<DK, DV, true>(sm, ha, NT, scale, lane);
        else run_walk_producer<DK, DV, false>(sm, ha, NT, scale, lane);
    }
#undef GDN_JOB
}

// Producer of the states walk: the raw K rows of chunk c + 2 and the V tile
// and gate tables of chunk c + 1 in iteration c (run_walk_producer without A:
// the states walk reads T - I from memory).
template <int DK, int DV>
__device__ __forceinline__ void run_states_producer(FusedSmem<DK, DV> &sm, const HeadArgs &ha, int NT, int lane) {
    using C = FusedCfg<DK, DV>;
    ChunkRegs<C::NS> RA, RP;
    // chunk c2's rows (in RA) to kq-buffer kb, then fetch chunk c2 + 1's
    auto put_k = [&](int c2, int kb) {
        write_rows<DK>(sm.K[kb], RA.k, lane);
        load_rows<DK>(RA.k, ha.k, ha, min(c2 + 1, NT - 1), lane);
    };
    if (NT > 0) {
        load_rows<DK>(RA.k, ha.k, ha, 0, lane);
        load_v<DV>(RP.v, ha, 0, lane);
        load_gates(RP.g, RP.beta, ha, 0, lane);
        put_k(0, 0);
    }
    __syncthreads();
    for (int c2 = 1; c2 <= NT + 1; c2 += 3) {
        if (c2 < NT) put_k(c2, 1);
        if (c2 - 1 < NT) produce_P<DK, DV, false, false>(sm, RP, c2 - 1, 0, NT, ha, 1.f, lane);
        __syncthreads();
        if (c2 + 1 <= NT + 1) {
            if (c2 + 1 < NT) put_k(c2 + 1, 2);
            if (c2 < NT) produce_P<DK, DV, false, false>(sm, RP, c2, 1, NT, ha, 1.f, lane);
            __syncthreads();
        }
        if (c2 + 2 <= NT + 1) {
            if (c2 + 2 < NT) put_k(c2 + 2, 0);
            if (c2 + 1 < NT) produce_P<DK, DV, false, false>(sm, RP, c2 + 1, 2, NT, ha, 1.f, lane);
            __syncthreads();
        }
    }
}

// T - I of chunk c + 1 from memory (fp32 [64][64] per chunk, this head's
// chunks from Tw on) into LDS half (c + 1) & 1 in iteration c, as fp16 hi
// (the T - I buffer) and lo (the P buffer) parts; the next chunk's is
// fetched into registers meanwhile.
template <int DK, int DV>
__device__ __forceinline__ void run_tm_loader(FusedSmem<DK, DV> &sm, const float *__restrict__ Tw, int NT, int lane) {
    using C = FusedCfg<DK, DV>;
    constexpr int U = BT * BT / 4 / 64;  // 16-byte pieces per lane
    f32x4 x[U];
    auto fetch = [&](int c) {
        const float *src = Tw + (long)c * BT * BT;
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = *(const f32x4 *)(src + 4 * (lane + 64 * u));
    };
    auto put = [&](int c) {
        _Float16 *hi = sm.Tm[c & 1], *lo = sm.P[c & 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = 4 * (lane + 64 * u), row = idx / BT, col = idx % BT;
            const f16x4 h = __builtin_convertvector(x[u], f16x4);
            const f16x4 l = __builtin_convertvector(x[u] - __builtin_convertvector(h, f32x4), f16x4);
            *(f16x4 *)&hi[row * C::LDP + col] = h;
            *(f16x4 *)&lo[row * C::LDP + col] = l;
        }
    };
    if (NT > 0) fetch(0);
    __syncthreads();
    for (int c = -1; c < NT; ++c) {
        if (c + 1 < NT) {
            put(c + 1);
            if (c + 2 < NT) fetch(c + 2);
        }
        __syncthreads();
    }
}

// The forward walk of every dense sequence, storing the state that enters each
// chunk, states[b, h, c] ([DK][DV] fp32), and nothing else: the recompute of
// a backward pass.  T - I comes from memory (Tws: fp32 [B, H, NT, 64, 64])
// and enters the products as fp16 hi + lo parts, as do the residuals, so the
// stored states keep the accuracy the backward needs.  Four waves, one per
// SIMD: T - I loader, two consumers, K/V/gate producer.
template <int DK, int DV>
__global__ __launch_bounds__(kWalkThreads, 1) void fused_states_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v,
                                                         const float *__restrict__ gin,
                                                         const float *__restrict__ betain,
                                                         const float *__restrict__ Tws,
                                                         const float *__restrict__ h0, float *__restrict__ states,
                                                         int T, int H) {
    using C = FusedCfg<DK, DV>;
    static_assert(sizeof(FusedSmem<DK, DV>) <= 160 * 1024, "LDS budget");
    __shared__ FusedSmem<DK, DV> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x, nwg = gridDim.x;
    const int L = (nwg % 8 == 0) ? (n % 8) * (nwg / 8) + n / 8 : n;
    const SegArgs none{};
    const int NT = (T + BT - 1) / BT;
    const long bh = L / (DV / C::BV);
#define GDN_JOB decode_job<DK, DV, false>(L, q, k, v, gin, betain, h0, nullptr, nullptr, nullptr, T, H, none)
    if (wave == 1 || wave == 2) {
        const WgJob job = GDN_JOB;
        run_consumer<DK, DV, false, true, true>(sm, job, NT, wave - 1, 1.f, lane,
                                                states + bh * NT * (long)DK * DV);
    } else if (wave == 0) {
        run_tm_loader(sm, Tws + bh * NT * (long)BT * BT, NT, lane);
    } else {
        const WgJob job = GDN_JOB;
        run_states_producer(sm, job.ha, NT, lane);
    }
#undef GDN_JOB
}

// Scan over the segments of one head, for a 32-column slice of the state:
// Hin[b NS] = h0 (zeros when null); S = Hin[b NS + 1]; for s = 1 .. NS - 2:
// S = M_s S + Hin[b NS + s + 1] (which holds E_s), stored back.  fp32 FMA with
// M_s and the slice staged in LDS.  Workgroup 0 also writes the segment
// offsets cu[n] (n = b NS + s: b T + s L 64; cu[B NS] = B T).
template <int D>
__global__ __launch_bounds__(256) void seg_scan_kernel(float *__restrict__ Hin, const float *__restrict__ M,
                                                       const float *__restrict__ h0, int *__restrict__ cu, int B,
                                                       int T, int H, int NS, int L) {
    constexpr int CW = 32;
    __shared__ float sM[D * (D + 1)];
    __shared__ __align__(16) float sS[D * CW];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0)
        for (int n = tid; n <= B * NS; n += 256) {
            const int bb = n / NS, sg = n % NS;
            cu[n] = n == B * NS ? B * T : bb * T + min(sg * L * BT, T);
        }
    const int slice = blockIdx.x % (D / CW);
    const long bh = blockIdx.x / (D / CW);
    const long b = bh / H, h = bh % H;
    const long hs = (long)D * D;
    const int col = tid % CW, rg = tid / CW;  // 8 row groups of D / 8 rows
    constexpr int RPT = D / 8;
    // Each thread requests all of its loads of a stage before its first
    // store; the workspace sections move in float4 pieces (16-byte aligned
    // rows), the caller's h0 element by element.
    constexpr int SV = D * CW / 4 / 256, MV = D * D / 4 / 256;  // float4 per thread
    float *H0 = Hin + ((b * NS + 0) * H + h) * hs;
    {
        float hv[4 * SV];
#pragma unroll
        for (int x = 0; x < 4 * SV; ++x) {
            const int idx = tid + 256 * x;
            hv[x] = h0 ? h0[bh * hs + (long)(idx / CW) * D + slice * CW + idx % CW] : 0.f;
        }
#pragma unroll
        for (int x = 0; x < 4 * SV; ++x) {
            const int idx = tid + 256 * x;
            H0[(long)(idx / CW) * D + slice * CW + idx % CW] = hv[x];
        }
    }
    float *E1 = Hin + ((b * NS + 1) * H + h) * hs;
    {
        float4 ev[SV];
#pragma unroll
        for (int x = 0; x < SV; ++x) {
            const int idx = 4 * (tid + 256 * x);
            ev[x] = *(const float4 *)(E1 + (long)(idx / CW) * D + slice * CW + idx % CW);
        }
#pragma unroll
        for (int x = 0; x < SV; ++x) *(float4 *)&sS[4 * (tid + 256 * x)] = ev[x];
    }
    for (int sgm = 1; sgm <= NS - 2; ++sgm) {
        const float *Ms = M + ((b * NS + sgm) * H + h) * hs;
        float *Es = Hin + ((b * NS + sgm + 1) * H + h) * hs;
        float4 mv[MV];
#pragma unroll
        for (int x = 0; x < MV; ++x) mv[x] = *(const float4 *)(Ms + 4 * (tid + 256 * x));
        __syncthreads();
#pragma unroll
        for (int x = 0; x < MV; ++x) {
            const int idx = 4 * (tid + 256 * x), row = idx / D, c = idx % D;
            float *d = &sM[row * (D + 1) + c];  // padded rows: four scalar stores
            d[0] = mv[x].x;
            d[1] = mv[x].y;
            d[2] = mv[x].z;
            d[3] = mv[x].w;
        }
        __syncthreads();
        float acc[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) acc[i] = Es[(long)(rg * RPT + i) * D + slice * CW + col];
        for (int kk = 0; kk < D; ++kk) {
            const float sv = sS[kk * CW + col];
#pragma unroll
            for (int i = 0; i < RPT; ++i) acc[i] = fmaf(sM[(rg * RPT + i) * (D + 1) + kk], sv, acc[i]);
        }
        __syncthreads();  // every thread has read sS
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            sS[(rg * RPT + i) * CW + col] = acc[i];
            Es[(long)(rg * RPT + i) * D + slice * CW + col] = acc[i];
        }
    }
}

// Final state of each sequence: the last segment's, Hout[b NS + NS - 1] -> ht[b].
__global__ __launch_bounds__(256) void seg_final_kernel(const float *__restrict__ Hout, float *__restrict__ ht,
                                                        long per_seq, int NS) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    const long b = blockIdx.y;
    if (i < per_seq) ht[b * per_seq + i] = Hout[(b * NS + NS - 1) * per_seq + i];
}

template <int DK, int DV>
static hipError_t launch_fused_t(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                 const float *h0, float *o, float *ht, const int *cu_seqlens, int B, int T, int H,
                                 float scale, hipStream_t st) {
    const long grid = (long)B * H * (DV / FusedCfg<DK, DV>::BV);
    hipLaunchKernelGGL((fused_kernel<DK, DV>), dim3((unsigned)grid), dim3(kFusedThreads), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, g, beta, h0, o, ht, cu_seqlens, T, H, scale);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fused_seg_t(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                     const float *h0, float *o, float *ht, int B, int T, int H, float scale, int NS,
                                     int L, float *Hin, float *Hout, float *M, int *cu, hipStream_t st) {
    constexpr int W = D / FusedCfg<D, D>::BV;
    const SegArgs sg{L, NS, Hin, M};
    const long gridA = (long)B * H * (W + 2 * W * (NS - 2));
    hipLaunchKernelGGL((fused_walk_kernel<D, D>), dim3((unsigned)gridA), dim3(kWalkThreads), 0, st,
                       (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, g, beta, h0, (float *)nullptr,
                       (float *)nullptr, T, H, scale, sg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((seg_scan_kernel<D>), dim3((unsigned)(B * H * (D / 32))), dim3(256), 0, st, Hin,
                       (const float *)M, h0, cu, B, T, H, NS, L);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_fused_t<D, D>(q, k, v, g, beta, Hin, o, ht ? Hout : nullptr, cu, B * NS, B * T, H, scale, st);
    if (e != hipSuccess || !ht) return e;
    const long per_seq = (long)H * D * D;
    hipLaunchKernelGGL(seg_final_kernel, dim3((unsigned)((per_seq + 255) / 256), (unsigned)B), dim3(256), 0, st,
                       (const float *)Hout, ht, per_seq, NS);
    return hipGetLastError();
}

hipError_t launch_fused_seg_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                 const float *h0, float *o, float *ht, int B, int T, int H, int D, float scale,
                                 int NS, int L, float *Hin, float *Hout, float *M, int *cu, hipStream_t st) {
    if (NS < 2) return hipErrorInvalidValue;
    if (D == 64)
        return launch_fused_seg_t<64>(q, k, v, g, beta, h0, o, ht, B, T, H, scale, NS, L, Hin, Hout, M, cu, st);
    if (D == 128)
        return launch_fused_seg_t<128>(q, k, v, g, beta, h0, o, ht, B, T, H, scale, NS, L, Hin, Hout, M, cu, st);
    return hipErrorInvalidValue;
}

hipError_t launch_fused_states_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                    const float *Tws, const float *h0, float *states, int B, int T, int H, int Dk,
                                    int Dv, hipStream_t st) {
#define GDN_STATES(DKv, DVv)                                                                                    \
    if (Dk == DKv && Dv == DVv) {                                                                               \
        const long grid = (long)B * H * (DVv / FusedCfg<DKv, DVv>::BV);                                         \
        hipLaunchKernelGGL((fused_states_kernel<DKv, DVv>), dim3((unsigned)grid), dim3(kWalkThreads), 0, st,    \
                           (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, g, beta, Tws, h0, states, \
                           T, H);                                                                                  \
        return hipGetLastError();                                                                               \
    }
    GDN_STATES(64, 64);
    GDN_STATES(64, 128);
    GDN_STATES(128, 64);
    GDN_STATES(128, 128);
#undef GDN_STATES
    return hipErrorInvalidValue;
}

hipError_t launch_fused_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                             const float *h0, float *o, float *ht, const int *cu_seqlens, int B, int T, int H, int Dk,
                             int Dv, float scale, hipStream_t st) {
#define GDN_FUSED(DKv, DVv)                                                                                     \
    if (Dk == DKv && Dv == DVv)                                                                                 \
    return launch_fused_t<DKv, DVv>(q, k, v, g, beta, h0, o, ht, cu_seqlens, B, T, H, scale, st)
    GDN_FUSED(64, 64);
    GDN_FUSED(64, 128);
    GDN_FUSED(128, 64);
    GDN_FUSED(128, 128);
#undef GDN_FUSED
    return hipErrorInvalidValue;
}

}  // namespace gdn
