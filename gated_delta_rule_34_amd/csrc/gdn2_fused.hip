// gdn2_fused.hip -- chunked Gated DeltaNet-2 forward for bf16 inputs on
// gfx950, in two kernels.
//
// Recurrence (Gated DeltaNet-2 article, "Regla-2 del Delta cerrado"): per
// token, S <- Diag(alpha) S, u = w . v - S^T (b . k), S <- S + k u^T, and the
// readout o = scale S^T q.  Chunk form over 64 tokens, with the chunk-local
// per-channel log-decay sums G_i = sum_{s<=i} log alpha_s and Gamma_i = e^{G_i}
// (the chunked-training section of the same article: the channel decay is
// absorbed into both factors of each product):
//   A_ij = sum_c b_ic k_ic k_jc e^{G_ic - G_jc}        (j < i)
//   P_ij = sum_c q_ic k_jc e^{G_ic - G_jc}             (j <= i)
//   Vnew = (I + A)^-1 (w . V - Ehat S),   Ehat_i = Gamma_i . b_i . k_i
//   O    = scale (Qhat S + P Vnew),       Qhat_i = Gamma_i . q_i
//   S'   = Diag(Gamma_C) S + Khat^T Vnew, Khat_j = k_j . Gamma_C / Gamma_j
//
// prep kernel (persistent: one workgroup per compute unit, looping over the
// (batch, head, chunk) blocks, with the next chunk's raw rows and
// log-decays fetched into registers while the current chunk is computed):
// the cumsum, Ehat, Qhat, Khat, Gamma_C, T - I = (I + A)^-1 - I and the
// strict and diagonal parts of P, written as one block per chunk.
//   Off-diagonal 16x16 blocks of A and P are fp16 MFMA products of factors
//   anchored at the first row a of the block row: (x_i e^{G_i - G_a}) and
//   (k_j e^{G_a - G_j}), both at most 1 in size since j < a <= i.  Diagonal
//   blocks are anchored at their own first row, with the fp32 factors split
//   into bf16 hi + lo parts on bf16 MFMA (hi.hi + hi.lo + lo.hi), while the
//   block's decay keeps both factors inside 2^(+-100); otherwise they are
//   summed directly.
// walk kernel (one workgroup per (batch, head, 32 value columns)): two
//   consumer waves carry the state in registers through the chunks, two
//   loader waves stage the next chunk's block and value slices into LDS.
// When the walk leaves at least half of the compute units idle, the chunks
// run in time parts: the prep of part p and the walk of part p - 1 share one
// launch (gdn2_pipe_kernel) on disjoint workgroups, and the state crosses the
// launches in an fp32 carry in the workspace.
//
// Precision: Ehat, Qhat, Khat, T - I and P are fp16; the state enters K S and
// Q S as fp16 hi + lo parts and Vnew enters the state update the same way;
// accumulation, the state and the output are fp32.  fp16 operands bound the
// state entries below 65504.
#include "gdn_launch.h"
#include "gdn_tile.h"

namespace gdn {

// Per-chunk block of the workspace (all offsets in bytes, 256-aligned total).
template <int DK>
struct Gdn2Blk {
    static constexpr int E = 0;                       // fp16 [64][DK]
    static constexpr int Q = E + BT * DK * 2;         // fp16 [64][DK]
    static constexpr int K = Q + BT * DK * 2;         // fp16 [64][DK]
    static constexpr int TM = K + BT * DK * 2;        // fp16 [64][64], T - I (lower tiles)
    static constexpr int PM = TM + BT * BT * 2;       // fp16 [64][64], strict lower P
    static constexpr int DG = PM + BT * BT * 2;       // fp32 [64], P_ii = q_i . k_i
    static constexpr int GAM = DG + BT * 4;           // fp32 [DK], Gamma_C
    static constexpr int BYTES = (GAM + DK * 4 + 255) / 256 * 256;
};

size_t gdn2_fused_block_bytes(int Dk) { return Dk == 64 ? Gdn2Blk<64>::BYTES : Gdn2Blk<128>::BYTES; }

// Packed variable-length sequences.  The chunks of all sequences are numbered
// g = 0 .. NC - 1 in sequence order and the block of (head h, chunk g) is
// block h NC + g of the workspace.  seq[n] = {first token, tokens walked,
// first chunk number, 0} of sequence n (seq[N].z = chunks in use); tab[g] =
// the sequence of chunk g, or N for the unused numbers at the end.  seq null:
// a dense batch.
struct Gdn2Var {
    const int4 *seq;
    const int *tab;
    int N, NC;
};


// --------------------------------------------------------------- prep kernel
template <int DK>
struct Gdn2PrepSmem {
    static constexpr int LDR = DK + 8;   // raw bf16 rows
    static constexpr int LDG = DK + 4;   // fp32 rows of G2
    static constexpr int LDP = BT + 8;   // fp16 rows of A, T - I, P
    static constexpr int NG = 512 / DK;  // row groups of the cumsum
    alignas(16) uint16_t k[BT * LDR];
    alignas(16) uint16_t q[BT * LDR];
    alignas(16) uint16_t b[BT * LDR];
    alignas(16) float G2[BT * LDG];      // log2(e) * chunk-local cumsum of log alpha
    alignas(16) float part[NG][DK];      // per-group totals of the cumsum
    alignas(16) _Float16 A[BT * LDP];
    alignas(16) _Float16 Tm[BT * LDP];
    alignas(16) _Float16 P[BT * LDP];
    alignas(16) float dg[BT];
};

// Four consecutive bf16 values (8 bytes, 8-byte aligned) as floats.
__device__ __forceinline__ f32x4 bf16x4_at(const uint16_t *p) {
    const uint2 u = *(const uint2 *)p;
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}

// Largest |G2[x][c] - G2[a][c]| over the 16 rows x of the block at row a and
// all channels: the size of the anchored factors in log2 units.
template <int DK, int LDG>
__device__ __forceinline__ float block_span(const float *G2, int a, int lane) {
    float m = 0.f;
    for (int c = lane; c < DK; c += 64) {
        const float ga = G2[a * LDG + c];
#pragma unroll
        for (int x = 1; x < 16; ++x) m = fmaxf(m, fabsf(G2[(a + x) * LDG + c] - ga));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    return m;
}

// Diagonal block (rows and columns a .. a + 15) of A and P, one wave.  When
// every channel's decay within the block stays inside 2^(+-100) of row a, the
// block is a product of factors anchored at a, e_i 2^(G2_i - G2_a) and
// k_j 2^(G2_a - G2_j), formed in fp32 (no overflow or underflow of either
// factor) and multiplied on bf16 MFMA as hi + lo parts; otherwise each entry
// is summed directly.
template <int DK>
__device__ __forceinline__ void diag_block(Gdn2PrepSmem<DK> &sm, int a, int lane) {
    using SM = Gdn2PrepSmem<DK>;
    constexpr int LDR = SM::LDR, LDG = SM::LDG, LDP = SM::LDP;
    const int r = lane & 15, g = lane >> 4;
    if (block_span<DK, LDG>(sm.G2, a, lane) < 100.f) {
        f32x4 accA = zero4(), accP = zero4();
        const int i = a + r;  // A-operand row and B-operand column of this lane
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            float fa[8], fq[8], fb[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // columns c0 .. c0 + 3, one read per row and array
                const int c0 = 32 * s + 16 * h + 4 * g;
                const f32x4 Ga = *(const f32x4 *)&sm.G2[a * LDG + c0], Gi = *(const f32x4 *)&sm.G2[i * LDG + c0];
                const f32x4 kk = bf16x4_at(&sm.k[i * LDR + c0]), bb = bf16x4_at(&sm.b[i * LDR + c0]);
                const f32x4 qq = bf16x4_at(&sm.q[i * LDR + c0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ri = __builtin_amdgcn_exp2f(Gi[e] - Ga[e]);
                    fa[4 * h + e] = bb[e] * kk[e] * ri;
                    fq[4 * h + e] = qq[e] * ri;
                    fb[4 * h + e] = kk[e] * __builtin_amdgcn_exp2f(Ga[e] - Gi[e]);
                }
            }
            // bf16 hi + lo parts of each factor; the products hi.hi, hi.lo
            // and lo.hi keep about 16 bits of each factor with fp32's range
            uint4 ah, al, qh, ql, bh, bl;
            hilo_frags<bf16x2>(ah, al, f32x4{fa[0], fa[1], fa[2], fa[3]}, f32x4{fa[4], fa[5], fa[6], fa[7]});
            hilo_frags<bf16x2>(qh, ql, f32x4{fq[0], fq[1], fq[2], fq[3]}, f32x4{fq[4], fq[5], fq[6], fq[7]});
            hilo_frags<bf16x2>(bh, bl, f32x4{fb[0], fb[1], fb[2], fb[3]}, f32x4{fb[4], fb[5], fb[6], fb[7]});
            accA = mma_bf16_raw(accA, ah, bh);
            accP = mma_bf16_raw(accP, qh, bh);
            accA = mma_bf16_raw(accA, ah, bl);
            accP = mma_bf16_raw(accP, qh, bl);
            accA = mma_bf16_raw(accA, al, bh);
            accP = mma_bf16_raw(accP, ql, bh);
        }
        // lane holds [a + 4g + e][a + r]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ii = 4 * g + e;
            if (r < ii) {
                sm.A[(a + ii) * LDP + a + r] = (_Float16)accA[e];
                sm.P[(a + ii) * LDP + a + r] = (_Float16)accP[e];
            } else if (r == ii) {
                sm.dg[a + ii] = accP[e];
            }
        }
    } else {
        for (int pr = lane; pr < 256; pr += 64) {
            const int il = pr >> 4, jl = pr & 15;
            if (jl > il) continue;
            const int i = a + il, j = a + jl;
            float pa = 0.f, pp = 0.f;
            for (int c = 0; c < DK; ++c) {
                const float kd = bf16_to_f32(sm.k[j * LDR + c]) *
                                 __builtin_amdgcn_exp2f(sm.G2[i * LDG + c] - sm.G2[j * LDG + c]);
                pa = fmaf(bf16_to_f32(sm.b[i * LDR + c]) * bf16_to_f32(sm.k[i * LDR + c]), kd, pa);
                pp = fmaf(bf16_to_f32(sm.q[i * LDR + c]), kd, pp);
            }
            if (jl < il) {
                sm.A[i * LDP + j] = (_Float16)pa;
                sm.P[i * LDP + j] = (_Float16)pp;
            } else {
                sm.dg[i] = pp;
            }
        }
    }
}

// Off-diagonal tile (I > J) of A and P on fp16 MFMA, anchored at a = 16 I:
// e_i 2^(G2_i - G2_a) and k_j 2^(G2_a - G2_j) are both at most 1 since
// j < a <= i and the log-decays are not positive.
template <int DK>
__device__ __forceinline__ void offdiag_tile(Gdn2PrepSmem<DK> &sm, int t, int lane) {
    using SM = Gdn2PrepSmem<DK>;
    constexpr int LDR = SM::LDR, LDG = SM::LDG, LDP = SM::LDP;
    const int r = lane & 15, g = lane >> 4;
    const int I = t < 1 ? 1 : t < 3 ? 2 : 3;
    const int J = t < 1 ? 0 : t < 3 ? t - 1 : t - 3;
    const int a = 16 * I, i = 16 * I + r, j = 16 * J + r;
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        f16x8 fe, fq, fk;
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // columns c0 .. c0 + 3, one read per row and array
            const int c0 = 32 * s + 16 * h + 4 * g;
            const f32x4 Ga = *(const f32x4 *)&sm.G2[a * LDG + c0], Gi = *(const f32x4 *)&sm.G2[i * LDG + c0];
            const f32x4 Gj = *(const f32x4 *)&sm.G2[j * LDG + c0];
            const f32x4 ki = bf16x4_at(&sm.k[i * LDR + c0]), bi = bf16x4_at(&sm.b[i * LDR + c0]);
            const f32x4 qi = bf16x4_at(&sm.q[i * LDR + c0]), kj = bf16x4_at(&sm.k[j * LDR + c0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ri = __builtin_amdgcn_exp2f(Gi[e] - Ga[e]);
                fe[4 * h + e] = (_Float16)(bi[e] * ki[e] * ri);
                fq[4 * h + e] = (_Float16)(qi[e] * ri);
                fk[4 * h + e] = (_Float16)(kj[e] * __builtin_amdgcn_exp2f(Ga[e] - Gj[e]));
            }
        }
        accA = __builtin_amdgcn_mfma_f32_16x16x32_f16(fe, fk, accA, 0, 0, 0);
        accP = __builtin_amdgcn_mfma_f32_16x16x32_f16(fq, fk, accP, 0, 0, 0);
    }
    // lane holds [16I + 4g + e][16J + r]
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int ii = 16 * I + 4 * g + e, jj = 16 * J + r;
        sm.A[ii * LDP + jj] = (_Float16)accA[e];
        sm.P[ii * LDP + jj] = (_Float16)accP[e];
    }
}

// Persistent: over the chunks c0 .. c0 + nc - 1 of every (batch, head), in
// the order idx = bh nc + (c - c0), workgroup w of nw handles idx = w, w + nw,
// ...  The raw rows and log-decays of its next chunk are fetched into
// registers while the current chunk's A and P tiles are formed, so their
// latency overlaps the current chunk's work.
template <int DK, bool VAR>
__device__ __forceinline__ void prep_run(Gdn2PrepSmem<DK> &sm, const uint16_t *__restrict__ q,
                                         const uint16_t *__restrict__ k, const float *__restrict__ la,
                                         const uint16_t *__restrict__ bg, char *__restrict__ ws, int T, int H, int NT,
                                         int c0, int nc, int nidx, int w0, int nw, const Gdn2Var var) {
    using SM = Gdn2PrepSmem<DK>;
    using BL = Gdn2Blk<DK>;
    constexpr int NTH = 512;
    constexpr int LDR = SM::LDR, LDG = SM::LDG, LDP = SM::LDP, NG = SM::NG;
    constexpr int C8 = DK / 8;      // uint4 per row of a raw tile
    constexpr int RG = BT / NG;     // rows per cumsum group
    constexpr int NU = BT * C8 / NTH;  // uint4 per thread per raw tile
    const int tid0 = threadIdx.x;
    const int ch = tid0 % DK, gr = tid0 / DK;  // cumsum: rows RG gr .. RG gr + RG - 1 of channel ch
    typedef __attribute__((ext_vector_type(4))) unsigned int v4u;  // native vectors stay in registers
    v4u kr[NU], qr[NU], br[NU];
    float lv[RG];

    // the chunk (its index among all chunks: bh NT + c) of position idx
    auto chunk_of = [&](int idx) {
        const int bh = idx / nc;
        return bh * NT + c0 + (idx - bh * nc);
    };
    // token-head row of a chunk's first token, the chunk's first token within
    // its sequence and the sequence's length
    auto locate = [&](int cb, long &row0, int &t0, int &Tc) {  // 32-bit index math (cheap on the VALU)
        if constexpr (VAR) {  // packed sequences: cb = h NC + g
            const int h = cb / var.NC, gc = cb - h * var.NC;
            const int n = var.tab[gc];
            if (n >= var.N) {  // an unused chunk number: token 0 of head h, into its own block
                row0 = h;
                t0 = 0;
                Tc = 1;
                return;
            }
            const int4 sq = var.seq[n];
            t0 = (gc - sq.z) * BT;
            Tc = sq.y;
            row0 = ((long)sq.x + t0) * H + h;
            return;
        }
        const int bh = cb / NT;
        t0 = (cb - bh * NT) * BT;
        const int b = bh / H;
        row0 = ((long)b * T + t0) * H + (bh - b * H);
        Tc = T;
    };
    // raw rows and log-decays of chunk cb into registers; rows past T read the
    // last token (always in bounds) and are zeroed when staged
    auto fetch = [&](int cb) {
        long row0;
        int t0, Tc;
        locate(cb, row0, t0, Tc);
#pragma unroll
        for (int x = 0; x < NU; ++x) {
            const int u = tid0 + NTH * x, row = u / C8, c8 = u % C8;
            const int tr = min(t0 + row, Tc - 1) - t0;
            const long off = (row0 + (long)tr * H) * DK + 8 * c8;
            kr[x] = __builtin_nontemporal_load((const v4u *)(k + off));
            qr[x] = __builtin_nontemporal_load((const v4u *)(q + off));
            br[x] = __builtin_nontemporal_load((const v4u *)(bg + off));
        }
#pragma unroll
        for (int x = 0; x < RG; ++x) {
            const int tr = min(t0 + RG * gr + x, Tc - 1) - t0;
            lv[x] = __builtin_nontemporal_load(&la[(row0 + (long)tr * H) * DK + ch]);
        }
    };

    fetch(chunk_of(w0));  // w0 < nidx: the grid never exceeds the chunk count
    for (int idx = w0; idx < nidx; idx += nw) {
        const int cb = chunk_of(idx);
        // The thread index passes through an opaque move each chunk, so that
        // the many lane-derived LDS addresses below are formed where they are
        // used instead of being hoisted out of the loop into registers.
        int tid;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(tid0));
        const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        long row0;
        int t0, Tc;
        locate(cb, row0, t0, Tc);
        char *blk = ws + (long)cb * BL::BYTES;
        // 1. raw rows (zero past T) and the per-channel cumsum of log alpha
#pragma unroll
        for (int x = 0; x < NU; ++x) {
            const int u = tid + NTH * x, row = u / C8, c8 = u % C8;
            const bool in = t0 + row < Tc;
            const v4u z = {0u, 0u, 0u, 0u};
            *(v4u *)&sm.k[row * LDR + 8 * c8] = in ? kr[x] : z;
            *(v4u *)&sm.q[row * LDR + 8 * c8] = in ? qr[x] : z;
            *(v4u *)&sm.b[row * LDR + 8 * c8] = in ? br[x] : z;
        }
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < RG; ++x) {
            acc += (t0 + RG * gr + x < Tc) ? lv[x] * 1.4426950408889634f : 0.f;
            lv[x] = acc;
        }
        sm.part[gr][ch] = acc;
        // the upper tiles of T - I and P are never written below
        for (int u = tid; u < BT * LDP; u += NTH) {
            sm.Tm[u] = (_Float16)0.f;
            sm.P[u] = (_Float16)0.f;
        }
        __syncthreads();
        {
            float off = 0.f;
            for (int x = 0; x < gr; ++x) off += sm.part[x][ch];
#pragma unroll
            for (int x = 0; x < RG; ++x) sm.G2[(RG * gr + x) * LDG + ch] = lv[x] + off;
        }
        __syncthreads();

        // 2. A and P: waves 0..3 the diagonal blocks, waves 4..7 the 6 off-diagonal tiles.
        // The staging registers are free now, so the next chunk is fetched here:
        // first by waves 4 and 5, which have two tiles each, and by the others
        // after their tile, where they would otherwise wait at the barrier.
        const bool more = idx + nw < nidx, fetch_first = wave == 4 || wave == 5;
        const int cnext = more ? chunk_of(idx + nw) : 0;
        if (fetch_first && more) fetch(cnext);
        if (wave < 4) {
            diag_block<DK>(sm, 16 * wave, lane);
        } else {
            offdiag_tile<DK>(sm, wave - 4, lane);
            if (wave < 6) offdiag_tile<DK>(sm, wave, lane);
        }
        if (!fetch_first && more) fetch(cnext);
        __syncthreads();

        // 3. wave 0: T - I; the other waves: decayed operands, Gamma_C, P, diag P
        if (wave == 0) {
            unit_lower_inverse<LDP>(sm.A, sm.Tm, lane);
        } else {
            const int ot = tid - 64;  // 0 .. 447
            for (int u = ot; u < BT * C8; u += NTH - 64) {
                const int row = u / C8, c0 = 8 * (u % C8);
                const uint4 kv = *(const uint4 *)&sm.k[row * LDR + c0];
                const uint4 qv = *(const uint4 *)&sm.q[row * LDR + c0];
                const uint4 bv = *(const uint4 *)&sm.b[row * LDR + c0];
                const uint16_t *kk = (const uint16_t *)&kv, *qq = (const uint16_t *)&qv, *bq = (const uint16_t *)&bv;
                f16x8 eo, qo, ko;
                const f32x4 G0 = *(const f32x4 *)&sm.G2[row * LDG + c0];
                const f32x4 G1 = *(const f32x4 *)&sm.G2[row * LDG + c0 + 4];
                const f32x4 L0 = *(const f32x4 *)&sm.G2[(BT - 1) * LDG + c0];
                const f32x4 L1 = *(const f32x4 *)&sm.G2[(BT - 1) * LDG + c0 + 4];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float G = e < 4 ? G0[e] : G1[e - 4], GL = e < 4 ? L0[e] : L1[e - 4];
                    const float gam = __builtin_amdgcn_exp2f(G);
                    const float kf = bf16_to_f32(kk[e]);
                    eo[e] = (_Float16)(bf16_to_f32(bq[e]) * kf * gam);
                    qo[e] = (_Float16)(bf16_to_f32(qq[e]) * gam);
                    ko[e] = (_Float16)(kf * __builtin_amdgcn_exp2f(GL - G));
                }
                const long o = ((long)row * DK + c0) * 2;
                *(f16x8 *)(blk + BL::E + o) = eo;
                *(f16x8 *)(blk + BL::Q + o) = qo;
                *(f16x8 *)(blk + BL::K + o) = ko;
            }
            for (int u = ot; u < BT * 8; u += NTH - 64) {
                const int row = u >> 3, c0 = 8 * (u & 7);
                *(uint4 *)(blk + BL::PM + (row * BT + c0) * 2) = *(const uint4 *)&sm.P[row * LDP + c0];
            }
            if (ot < BT) ((float *)(blk + BL::DG))[ot] = sm.dg[ot];
            if (ot >= BT && ot < BT + DK)
                ((float *)(blk + BL::GAM))[ot - BT] = __builtin_amdgcn_exp2f(sm.G2[(BT - 1) * LDG + ot - BT]);
        }
        __syncthreads();
        // 4. T - I out
        for (int u = tid; u < BT * 8; u += NTH) {
            const int row = u >> 3, c0 = 8 * (u & 7);
            *(uint4 *)(blk + BL::TM + (row * BT + c0) * 2) = *(const uint4 *)&sm.Tm[row * LDP + c0];
        }
        __syncthreads();  // this chunk's LDS is read before the next one is staged
    }
}

template <int DK, bool VAR>
__global__ __launch_bounds__(512) void gdn2_prep_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                         const float *__restrict__ la, const uint16_t *__restrict__ bg,
                                                         char *__restrict__ ws, int T, int H, int NT, int c0, int nc,
                                                         int nidx, Gdn2Var var) {
    __shared__ Gdn2PrepSmem<DK> sm;
    prep_run<DK, VAR>(sm, q, k, la, bg, ws, T, H, NT, c0, nc, nidx, blockIdx.x, gridDim.x, var);
}

// --------------------------------------------------------------- walk kernel
template <int DK, int DV>
struct Gdn2WalkCfg {
    static constexpr int BV = 32;
    static constexpr int NS = DK / 32;
    static constexpr int NKB = DK / 16;
    static constexpr int LDK = DK;   // paired-group rows (tile_off_pg), unpadded
    static constexpr int LDP = BT + 8;    // fp16 rows of T - I and P (16-byte aligned)
    static constexpr int LDV = BV + 8;   // bf16 rows of the v and w slices
    static constexpr int UT = BT * DK / 8 / 128;  // uint4 per loader thread per DK tile
};

template <int DK, int DV>
struct Gdn2WalkSmem {
    using C = Gdn2WalkCfg<DK, DV>;
    alignas(16) uint16_t E[2][BT * C::LDK];   // fp16 bits, paired-group layout (tile_off_pg)
    alignas(16) uint16_t Q[2][BT * C::LDK];
    alignas(16) uint16_t K[2][BT * C::LDK];
    alignas(16) _Float16 Tm[2][BT * C::LDP];
    alignas(16) _Float16 P[2][BT * C::LDP];
    alignas(16) uint16_t V[2][BT * C::LDV];   // raw bf16
    alignas(16) uint16_t W[2][BT * C::LDV];
    alignas(16) float dg[2][BT];
    alignas(16) float gam[2][DK];
};

struct Gdn2Head {
    const char *ws;      // this head's first chunk block
    const uint16_t *v, *w;
    long row0;           // token-head row of token 0 of this head
    int T, H, vcol0;
};

// Everything a loader thread moves for one chunk, as native 16-byte vectors
// (HIP's uint4 is a struct the compiler keeps in scratch memory here).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <int DK>
struct Gdn2Stage {
    u32x4 e[Gdn2WalkCfg<DK, DK>::UT], q[Gdn2WalkCfg<DK, DK>::UT], k[Gdn2WalkCfg<DK, DK>::UT];
    u32x4 tm[4], p[4], v[2], w[2], tab;
};

template <int DK, int DV>
__device__ __forceinline__ void stage_load(Gdn2Stage<DK> &R, const Gdn2Head &hd, int chunk, int lt) {
    using BL = Gdn2Blk<DK>;
    using C = Gdn2WalkCfg<DK, DV>;
    const char *blk = hd.ws + (long)chunk * BL::BYTES;
#pragma unroll
    for (int x = 0; x < C::UT; ++x) {
        const int u = lt + 128 * x;
        R.e[x] = *(const u32x4 *)(blk + BL::E + u * 16);
        R.q[x] = *(const u32x4 *)(blk + BL::Q + u * 16);
        R.k[x] = *(const u32x4 *)(blk + BL::K + u * 16);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int u = lt + 128 * x;
        R.tm[x] = *(const u32x4 *)(blk + BL::TM + u * 16);
        R.p[x] = *(const u32x4 *)(blk + BL::PM + u * 16);
    }
    // dg (16 uint4) then Gamma_C (DK / 4 uint4), contiguous in the block
    R.tab = (lt < 16 + DK / 4) ? *(const u32x4 *)(blk + BL::DG + lt * 16) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int u = lt + 128 * x, row = u >> 2, c4 = u & 3;
        const int t = chunk * BT + row;
        const long off = (hd.row0 + (long)t * hd.H) * DV + hd.vcol0 + 8 * c4;
        const bool in = t < hd.T;
        R.v[x] = in ? __builtin_nontemporal_load((const u32x4 *)(hd.v + off)) : (u32x4){0u, 0u, 0u, 0u};
        R.w[x] = in ? __builtin_nontemporal_load((const u32x4 *)(hd.w + off)) : (u32x4){0u, 0u, 0u, 0u};
    }
}

template <int DK, int DV>
__device__ __forceinline__ void stage_store(Gdn2WalkSmem<DK, DV> &sm, const Gdn2Stage<DK> &R, int buf, int lt) {
    using C = Gdn2WalkCfg<DK, DV>;
    constexpr int C8 = DK / 8;
#pragma unroll
    for (int x = 0; x < C::UT; ++x) {
        const int u = lt + 128 * x, row = u / C8, c0 = 8 * (u % C8);
        // the two 4-column halves of each 16-byte piece go to their stored groups
        const int lo = tile_off_pg<DK>(row, pair_col(c0)), hi = tile_off_pg<DK>(row, pair_col(c0 + 4));
        *(uint2 *)&sm.E[buf][lo] = make_uint2(R.e[x].x, R.e[x].y);
        *(uint2 *)&sm.E[buf][hi] = make_uint2(R.e[x].z, R.e[x].w);
        *(uint2 *)&sm.Q[buf][lo] = make_uint2(R.q[x].x, R.q[x].y);
        *(uint2 *)&sm.Q[buf][hi] = make_uint2(R.q[x].z, R.q[x].w);
        *(uint2 *)&sm.K[buf][lo] = make_uint2(R.k[x].x, R.k[x].y);
        *(uint2 *)&sm.K[buf][hi] = make_uint2(R.k[x].z, R.k[x].w);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int u = lt + 128 * x, row = u >> 3, c0 = 8 * (u & 7);
        *(u32x4 *)&sm.Tm[buf][row * C::LDP + c0] = R.tm[x];
        *(u32x4 *)&sm.P[buf][row * C::LDP + c0] = R.p[x];
    }
    if (lt < 16)
        *(u32x4 *)&sm.dg[buf][4 * lt] = R.tab;
    else if (lt < 16 + DK / 4)
        *(u32x4 *)&sm.gam[buf][4 * (lt - 16)] = R.tab;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int u = lt + 128 * x, row = u >> 2, c0 = 8 * (u & 3);
        *(u32x4 *)&sm.V[buf][row * C::LDV + c0] = R.v[x];
        *(u32x4 *)&sm.W[buf][row * C::LDV + c0] = R.w[x];
    }
}

// One chunk on consumer wave `wave` (value columns 16 wave .. +15 of the
// slice); S holds d_k x 16 of the state as accumulator tiles.
template <int DK, int DV>
__device__ __forceinline__ void gdn2_consume(Gdn2WalkSmem<DK, DV> &sm, f32x4 (&S)[DK / 16], int buf,
                                             float *__restrict__ o, const Gdn2Head &hd, int chunk, int wave,
                                             float scale, int lane) {
    using C = Gdn2WalkCfg<DK, DV>;
    const int r = lane & 15, g = lane >> 4;
    // X = Ehat S, Y = Qhat S with the state as fp16 hi + lo.  Every fragment
    // of the chunk is requested first and the w . v elements after them, so
    // the 64 MFMAs run back to back behind one wait on the LDS.
    f32x4 X[4], Y[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) X[I] = Y[I] = zero4();
    uint4 ea[C::NS][4], qa[C::NS][4];
#pragma unroll
    for (int s = 0; s < C::NS; ++s)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            ea[s][I] = frag_rows_pg<DK>(sm.E[buf], 16 * I, 32 * s, lane);
            qa[s][I] = frag_rows_pg<DK>(sm.Q[buf], 16 * I, 32 * s, lane);
        }
    const int cl = wave * 16 + r;
    uint16_t wr[4][4], vr[4][4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            wr[I][e] = sm.W[buf][i * C::LDV + cl];
            vr[I][e] = sm.V[buf][i * C::LDV + cl];
        }
    uint4 shi[C::NS], slo[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) hilo_frags<f16x2>(shi[s], slo[s], S[2 * s], S[2 * s + 1]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        // all hi-part products, then all lo-part products: an accumulator's
        // two updates are eight MFMAs apart
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            X[I] = mma_f16_raw(X[I], ea[s][I], shi[s]);
            Y[I] = mma_f16_raw(Y[I], qa[s][I], shi[s]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            X[I] = mma_f16_raw(X[I], ea[s][I], slo[s]);
            Y[I] = mma_f16_raw(Y[I], qa[s][I], slo[s]);
        }
    }
    f32x4 wv[4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[I][e] = bf16_to_f32(wr[I][e]) * bf16_to_f32(vr[I][e]);
    // R = w . v - X
    f32x4 Rr[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) Rr[I] = wv[I] - X[I];
    // Vnew = R + (T - I) R
    _Float16 rf[2][8];
    frag_from_acc(rf[0], Rr[0], Rr[1]);
    frag_from_acc(rf[1], Rr[2], Rr[3]);
    f32x4 Vn[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        Vn[I] = Rr[I];
#pragma unroll
        for (int s = 0; s <= (I >> 1); ++s) {
            _Float16 a[8];
            frag_rows(a, sm.Tm[buf], C::LDP, 16 * I, 32 * s, lane);
            Vn[I] = mma_slab(Vn[I], a, rf[s]);
        }
    }
    // The state carry comes first: it is what the next chunk waits for, and
    // the output work below overlaps its MFMAs.
    // S = Diag(Gamma_C) S + Khat^T Vnew, Khat^T by transpose loads, Vnew as fp16 hi + lo
    uint4 vh[2], vl[2];
    hilo_frags<f16x2>(vh[0], vl[0], Vn[0], Vn[1]);
    hilo_frags<f16x2>(vh[1], vl[1], Vn[2], Vn[3]);
    uint4 ka[C::NKB][2];
#pragma unroll
    for (int m = 0; m < C::NKB; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) ka[m][s] = frag_T_pg<DK>(sm.K[buf], 32 * s, 16 * m, lane);
#pragma unroll
    for (int m = 0; m < C::NKB; ++m) {
        const f32x4 gm = *(const f32x4 *)&sm.gam[buf][16 * m + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][e] *= gm[e];
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int m = 0; m < C::NKB; ++m) S[m] = mma_f16_raw(S[m], ka[m][s], vh[s]);
#pragma unroll
        for (int m = 0; m < C::NKB; ++m) S[m] = mma_f16_raw(S[m], ka[m][s], vl[s]);
    }
    // O = scale (Y + diag(P) Vnew + strict(P) Vnew); each row block leaves
    // the MFMA as 4 rows of one column per lane and is stored, after a quad
    // transpose, as 4 adjacent columns of one row (16 bytes per lane)
    _Float16 vf[2][8];
    frag_from_acc(vf[0], Vn[0], Vn[1]);
    frag_from_acc(vf[1], Vn[2], Vn[3]);
    const int t0 = chunk * BT;
    const bool full = t0 + BT <= hd.T;
    const int qb = r & 3;
    float *ob = o + (hd.row0 + (long)(t0 + 4 * g + qb) * hd.H) * DV + hd.vcol0 + wave * 16 + 4 * (r >> 2);
    const long ostride = (long)hd.H * DV;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const f32x4 dgv = *(const f32x4 *)&sm.dg[buf][16 * I + 4 * g];
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = Y[I][e] + dgv[e] * Vn[I][e];
#pragma unroll
        for (int s = 0; s <= (I >> 1); ++s) {
            _Float16 a[8];
            frag_rows(a, sm.P[buf], C::LDP, 16 * I, 32 * s, lane);
            acc = mma_slab(acc, a, vf[s]);
        }
        const f32x4 v = quad_transpose(acc * scale, lane);
        if (full || t0 + 16 * I + 4 * g + qb < hd.T) *(f32x4 *)&ob[16 * I * ostride] = v;
    }
}

// The walk over chunks c0 .. c1 - 1 of one (batch, head, 32 value columns):
// workgroup n of nwg.  Waves 0 and 1 carry the state, waves 2 and 3 stage the
// blocks; any further waves of the workgroup only keep the barrier count.
template <int DK, int DV, bool VAR>
__device__ __forceinline__ void walk_run(Gdn2WalkSmem<DK, DV> &sm, const char *__restrict__ ws,
                                         const uint16_t *__restrict__ v, const uint16_t *__restrict__ wg,
                                         const float *__restrict__ h0, float *__restrict__ o, float *__restrict__ ht,
                                         int T, int H, int NT, float scale, int n, int nwg, int c0, int c1,
                                         const Gdn2Var var) {
    using C = Gdn2WalkCfg<DK, DV>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    constexpr int NTILE = DV / C::BV;
    // the column slices of one head get consecutive ids on one XCD (shared L2)
    const int L = (nwg % 8 == 0) ? (n % 8) * (nwg / 8) + n / 8 : n;
    const int vt = L % NTILE;
    const long bh = L / NTILE;
    Gdn2Head hd;
    hd.ws = ws + bh * NT * (long)Gdn2Blk<DK>::BYTES;
    hd.v = v;
    hd.w = wg;
    hd.H = H;
    hd.T = T;
    hd.row0 = (bh / H) * (long)T * H + (bh % H);
    hd.vcol0 = vt * C::BV;
    if constexpr (VAR) {  // packed sequences: bh = n H + h walks sequence n's chunks
        const int sn = (int)(bh / H), h = (int)(bh - (long)sn * H);
        const int4 sq = var.seq[sn];
        hd.ws = ws + ((long)h * var.NC + sq.z) * Gdn2Blk<DK>::BYTES;
        hd.T = sq.y;
        hd.row0 = (long)sq.x * H + h;
        c0 = 0;
        c1 = (sq.y + BT - 1) / BT;
    }
    const long sbase = bh * (long)DK * DV;

    if (wave < 2) {
        f32x4 S[C::NKB];
        const int col = hd.vcol0 + wave * 16 + r;
#pragma unroll
        for (int m = 0; m < C::NKB; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = h0 ? h0[sbase + (long)(16 * m + 4 * g + e) * DV + col] : 0.f;
        __syncthreads();
        for (int c = c0 - 1; c < c1; ++c) {
            if (c >= c0) gdn2_consume(sm, S, c & 1, o, hd, c, wave, scale, lane);
            __syncthreads();
        }
        if (ht) {
#pragma unroll
            for (int m = 0; m < C::NKB; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) ht[sbase + (long)(16 * m + 4 * g + e) * DV + col] = S[m][e];
        }
    } else if (wave < 4) {
        // loaders: iteration c stores chunk c + 1 and fetches chunk c + 2
        const int lt = tid - 128;
        Gdn2Stage<DK> R;
        if (!VAR || c0 < c1) stage_load<DK, DV>(R, hd, c0, lt);  // an empty sequence loads nothing
        __syncthreads();
        for (int c = c0 - 1; c < c1; ++c) {
            if (c + 1 < c1) {
                stage_store(sm, R, (c + 1) & 1, lt);
                if (c + 2 < c1) stage_load<DK, DV>(R, hd, c + 2, lt);
            }
            __syncthreads();
        }
    } else {
        __syncthreads();
        for (int c = c0 - 1; c < c1; ++c) __syncthreads();
    }
}

template <int DK, int DV, bool VAR>
__global__ __launch_bounds__(256, 1) void gdn2_walk_fused_kernel(const char *__restrict__ ws,
                                                                  const uint16_t *__restrict__ v,
                                                                  const uint16_t *__restrict__ wg,
                                                                  const float *__restrict__ h0, float *__restrict__ o,
                                                                  float *__restrict__ ht, int T, int H, int NT,
                                                                  int c0, int c1, float scale, Gdn2Var var) {
    static_assert(sizeof(Gdn2WalkSmem<DK, DV>) <= 160 * 1024, "LDS budget");
    __shared__ Gdn2WalkSmem<DK, DV> sm;
    walk_run<DK, DV, VAR>(sm, ws, v, wg, h0, o, ht, T, H, NT, scale, blockIdx.x, gridDim.x, c0, c1, var);
}

// One launch of the pipelined forward: workgroups below nwalk walk chunks
// wc0 .. wc1 - 1 (their blocks were prepared by an earlier launch), the rest
// prepare the blocks of chunks pc0 .. pc0 + pnc - 1 for the next launch.  The
// two parts share no memory, so no workgroup waits for another.
template <int DK, int DV>
union Gdn2PipeSmem {
    Gdn2PrepSmem<DK> prep;
    Gdn2WalkSmem<DK, DV> walk;
};

template <int DK, int DV>
__global__ __launch_bounds__(512, 1) void gdn2_pipe_kernel(const uint16_t *__restrict__ q,
                                                            const uint16_t *__restrict__ k,
                                                            const float *__restrict__ la,
                                                            const uint16_t *__restrict__ bg, char *__restrict__ ws,
                                                            const uint16_t *__restrict__ v,
                                                            const uint16_t *__restrict__ wg,
                                                            const float *__restrict__ h0, float *__restrict__ o,
                                                            float *__restrict__ ht, int T, int H, int NT, float scale,
                                                            int nwalk, int wc0, int wc1, int pc0, int pnc, int pidx) {
    static_assert(sizeof(Gdn2PipeSmem<DK, DV>) <= 160 * 1024, "LDS budget");
    __shared__ Gdn2PipeSmem<DK, DV> sm;
    const int n = blockIdx.x;
    if (n < nwalk)
        walk_run<DK, DV, false>(sm.walk, ws, v, wg, h0, o, ht, T, H, NT, scale, n, nwalk, wc0, wc1, Gdn2Var{});
    else
        prep_run<DK, false>(sm.prep, q, k, la, bg, ws, T, H, NT, pc0, pnc, pidx, n - nwalk, gridDim.x - nwalk, Gdn2Var{});
}

// ----------------------------------------------------------------- launchers
// Workspace: the per-chunk blocks, then one fp32 state [B, H, Dk, Dv] that
// carries the state between the launches of the pipelined form.
static size_t gdn2_blocks_bytes(int B, int T, int H, int Dk) {
    const size_t NT = (size_t)(T + BT - 1) / BT;
    return ((size_t)B * H * NT * gdn2_fused_block_bytes(Dk) + 255) / 256 * 256;
}

size_t gdn2_fused_ws_bytes(int B, int T, int H, int Dk, int Dv) {
    return gdn2_blocks_bytes(B, T, H, Dk) + ((size_t)B * H * Dk * Dv * sizeof(float) + 255) / 256 * 256;
}

// Number of time parts of the pipelined form: while the walk of part k runs
// on its workgroups (one per compute unit), the other compute units prepare
// the blocks of part k + 1 in the same launch.  Worth it when the walk leaves
// at least half of the compute units idle and the parts stay a few chunks long.
static int gdn2_parts(long walk_grid, int ncu, int NT) {
    return (2 * walk_grid <= ncu && NT >= 8) ? 4 : 1;
}

template <int DK, int DV>
static hipError_t launch_gdn2_fused_t(const void *q, const void *k, const float *la, const void *bg, const void *v,
                                      const void *wg, const float *h0, float *o, float *ht, void *ws, int B, int T,
                                      int H, float scale, hipStream_t st) {
    const int NT = (T + BT - 1) / BT;
    const int BH = B * H;
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu < 1) ncu = 1;
    const long walk_grid = (long)BH * (DV / Gdn2WalkCfg<DK, DV>::BV);
    const int K = gdn2_parts(walk_grid, ncu, NT);
    auto bound = [&](int p) { return (int)((long)p * NT / K); };  // first chunk of part p
    float *carry = (float *)((char *)ws + gdn2_blocks_bytes(B, T, H, DK));
    const uint16_t *q16 = (const uint16_t *)q, *k16 = (const uint16_t *)k, *b16 = (const uint16_t *)bg;
    const uint16_t *v16 = (const uint16_t *)v, *w16 = (const uint16_t *)wg;
    // part 0's blocks: a persistent prep on every compute unit (its LDS allows one per unit)
    {
        const int nc = bound(1) - bound(0);
        const long nidx = (long)BH * nc;
        const long pgrid = nidx < ncu ? nidx : ncu;
        hipLaunchKernelGGL((gdn2_prep_kernel<DK, false>), dim3((unsigned)pgrid), dim3(512), 0, st, q16, k16, la, b16,
                           (char *)ws, T, H, NT, bound(0), nc, (int)nidx, Gdn2Var{});
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // walk part p - 1 beside the prep of part p; the state crosses the
    // launches in `carry` (each workgroup reads and writes its own columns)
    for (int p = 1; p < K; ++p) {
        const int nc = bound(p + 1) - bound(p);
        const long pidx = (long)BH * nc;
        const long room = ncu - walk_grid;
        const long pgrid = pidx < room ? pidx : room;
        hipLaunchKernelGGL((gdn2_pipe_kernel<DK, DV>), dim3((unsigned)(walk_grid + pgrid)), dim3(512), 0, st, q16,
                           k16, la, b16, (char *)ws, v16, w16, p == 1 ? h0 : carry, o, carry, T, H, NT, scale,
                           (int)walk_grid, bound(p - 1), bound(p), bound(p), nc, (int)pidx);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gdn2_walk_fused_kernel<DK, DV, false>), dim3((unsigned)walk_grid), dim3(256), 0, st,
                       (const char *)ws, v16, w16, K == 1 ? h0 : carry, o, ht, T, H, NT, bound(K - 1), NT, scale,
                       Gdn2Var{});
    return hipGetLastError();
}

hipError_t launch_gdn2_fused_bf16(const void *q, const void *k, const float *la, const void *bg, const void *v,
                                  const void *wg, const float *h0, float *o, float *ht, void *ws, int B, int T,
                                  int H, int Dk, int Dv, float scale, hipStream_t st) {
    if (Dk == 64 && Dv == 64) return launch_gdn2_fused_t<64, 64>(q, k, la, bg, v, wg, h0, o, ht, ws, B, T, H, scale, st);
    if (Dk == 64 && Dv == 128) return launch_gdn2_fused_t<64, 128>(q, k, la, bg, v, wg, h0, o, ht, ws, B, T, H, scale, st);
    if (Dk == 128 && Dv == 64) return launch_gdn2_fused_t<128, 64>(q, k, la, bg, v, wg, h0, o, ht, ws, B, T, H, scale, st);
    if (Dk == 128 && Dv == 128)
        return launch_gdn2_fused_t<128, 128>(q, k, la, bg, v, wg, h0, o, ht, ws, B, T, H, scale, st);
    return hipErrorInvalidValue;
}

// ------------------------------------------------- packed sequences (varlen)
// The sequence table from the offsets, in one workgroup: sequence n holds
// tokens [s0, s1) with both offsets clamped into [0, total_T] and s1 >= s0, so
// that malformed offsets never address out of range.  Its chunk numbers start
// at the running sum of ceil(len / 64) over the earlier sequences, saturated
// at NC; a sequence whose chunks would pass NC walks only the chunks that fit.
__global__ __launch_bounds__(256) void gdn2_var_seq_kernel(const int *__restrict__ cu, int4 *__restrict__ seq, int N,
                                                           int total_T, int NC) {
    __shared__ long long part[256];
    __shared__ long long carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        int s0 = 0, len = 0;
        long long want = 0;
        if (n < N) {
            s0 = min(max(cu[n], 0), total_T);
            const int s1 = min(max(cu[n + 1], s0), total_T);
            len = s1 - s0;
            want = (len + BT - 1) / BT;
        }
        part[tid] = want;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive scan over the workgroup
            const long long add = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        const long long incl = carry + part[tid];
        if (n < N) {
            const long long cs = min(incl - want, (long long)NC), ce = min(incl, (long long)NC);
            seq[n] = make_int4(s0, (int)min((long long)len, (ce - cs) * BT), (int)cs, 0);
        }
        __syncthreads();
        if (tid == 255) carry = incl;
        __syncthreads();
    }
    if (tid == 0) seq[N] = make_int4(0, 0, (int)min(carry, (long long)NC), 0);
}

// tab[g] for g < NC: the last sequence n < N whose first chunk number is <= g
// (the numbers never decrease, so its range holds g), or N past the chunks in use.
__global__ __launch_bounds__(256) void gdn2_var_tab_kernel(const int4 *__restrict__ seq, int *__restrict__ tab, int N,
                                                           int NC) {
    const long gi = (long)blockIdx.x * 256 + threadIdx.x;
    if (gi >= NC) return;
    const int gc = (int)gi;
    int n = N;
    if (gc < seq[N].z) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seq[mid].z <= gc) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
    }
    tab[gc] = n;
}

// Workspace of the packed form: blocks [H][NC], then seq [N + 1] and tab [NC].
Gdn2VarWs gdn2_var_ws(int N, int total_T, int H, int Dk) {
    Gdn2VarWs w;
    w.NC = (long long)(total_T + BT - 1) / BT + N;
    const size_t blocks = ((size_t)H * w.NC * gdn2_fused_block_bytes(Dk) + 255) / 256 * 256;
    w.seq_off = blocks;
    w.tab_off = w.seq_off + (((size_t)N + 1) * sizeof(int4) + 255) / 256 * 256;
    w.total = w.tab_off + ((size_t)w.NC * sizeof(int) + 255) / 256 * 256;
    return w;
}

template <int DK, int DV>
static hipError_t launch_gdn2_varlen_t(const void *q, const void *k, const float *la, const void *bg, const void *v,
                                       const void *wg, const int *cu, const float *h0, float *o, float *ht, void *ws,
                                       int N, int total_T, int H, float scale, hipStream_t st) {
    const Gdn2VarWs lay = gdn2_var_ws(N, total_T, H, DK);
    const int NC = (int)lay.NC;
    int4 *seq = (int4 *)((char *)ws + lay.seq_off);
    int *tab = (int *)((char *)ws + lay.tab_off);
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu < 1) ncu = 1;
    hipLaunchKernelGGL(gdn2_var_seq_kernel, dim3(1), dim3(256), 0, st, cu, seq, N, total_T, NC);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gdn2_var_tab_kernel, dim3((unsigned)((NC + 255) / 256)), dim3(256), 0, st,
                       (const int4 *)seq, tab, N, NC);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const Gdn2Var var{seq, tab, N, NC};
    // every (head, chunk number) block, unused numbers included (they read token 0)
    const long nidx = (long)H * NC;
    const long pgrid = nidx < ncu ? nidx : ncu;
    hipLaunchKernelGGL((gdn2_prep_kernel<DK, true>), dim3((unsigned)pgrid), dim3(512), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, la, (const uint16_t *)bg, (char *)ws, total_T, H, NC, 0, NC, (int)nidx, var);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long walk_grid = (long)N * H * (DV / Gdn2WalkCfg<DK, DV>::BV);
    hipLaunchKernelGGL((gdn2_walk_fused_kernel<DK, DV, true>), dim3((unsigned)walk_grid), dim3(256), 0, st,
                       (const char *)ws, (const uint16_t *)v, (const uint16_t *)wg, h0, o, ht, total_T, H, NC, 0, 0,
                       scale, var);
    return hipGetLastError();
}

hipError_t launch_gdn2_fused_varlen_bf16(const void *q, const void *k, const float *la, const void *bg,
                                         const void *v, const void *wg, const int *cu, const float *h0, float *o,
                                         float *ht, void *ws, int N, int total_T, int H, int Dk, int Dv, float scale,
                                         hipStream_t st) {
#define GDN2_VAR(DKv, DVv)                                                                                       \
    if (Dk == DKv && Dv == DVv)                                                                                  \
    return launch_gdn2_varlen_t<DKv, DVv>(q, k, la, bg, v, wg, cu, h0, o, ht, ws, N, total_T, H, scale, st)
    GDN2_VAR(64, 64);
    GDN2_VAR(64, 128);
    GDN2_VAR(128, 64);
    GDN2_VAR(128, 128);
#undef GDN2_VAR
    return hipErrorInvalidValue;
}

}  // namespace gdn

