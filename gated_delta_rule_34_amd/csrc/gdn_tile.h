// gdn_tile.h -- pieces shared by the single-kernel chunked forwards on gfx950:
// raw 16-bit row tiles in LDS and their MFMA fragments, the hi + lo split of
// fp32 operands, the chunk-local gate scan on DPP, and the unit
// lower-triangular inverse (I + A)^-1 of one 64-token chunk.
//
// Fragment convention (as in gdn_device.h): lane l = 16 g + r of a
// 16x16x32 MFMA supplies row r of the A operand / column r of the B operand
// at k-slots 4g + e (e = 0..3) and 16 + 4g + e of a 32-wide slab; the
// accumulator holds D[4g + e][r].
#pragma once
#include "gdn_device.h"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
// 16 bytes as a native vector: arrays of it stay in registers where arrays of
// HIP's uint4 struct can be demoted to scratch
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ f32x4 mma_bf16_raw(f32x4 acc, const uint4 &a, const uint4 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16_raw(f32x4 acc, const u32x4 &a, const u32x4 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_f16_raw(f32x4 acc, const uint4 &a, const uint4 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                  0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_f16_block(f32x4 acc, const f16x4 &a, const f16x4 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
}

// The 10 lower-triangular 16x16 tiles (I >= J) of a 64x64 chunk matrix;
// compile-time so that register arrays are indexed statically.
__device__ constexpr int tileI(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__device__ constexpr int tileJ(int t) { return t - tileI(t) * (tileI(t) + 1) / 2; }

typedef __attribute__((ext_vector_type(4))) short s16x4;

// Paired-group column layout: within each 32-column slab the 4-column groups
// a and a + 4 (a = 0..3) sit side by side, so the 8 values that MFMA lane
// group g supplies for a 32-deep slab (columns 4g.. and 16 + 4g..) are 16
// contiguous bytes.  pair_col maps a logical column to its stored column
// before the row swizzle of tile_off_pg.
__device__ __forceinline__ int pair_col(int c) {
    const int a = (c >> 2) & 7;
    const int pa = (a < 4) ? 2 * a : 2 * a - 7;
    return (c & ~31) | (pa << 2) | (c & 3);
}

// Offset (in halves) of stored column `col` of row `row` in a paired-group
// tile (unpadded rows of D halves).  The 16-byte units of a row are
// XOR-swizzled by the row's low four bits.  gfx950's LDS (64 banks of 4 bytes)
// serves a 16-byte read in four passes of 16 lanes, lanes (l >> 5, parity of
// l >> 2) alike sharing a pass, and an 8-byte access in two passes of 32
// contiguous lanes (both measured with the bank-conflict counters).  The
// swizzle gives each pass of a fragment read (16 rows, one unit each) 16
// distinct units, and each pass of a transpose read (8 rows x 4 units of one
// half) or of a row store (16 rows x 2 units of one half) at most two lanes
// per bank pair, which is the least those two can have: the paired-group
// order puts all their 8-byte pieces in the same half of a unit.
template <int D>
__device__ __forceinline__ int tile_off_pg(int row, int col) {
    static_assert(D == 64 || D == 128, "head size");
    if (D == 128) return row * D + (col ^ (((row & 1) << 3) | (((row >> 3) & 1) << 4) | (((row >> 1) & 3) << 5)));
    // 128-byte rows: row parity already picks the bank half
    return row * D + (col ^ ((((row >> 1) & 1) << 3) | (((row >> 3) & 1) << 4) | (((row >> 2) & 1) << 5)));
}

// Fragment of the 32-wide slab at column k0 of rows row0 .. row0 + 15 of a
// paired-group tile: one 16-byte read per lane.
template <int D>
__device__ __forceinline__ uint4 frag_rows_pg(const uint16_t *M, int row0, int k0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    // row0 is a multiple of 16 and the swizzle reads only the low 4 row bits,
    // so the block's offset is a constant the LDS read can carry as its
    // immediate offset
    typedef __attribute__((address_space(3))) const uint16_t lds_u16;
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    lds_u16 *m3 = (lds_u16 *)M;
    const u32x4 v = *(lds_u32x4 *)(m3 + tile_off_pg<D>(r, k0 + 8 * g) + row0 * D);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// A fragment of the transpose (rows kc0 .. kc0 + 15 of M^T, slab of M rows
// j0 .. j0 + 31) read from a row-major paired-group tile with the gfx950 LDS
// transpose load: within each 16-lane group, lane j receives element (j % 4)
// of the 8-byte chunks addressed by lanes j/4, j/4 + 4, j/4 + 8, j/4 + 12.
// Lane (g, r) therefore addresses row j0 + 4g + r/4, logical columns
// kc0 + 4(r % 4) .. + 3 (one stored 4-column group), and receives
// M[j0 + 4g + e][kc0 + r], e = 0..3.  Two such loads (j0 and j0 + 16) make
// the 32-wide slab.
template <int D>
__device__ __forceinline__ uint4 frag_T_pg(const uint16_t *M, int j0, int kc0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int pc = pair_col(kc0 + 4 * (r & 3));
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    lds_u16 *m3 = (lds_u16 *)M;
    // j0 is a multiple of 16: the row block's offset is a constant (see frag_rows_pg)
    lds_u16 *p0 = m3 + tile_off_pg<D>(4 * g + (r >> 2), pc) + j0 * D;
    lds_u16 *p1 = p0 + 16 * D;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
}

// hi = round(x), lo = round(x - hi) for a pair of floats in the 16-bit type
// of V2 (bf16x2 or f16x2), on the packed round-to-nearest conversion.
template <class V2>
__device__ __forceinline__ void split_pair(V2 &h, V2 &l, float a, float b) {
    const f32x2 x = {a, b};
    h = __builtin_convertvector(x, V2);
    l = __builtin_convertvector(x - __builtin_convertvector(h, f32x2), V2);
}

// Two accumulator tiles (k-blocks 2s, 2s + 1 of a slab) as hi and lo B
// fragments whose sum carries about twice the 16-bit type's significand.
template <class V2>
__device__ __forceinline__ void hilo_frags(uint4 &hi, uint4 &lo, const f32x4 &t0, const f32x4 &t1) {
    V2 h[4], l[4];
    split_pair(h[0], l[0], t0[0], t0[1]);
    split_pair(h[1], l[1], t0[2], t0[3]);
    split_pair(h[2], l[2], t1[0], t1[1]);
    split_pair(h[3], l[3], t1[2], t1[3]);
    hi = make_uint4(__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                    __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3]));
    lo = make_uint4(__builtin_bit_cast(uint32_t, l[0]), __builtin_bit_cast(uint32_t, l[1]),
                    __builtin_bit_cast(uint32_t, l[2]), __builtin_bit_cast(uint32_t, l[3]));
}

// Value of `x` moved by a DPP row operation; lanes without a source get 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xf,
                                                                 false));
}

// Value of `x` from another lane of the same quad (a DPP quad permutation,
// where every lane has a source, so no old value is needed and the move can
// fold into the instruction that uses it).
template <int CTRL>
__device__ __forceinline__ float quad_perm_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// 4 x 4 transpose within each quad of lanes (DPP quad permutations): lane
// 4a + b holds v[e] = M[e][b] of its quad's 4 x 4 block on entry and
// M[b][e] on return.  Used to turn an MFMA accumulator tile (4 rows of one
// column per lane) into 4 adjacent columns of one row per lane.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 v, int lane) {
    const int b = lane & 3;
    f32x4 p;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = quad_perm_f32<0xB1>(v[e]);  // from lane b ^ 1
    if (b & 1) v = f32x4{p[1], v[1], p[3], v[3]};
    else v = f32x4{v[0], p[0], v[2], p[2]};
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = quad_perm_f32<0x4E>(v[e]);  // from lane b ^ 2
    if (b & 2) v = f32x4{p[2], p[3], v[2], v[3]};
    else v = f32x4{v[0], v[1], p[0], p[1]};
    return v;
}

// log2(e) * chunk-local inclusive cumsum of g, one token per lane: an fp32
// wave scan on DPP (shifts 1, 2, 4, 8 within each row of 16 lanes, then the
// row totals broadcast by lane 15 and lane 31), no LDS round trip.
__device__ __forceinline__ float chunk_g2(float gv) {
    float x = gv * 1.4426950408889634f;
    x += dpp_f32<0x111, 0xf>(x);  // row_shr:1
    x += dpp_f32<0x112, 0xf>(x);  // row_shr:2
    x += dpp_f32<0x114, 0xf>(x);  // row_shr:4
    x += dpp_f32<0x118, 0xf>(x);  // row_shr:8
    x += dpp_f32<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_f32<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Four rows of one column of a 16x16 fp16 block by the gfx950 LDS transpose
// load: lane (g, r) receives M[row0 + 4g + e][col0 + r], e = 0..3 (row
// stride LDP halves, a multiple of 4; col0 a multiple of 4).
template <int LDP>
__device__ __forceinline__ f16x4 col4_tr(const _Float16 *M, int row0, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    typedef __attribute__((ext_vector_type(4))) short s16x4_t;
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)&M[(row0 + 4 * g + (r >> 2)) * LDP + col0 + 4 * (r & 3)]);
    return __builtin_bit_cast(f16x4, v);
}

// Four entries of one row of a 16x16 fp16 block: lane (g, r) receives
// M[row0 + r][col0 + 4g + e], e = 0..3 (an A operand, or the B operand of a
// product formed transposed).
template <int LDP>
__device__ __forceinline__ f16x4 row4(const _Float16 *M, int row0, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    return *(const f16x4 *)&M[(row0 + r) * LDP + col0 + 4 * g];
}

// A fragment of T - I (zero diagonal) turned into T: entry e of lane (g, r)
// sits on the diagonal when 4g + e == r, for a column read and a row read.
__device__ __forceinline__ f16x4 plus_eye(f16x4 v, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (4 * g + e == r) v[e] = (_Float16)1.f;
    return v;
}

__device__ __forceinline__ void split_hl(f16x4 &h, f16x4 &l, const f32x4 &x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (_Float16)x[e];
        l[e] = (_Float16)(x[e] - (float)h[e]);
    }
}

__device__ __forceinline__ f16x8 cat8(const f16x4 &a, const f16x4 &b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// T - I for T = (I + A)^-1 of one chunk, A strictly lower (fp16, row stride
// LDP, the strict-lower part of every 16x16 block filled, other entries of
// the lower tiles zero); one wave.  Tm receives the lower tiles of T - I;
// its upper 16x16 tiles and the upper-right 8x8 quadrant of each diagonal
// block must be zero on entry (they are read as zero and never written).
// For a block-lower matrix L = [L11 0; L21 L22], L^-1 has the diagonal
// blocks L11^-1, L22^-1 and the off-diagonal block -L22^-1 L21 L11^-1, so
// the inverse doubles its block size level by level:
//  8 x 8:   lane (block b, column c) solves its column by forward
//           substitution, x_i = [i == c] - sum_{j<i} A_ij x_j;
//  16 x 16: the lower-left 8x8 quadrant of each diagonal block,
//           -T22 A21 T11, four blocks side by side on MFMA;
//  32 x 32: blocks (1,0) and (3,2), -T_II A_IJ T_JJ;
//  64 x 64: blocks (2..3, 0..1): Z = A_[23][01] T_[01][01] on 32-deep MFMA,
//           then -T_[23][23] Z.
// Each product W = A T is exact (fp16 operands from LDS, fp32 sums); the
// outer product -T W takes W as fp16 hi + lo parts (~22 bits) and is
// formed transposed, (W^T T^T)^T, so that a lane holds 4 adjacent entries
// of a row of the result and stores them at once.  Quadrants of Tm left by
// an earlier chunk are masked where an operand would read them.
template <int LDP>
__device__ __forceinline__ void unit_lower_inverse(const _Float16 *A, _Float16 *Tm, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const bool ll_col = g >= 2 && r < 8, ll_row = r >= 8 && g < 2;
    const f16x4 z4 = {};
    // Every read of A is issued first: the levels below then wait only on
    // their own reads of Tm, one LDS round trip per level.
    const int b8 = lane >> 3, cc = lane & 7;
    const _Float16 *Ab = &A[8 * b8 * LDP + 8 * b8];
    f16x4 a8[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a8[i][0] = (i > 0) ? *(const f16x4 *)&Ab[i * LDP] : z4;
        a8[i][1] = (i > 4) ? *(const f16x4 *)&Ab[i * LDP + 4] : z4;
    }
    f16x4 a16[4], a32[2], a64[2][2];
#pragma unroll
    for (int B = 0; B < 4; ++B) a16[B] = row4<LDP>(A, 16 * B, 16 * B, lane);
#pragma unroll
    for (int p = 0; p < 2; ++p) a32[p] = row4<LDP>(A, 16 * (2 * p + 1), 32 * p, lane);
#pragma unroll
    for (int K = 0; K < 2; ++K)
#pragma unroll
        for (int L = 0; L < 2; ++L) a64[K][L] = row4<LDP>(A, 16 * (K + 2), 16 * L, lane);
    __builtin_amdgcn_sched_barrier(0);
    // 8 x 8
    {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) {
                const float a = (float)a8[i][j >> 2][j & 3];
                if (j & 1) s1 = fmaf(a, x[j], s1);
                else s0 = fmaf(a, x[j], s0);
            }
            x[i] = ((i == cc) ? 1.f : 0.f) - (s0 + s1);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) Tm[(8 * b8 + i) * LDP + 8 * b8 + cc] = (_Float16)(x[i] - (i == cc ? 1.f : 0.f));
    }
    __builtin_amdgcn_sched_barrier(0);
    // 16 x 16: W = A21 T11 as the 16x16 product Atilde T8 (Atilde: A's
    // lower-left quadrant of the block, T8: the two 8x8 inverses), then
    // the quadrant -T8 W.  D-layout entry (4g + e, r) is in the lower-left
    // quadrant when g >= 2 and r < 8; row entry (r, 4g + e) when r >= 8 and
    // g < 2.
    {
        f16x4 tc[4], tr[4];
#pragma unroll
        for (int B = 0; B < 4; ++B) {
            tc[B] = col4_tr<LDP>(Tm, 16 * B, 16 * B, lane);
            tr[B] = row4<LDP>(Tm, 16 * B, 16 * B, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 W[4];
#pragma unroll
        for (int B = 0; B < 4; ++B)
            W[B] = mma_f16_block(zero4(), ll_row ? a16[B] : z4, plus_eye(ll_col ? z4 : tc[B], lane));
#pragma unroll
        for (int B = 0; B < 4; ++B) {
            const f16x4 t8 = plus_eye(ll_row ? z4 : tr[B], lane);
            f16x4 wh, wl;
            split_hl(wh, wl, W[B]);
            const f32x4 res = mma_f16_block(mma_f16_block(zero4(), wh, t8), wl, t8);
            if (ll_row) *(f16x4 *)&Tm[(16 * B + r) * LDP + 16 * B + 4 * g] = -__builtin_convertvector(res, f16x4);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 32 x 32: blocks (1,0) and (3,2)
    {
        f16x4 tc[2], tr[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            tc[p] = col4_tr<LDP>(Tm, 32 * p, 32 * p, lane);
            tr[p] = row4<LDP>(Tm, 32 * p + 16, 32 * p + 16, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 W[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) W[p] = mma_f16_block(zero4(), a32[p], plus_eye(tc[p], lane));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const f16x4 ti = plus_eye(tr[p], lane);
            f16x4 wh, wl;
            split_hl(wh, wl, W[p]);
            const f32x4 res = mma_f16_block(mma_f16_block(zero4(), wh, ti), wl, ti);
            *(f16x4 *)&Tm[(32 * p + 16 + r) * LDP + 32 * p + 4 * g] = -__builtin_convertvector(res, f16x4);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 64 x 64: Z_KJ = A_K0 T_0J + A_K1 T_1J (K = 2, 3; J = 0, 1; T_01 is an
    // upper tile, zero), then block (I, J) = -(T_I2 Z_2J + T_I3 Z_3J)
    {
        f16x4 tc[2][2], tr[2][2];
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int L = 0; L < 2; ++L) tc[J][L] = col4_tr<LDP>(Tm, 16 * L, 16 * J, lane);
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int K = 0; K < 2; ++K) tr[I][K] = row4<LDP>(Tm, 16 * (I + 2), 16 * (K + 2), lane);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 Z[2][2];
#pragma unroll
        for (int J = 0; J < 2; ++J) {
            const f16x8 b = cat8(J == 0 ? plus_eye(tc[J][0], lane) : tc[J][0], J == 1 ? plus_eye(tc[J][1], lane) : tc[J][1]);
#pragma unroll
            for (int K = 0; K < 2; ++K)
                Z[K][J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat8(a64[K][0], a64[K][1]), b, zero4(), 0, 0, 0);
        }
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            const f16x8 bt = cat8(I == 0 ? plus_eye(tr[I][0], lane) : tr[I][0], I == 1 ? plus_eye(tr[I][1], lane) : tr[I][1]);
#pragma unroll
            for (int J = 0; J < 2; ++J) {
                f16x4 h2, l2, h3, l3;
                split_hl(h2, l2, Z[0][J]);
                split_hl(h3, l3, Z[1][J]);
                f32x4 res = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat8(h2, h3), bt, zero4(), 0, 0, 0);
                res = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat8(l2, l3), bt, res, 0, 0, 0);
                *(f16x4 *)&Tm[(16 * (I + 2) + r) * LDP + 16 * J + 4 * g] = -__builtin_convertvector(res, f16x4);
            }
        }
    }
}

}  // namespace gdn
