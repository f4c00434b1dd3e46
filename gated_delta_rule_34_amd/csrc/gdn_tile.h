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

__device__ __forceinline__ f32x4 mma_bf16_raw(f32x4 acc, const uint4 &a, const uint4 &b) {
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

// A 64 x D tile of raw 16-bit values in LDS.  With D = 128 a row is 64
// dwords (every row starts on bank 0), so column groups are XOR-swizzled
// per row: 16-half segments by (row & 7), 8-half groups by bit 3 of the row.
// The 8-byte fragment reads (16 rows x 2 column groups per half-wave) and
// the transpose reads (8 rows x one 16-half segment) then each cover 64
// distinct banks.  With D = 64 rows are padded instead.
template <int D>
struct RowTile {
    static constexpr bool SWZ = D == 128;
    static constexpr int LD = SWZ ? D : D + 8;  // row stride in halves
};

// Offset (in halves) of column `col` (a multiple of 4) of row `row`.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
    if (RowTile<D>::SWZ) return row * RowTile<D>::LD + (col ^ (((row & 7) << 4) ^ (((row >> 3) & 1) << 3)));
    return row * RowTile<D>::LD + col;
}

// A/B fragment of the 32-wide slab at column k0 of rows row0 .. row0 + 15.
template <int D>
__device__ __forceinline__ uint4 frag_rows_sw(const uint16_t *M, int row0, int k0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const uint2 lo = *(const uint2 *)&M[tile_off<D>(row0 + r, k0 + 4 * g)];
    const uint2 hi = *(const uint2 *)&M[tile_off<D>(row0 + r, k0 + 16 + 4 * g)];
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

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
// tile (unpadded rows of D halves).  The 8-column units are XOR-swizzled by
// row so that both the 16-byte fragment reads (16 rows, one 8-column unit
// each) and the 8-byte transpose reads (4 rows x 4 alternate 4-column
// groups) touch 64 distinct banks (64 banks of 4 bytes).
template <int D>
__device__ __forceinline__ int tile_off_pg(int row, int col) {
    static_assert(D == 64 || D == 128, "head size");
    if (D == 128) return row * D + (col ^ (((row & 3) << 5) | (((row >> 2) & 3) << 3)));
    return row * D + (col ^ ((((row >> 1) & 1) << 5) | (((row >> 2) & 3) << 3)));
}

// Fragment of the 32-wide slab at column k0 of rows row0 .. row0 + 15 of a
// paired-group tile: one 16-byte read per lane.
template <int D>
__device__ __forceinline__ uint4 frag_rows_pg(const uint16_t *M, int row0, int k0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    return *(const uint4 *)&M[tile_off_pg<D>(row0 + r, k0 + 8 * g)];
}

// A fragment of the transpose (rows kc0 .. kc0 + 15 of M^T, slab of M rows
// j0 .. j0 + 31) read from the row-major tile with the gfx950 LDS transpose
// load: within each 16-lane group, lane j receives element (j % 4) of the
// 8-byte chunks addressed by lanes j/4, j/4 + 4, j/4 + 8, j/4 + 12.  Lane
// (g, r) therefore addresses row j0 + 4g + r/4, columns kc0 + 4(r % 4), and
// receives M[j0 + 4g + e][kc0 + r], e = 0..3.  Two such loads (j0 and
// j0 + 16) make the 32-wide slab.
template <int D>
__device__ __forceinline__ uint4 frag_T_sw(const uint16_t *M, int j0, int kc0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint16_t *p0 = &M[tile_off<D>(j0 + 4 * g + (r >> 2), kc0 + 4 * (r & 3))];
    const uint16_t *p1 = &M[tile_off<D>(j0 + 16 + 4 * g + (r >> 2), kc0 + 4 * (r & 3))];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
}

// frag_T_sw for a paired-group tile (logical columns kc0 + 4(r % 4) .. + 3
// are one stored 4-column group).
template <int D>
__device__ __forceinline__ uint4 frag_T_pg(const uint16_t *M, int j0, int kc0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int pc = pair_col(kc0 + 4 * (r & 3));
    const uint16_t *p0 = &M[tile_off_pg<D>(j0 + 4 * g + (r >> 2), pc)];
    const uint16_t *p1 = &M[tile_off_pg<D>(j0 + 16 + 4 * g + (r >> 2), pc)];
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

// T - I for T = (I + A)^-1 of one chunk, A strictly lower (fp16, row stride
// LDP, the strict-lower part of every 16x16 block filled, other entries of
// the lower tiles zero); one wave.  Tm receives the lower tiles of T - I.
//  Diagonal blocks: lane (block bb, column cc) solves its column of T_bb,
//    x_i = [i == cc] - sum_{j<i} A_ij x_j, with four partial sums per row.
//  Off-diagonal blocks, one sub-diagonal level d at a time (the blocks of a
//    level are independent and are computed together):
//    T_IJ = -T_II M,  M = A_IJ + sum_{K=J}^{I-1} A_IK (T - I)_KJ,
//    with column pieces read by transpose loads and T_IJ formed as
//    (M^T T_II^T)^T so each lane stores 4 adjacent entries of a row.
template <int LDP>
__device__ __forceinline__ void unit_lower_inverse(const _Float16 *A, _Float16 *Tm, int lane) {
    const int r = lane & 15, g = lane >> 4;
    {
        const int bb = lane >> 4, cc = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const _Float16 *arow = &A[(16 * bb + i) * LDP + 16 * bb];
            f16x4 av[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                if (4 * q4 < i) av[q4] = *(const f16x4 *)&arow[4 * q4];
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < i; ++j) part[j & 3] = fmaf((float)av[j >> 2][j & 3], x[j], part[j & 3]);
            x[i] = ((i == cc) ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Tm[(16 * bb + i) * LDP + 16 * bb + cc] = (_Float16)(x[i] - (i == cc ? 1.f : 0.f));
    }
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        f32x4 M[3];
#pragma unroll
        for (int J = 0; J < 4 - d; ++J) {
            const int I = J + d;
            // M starts as A_IJ: lane (g, r) holds A[16I + 4g + e][16J + r]
            const f16x4 aij = col4_tr<LDP>(A, 16 * I, 16 * J, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) M[J][e] = (float)aij[e];
#pragma unroll
            for (int K = J; K < I; ++K) {
                const f16x4 a = *(const f16x4 *)&A[(16 * I + r) * LDP + 16 * K + 4 * g];
                M[J] = mma_f16_block(M[J], a, col4_tr<LDP>(Tm, 16 * K, 16 * J, lane));
            }
        }
        // T_IJ = -T_II M, formed transposed as M^T T_II^T so that this lane
        // holds row 16I + r, columns 16J + 4g .. + 3 and stores them at once
#pragma unroll
        for (int J = 0; J < 4 - d; ++J) {
            const int I = J + d;
            f16x4 tb = *(const f16x4 *)&Tm[(16 * I + r) * LDP + 16 * I + 4 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * g + e == r) tb[e] = (_Float16)1.f;  // T_II = I + strict(T_II)
            // M enters as fp16 hi + lo parts, so T_II M keeps ~22 bits of M
            f16x4 mh, ml;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mh[e] = (_Float16)M[J][e];
                ml[e] = (_Float16)(M[J][e] - (float)mh[e]);
            }
            const f32x4 res = mma_f16_block(mma_f16_block(zero4(), mh, tb), ml, tb);
            f16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (_Float16)(-res[e]);
            *(f16x4 *)&Tm[(16 * I + r) * LDP + 16 * J + 4 * g] = out;
        }
    }
}

}  // namespace gdn
