// gdn_device.h -- device helpers shared by the gfx950 kernels: element
// types, numeric policies, and MFMA tile products with one fragment layout.
//
// Fragment convention (wave64, 16x16 output tiles).  For a product
// D[16x16] += A[16xK] * B[Kx16], lane l (g = l / 16, r = l % 16) supplies
//     A[r][k] and B[k][r] for k in its "k-slots",
// and receives D[4g + e][r], e = 0..3 (the MFMA accumulator layout).
// A 16-wide k-block gives lane l the slots k = 4g + e (e = 0..3); a 32-wide
// slab is two such blocks, slots k = 4g + e and 16 + 4g + e (frag8 element
// e and e + 4).  Because the sum over k does not depend on which lane
// carries which k, the same per-lane data feeds
//   * v_mfma_f32_16x16x32_f16  (one instruction per 32-wide slab), and
//   * v_mfma_f32_16x16x4_f32   (one instruction per element, e = 0..7),
// so the fp32 path and the fp16 path share every kernel.  The accumulator
// tile of one product, read as "rows 4g + e, column r", is exactly the B
// fragment of a 16-wide k-block of the next product: chained products
// (state -> K*S -> new values -> state update) stay in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

constexpr float LOG2E = 1.4426950408889634f;
constexpr int BT = 64;  // chunk length

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

__device__ __forceinline__ float load_elem(const float *p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t *p) { return bf16_to_f32(*p); }

// Eight consecutive inputs as fp32 (bf16 bits or fp32), from 16-byte aligned memory.
__device__ __forceinline__ void load8(float (&x)[8], const uint16_t *p) {
    const uint4 u = *(const uint4 *)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(float (&x)[8], const float *p) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Columns c0 .. c0 + D - 1 of rows t0 .. t0 + 63 of a [B, T, H, DFULL] tensor
// (head h of batch b) into LDS as type M with row stride LD; rows past T are
// zero.  Loads go out in groups of four per thread before their stores; rows
// past T read the last token (in bounds) and are then zeroed.  64 x D must be
// a multiple of 8 * NTHR.
template <int D, int LD, int NTHR, class M, class In>
__device__ __forceinline__ void stage_rows(M *dst, const In *src, long b, int h, int t0, int T, int H, int c0,
                                           int DFULL, int tid) {
    constexpr int U = BT * D / 8 / NTHR;
    static_assert(U * 8 * NTHR == BT * D, "staging layout");
    constexpr int GRP = U < 4 ? U : 4;
#pragma unroll
    for (int u0 = 0; u0 < U; u0 += GRP) {
        float x[GRP][8];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            const int idx = tid + NTHR * (u0 + u), row = idx / (D / 8), c8 = 8 * (idx % (D / 8));
            const int t = min(t0 + row, T - 1);
            load8(x[u], src + ((b * T + t) * H + h) * (long)DFULL + c0 + c8);
        }
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            const int idx = tid + NTHR * (u0 + u), row = idx / (D / 8), c8 = 8 * (idx % (D / 8));
            const bool in = t0 + row < T;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[row * LD + c8 + e] = (M)(in ? x[u][e] : 0.f);
        }
    }
}

// Numeric policies.  `in_t` is the storage type of q, k, v (and GDN-2 b, w);
// `mt` is the MFMA operand type used for products whose operands are not
// exact inputs (state, new values, decayed keys, the attention-like matrix).
struct PolF32 {
    using in_t = float;
    using mt = float;
};
struct PolBF16 {
    using in_t = uint16_t;  // bf16 bits
    using mt = _Float16;    // 11-bit significand; bf16 inputs in [2^-14, 65504] convert exactly
};
// bf16 inputs with fp32 operands everywhere (the backward's recompute of the
// forward, whose entry states must carry fp32 accuracy)
struct PolBF16F32 {
    using in_t = uint16_t;
    using mt = float;
};

template <class T> __device__ __forceinline__ T to_mt(float x);
template <> __device__ __forceinline__ float to_mt<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 to_mt<_Float16>(float x) { return (_Float16)x; }

// D += A * B over one 32-wide k slab, operands given per lane as 8 values.
__device__ __forceinline__ f32x4 mma_slab(f32x4 acc, const float (&a)[8], const float (&b)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 mma_slab(f32x4 acc, const _Float16 (&a)[8], const _Float16 (&b)[8]) {
    f16x8 va, vb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        va[e] = a[e];
        vb[e] = b[e];
    }
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(va, vb, acc, 0, 0, 0);
}

// D += A * B over one 16-wide k block, always in fp32 (used by the
// triangular inverse, whose operands are intermediate fp32 values).
__device__ __forceinline__ f32x4 mma_block_f32(f32x4 acc, const float (&a)[4], const float (&b)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    return acc;
}

// A/B fragment of a 32-wide slab from a row-major LDS matrix M[row][k]:
// lane supplies M[row0 + r][k0 + slot].
template <class T>
__device__ __forceinline__ void frag_rows(T (&f)[8], const T *M, int ld, int row0, int k0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const T *p = M + (row0 + r) * ld + k0 + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = p[e];
        f[e + 4] = p[16 + e];
    }
}

// Same for one 16-wide k block, fp32.
__device__ __forceinline__ void frag_rows4(float (&f)[4], const float *M, int ld, int row0, int k0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float *p = M + (row0 + r) * ld + k0 + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = p[e];
}

// B fragment of a 16-wide k block from a row-major LDS matrix M[k][col]:
// lane supplies M[k0 + 4g + e][col0 + r].
__device__ __forceinline__ void frag_cols4(float (&f)[4], const float *M, int ld, int k0, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = M[(k0 + 4 * g + e) * ld + col0 + r];
}

// B fragment of a 32-wide slab built from two accumulator tiles (k-blocks
// 2s and 2s+1) held in registers, converted to the operand type.
template <class T>
__device__ __forceinline__ void frag_from_acc(T (&f)[8], const f32x4 &lo, const f32x4 &hi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = to_mt<T>(lo[e]);
        f[e + 4] = to_mt<T>(hi[e]);
    }
}

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

}  // namespace gdn
