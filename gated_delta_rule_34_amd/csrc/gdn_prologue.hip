// gdn_prologue.hip -- the elementwise work around the rule, fused into one
// pass each side (GatedDeltaNet walkthrough, the data-flow overview and the
// sections on the short convolution and the gates):
//   prologue: q, k, v = SiLU(causal depthwise 4-tap convolution of their
//             projections), q and k L2-normalised per head, the decay
//             g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b);
//             q, k, v are written in bf16, the input type of the rule
//   epilogue: y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z) per head (bf16)
// The convolution has no bias and its last tap multiplies the current
// token; its 3-token history comes from the previous tokens or, before the
// first token, from the caller's convolution state (zeros when absent).
// Both kernels are HBM-bound.  The prologue gives each lane 8 consecutive
// channels (one 16-byte load per token) over a block of TB tokens, so the
// 4-tap window slides through registers and every input row is read once per
// block; the L2 norm of a head (Dk / 8 lanes) is summed with DPP row
// permutes.  SiLU runs on the hardware exp2 and reciprocal (about 1 ulp each,
// far below the bf16 rounding of the outputs); the fp32 gates use the
// accurate library functions.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_tile.h"

namespace gdn {

constexpr int kProTB = 8;  // tokens per wave in the prologue

__device__ __forceinline__ float silu_fast(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * LOG2E));
}

// Two fp32 values as a bf16 pair (round to nearest even), first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ void unpack8(float (&x)[8], uint4 p) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

// Sum over aligned groups of N lanes (N = 8 or 16) on DPP: swap neighbours,
// swap pairs, mirror within 8, mirror within 16.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_f32<0xB1, 0xf>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_f32<0x4E, 0xf>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_f32<0x141, 0xf>(x);  // row_half_mirror
    if (N == 16) x += dpp_f32<0x140, 0xf>(x);  // row_mirror
    return x;
}

// Grid: x = groups of 4 token blocks (one block of TB tokens per wave),
// y = groups of 64 channel octets over q, k, v (in that order).
template <int DK, int DV, int TB>
__global__ __launch_bounds__(256) void prologue_kernel(
    const uint16_t *__restrict__ xq, const uint16_t *__restrict__ xk, const uint16_t *__restrict__ xv,
    const float *__restrict__ a, const float *__restrict__ b, const float *__restrict__ wq,
    const float *__restrict__ wk, const float *__restrict__ wv, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, const float *state_in, uint16_t *__restrict__ q,
    uint16_t *__restrict__ k, uint16_t *__restrict__ v, float *__restrict__ g, float *__restrict__ beta,
    float *state_out, int B, int T, int H) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // workgroup n runs on XCD n % 8: give each XCD a contiguous range of tokens
    // so the rows shared by neighbouring blocks stay in one L2
    const int nx = gridDim.x, bx = blockIdx.x;
    const int lx = (nx % 8 == 0) ? (bx % 8) * (nx / 8) + bx / 8 : bx;
    const int NTB = (T + TB - 1) / TB;
    const int gtb = lx * 4 + wave;
    if (gtb >= B * NTB) return;
    const int bb = gtb / NTB, t0 = (gtb - bb * NTB) * TB;
    const long rowbase = (long)bb * T;

    if (blockIdx.y == 0) {  // gates of this block's tokens, one (token, head) per lane
        for (int it = lane; it < TB * H; it += 64) {
            const int tt = it / H, h = it - tt * H, t = t0 + tt;
            if (t < T) {
                const long row = (rowbase + t) * H + h;
                const float z = a[row] + dt_bias[h];
                const float sp = z > 20.f ? z : log1pf(expf(z));  // softplus
                g[row] = -expf(A_log[h]) * sp;
                beta[row] = 1.f / (1.f + expf(-b[row]));
            }
        }
    }

    constexpr int DK8 = DK / 8, DV8 = DV / 8;
    const int Q8 = H * DK8, C8 = 2 * Q8 + H * DV8, Ctot = 8 * C8;
    const int oct = blockIdx.y * 64 + lane;
    const bool live = oct < C8;
    const uint16_t *x = xv;
    uint16_t *out = v;
    const float *w = wv;
    int L = H * DV, j = 0, coff = 2 * H * DK;
    bool norm = false;
    if (oct < Q8) {
        x = xq; out = q; w = wq; L = H * DK; j = oct; coff = 0; norm = true;
    } else if (oct < 2 * Q8) {
        x = xk; out = k; w = wk; L = H * DK; j = oct - Q8; coff = H * DK; norm = true;
    } else if (live) {
        j = oct - 2 * Q8;
    }
    float wt[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float4 f = *(const float4 *)(w + (long)(j * 8 + c) * 4);
        wt[c][0] = f.x; wt[c][1] = f.y; wt[c][2] = f.z; wt[c][3] = f.w;
    }
    // the rows of tokens t0 - 3 .. t0 + TB - 1, clamped into [0, T - 1]; rows
    // outside the sequence are replaced below or feed no stored output
    uint4 raw[TB + 3];
#pragma unroll
    for (int i = 0; i < TB + 3; ++i) {
        const int uc = min(max(t0 - 3 + i, 0), T - 1);
        raw[i] = *(const uint4 *)(x + (rowbase + uc) * L + j * 8);
    }
    float hist[3][8];
#pragma unroll
    for (int i = 0; i < 3; ++i) unpack8(hist[i], raw[i]);
    if (t0 == 0) {  // before the first token: the carried state, or zeros
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (state_in) {
                const float *sp = state_in + ((long)bb * 3 + i) * Ctot + coff + j * 8;
                const float4 s0 = *(const float4 *)sp, s1 = *(const float4 *)(sp + 4);
                hist[i][0] = s0.x; hist[i][1] = s0.y; hist[i][2] = s0.z; hist[i][3] = s0.w;
                hist[i][4] = s1.x; hist[i][5] = s1.y; hist[i][6] = s1.z; hist[i][7] = s1.w;
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) hist[i][c] = 0.f;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
        float cur[8], y[8];
        unpack8(cur, raw[i + 3]);
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float acc = wt[c][0] * hist[0][c];
            acc = fmaf(wt[c][1], hist[1][c], acc);
            acc = fmaf(wt[c][2], hist[2][c], acc);
            acc = fmaf(wt[c][3], cur[c], acc);
            y[c] = silu_fast(acc);
            ss = fmaf(y[c], y[c], ss);
        }
        ss = group_sum<DK8>(ss);
        const float sc = norm ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.f;
        const int t = t0 + i;
        if (live && t < T) {
            uint4 o;
            o.x = pack_bf16x2(y[0] * sc, y[1] * sc);
            o.y = pack_bf16x2(y[2] * sc, y[3] * sc);
            o.z = pack_bf16x2(y[4] * sc, y[5] * sc);
            o.w = pack_bf16x2(y[6] * sc, y[7] * sc);
            *(uint4 *)(out + (rowbase + t) * L + j * 8) = o;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            hist[0][c] = hist[1][c];
            hist[1][c] = hist[2][c];
            hist[2][c] = cur[c];
        }
        // after the last token the window is the new convolution state (rows
        // T - 3 .. T - 1, cached values where those are negative); written
        // here when it does not replace state_in, else by conv_state_kernel
        if (state_out && t == T - 1 && live) {
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                float *sp = state_out + ((long)bb * 3 + r) * Ctot + coff + j * 8;  // 4-byte aligned
#pragma unroll
                for (int c = 0; c < 8; ++c) sp[c] = hist[r][c];
            }
        }
    }
}

// The convolution state after the last token: row j (0..2) holds the input
// of token T - 3 + j, taken from the previous state (or zero) when
// T - 3 + j < 0.  One thread per (batch entry, channel) reads its three
// values before writing any, so the new state may overwrite the old in place.
template <int DK, int DV>
__global__ __launch_bounds__(256) void conv_state_kernel(const uint16_t *__restrict__ xq,
                                                         const uint16_t *__restrict__ xk,
                                                         const uint16_t *__restrict__ xv, const float *state_in,
                                                         float *state_out, int B, int T, int H) {
    const int Ctot = H * (2 * DK + DV);
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;  // (b, channel)
    if (idx >= (long)B * Ctot) return;
    const int c = (int)(idx % Ctot);
    const long bb = idx / Ctot;
    const uint16_t *x;
    int D, cc;
    if (c < H * DK) {
        x = xq; D = DK; cc = c;
    } else if (c < 2 * H * DK) {
        x = xk; D = DK; cc = c - H * DK;
    } else {
        x = xv; D = DV; cc = c - 2 * H * DK;
    }
    const int h = cc / D, d = cc % D;
    float val[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int u = T - 3 + j;
        val[j] = 0.f;
        if (u >= 0)
            val[j] = bf16_to_f32(x[((bb * T + u) * H + h) * (long)D + d]);
        else if (state_in)
            val[j] = state_in[(bb * 3 + 3 + u) * (long)Ctot + c];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) state_out[(bb * 3 + j) * (long)Ctot + c] = val[j];
}

// One row of DV channels per DV / 8 lanes, 8 channels per lane.
template <int DV>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const float *__restrict__ o, const uint16_t *__restrict__ z,
                                                            const float *__restrict__ w, uint16_t *__restrict__ y,
                                                            long rows, float eps) {
    constexpr int LPR = DV / 8;
    const long gl = (long)blockIdx.x * 256 + threadIdx.x;
    const long row = gl / LPR;
    const int c = (int)(gl % LPR) * 8;
    const bool live = row < rows;
    const long base = (live ? row : rows - 1) * DV + c;  // dead lanes read the last row
    const float4 o0 = *(const float4 *)(o + base), o1 = *(const float4 *)(o + base + 4);
    const uint4 zr = *(const uint4 *)(z + base);
    const float4 w0 = *(const float4 *)(w + c), w1 = *(const float4 *)(w + c + 4);
    const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float zv[8];
    unpack8(zv, zr);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(ov[e], ov[e], ss);
    ss = group_sum<LPR>(ss);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = ov[e] * inv * wv[e] * silu_fast(zv[e]);
    if (live) {
        uint4 p;
        p.x = pack_bf16x2(r[0], r[1]);
        p.y = pack_bf16x2(r[2], r[3]);
        p.z = pack_bf16x2(r[4], r[5]);
        p.w = pack_bf16x2(r[6], r[7]);
        *(uint4 *)(y + base) = p;
    }
}

hipError_t launch_prologue(const void *xq, const void *xk, const void *xv, const float *a, const float *b,
                           const float *wq, const float *wk, const float *wv, const float *A_log,
                           const float *dt_bias, const float *state_in, void *q, void *k, void *v, float *g,
                           float *beta, float *state_out, int B, int T, int H, int Dk, int Dv, hipStream_t st) {
    const long nblk = (long)B * ((T + kProTB - 1) / kProTB);
    const dim3 grid((unsigned)((nblk + 3) / 4), (unsigned)((H * (2 * Dk + Dv) / 8 + 63) / 64));
    // A new state that does not replace the old one is written by the
    // prologue kernel itself; in place (state_out == state_in) the blocks
    // that read the old state could run after the one that writes the new
    // state, so conv_state_kernel writes it after the prologue.
    const bool fused_state = state_out && state_out != state_in;
#define GDN_PRO(DKv, DVv)                                                                                        \
    if (Dk == DKv && Dv == DVv) {                                                                                \
        hipLaunchKernelGGL((prologue_kernel<DKv, DVv, kProTB>), grid, dim3(256), 0, st, (const uint16_t *)xq,     \
                           (const uint16_t *)xk, (const uint16_t *)xv, a, b, wq, wk, wv, A_log, dt_bias, state_in, \
                           (uint16_t *)q, (uint16_t *)k, (uint16_t *)v, g, beta, fused_state ? state_out : nullptr, \
                           B, T, H);                                                                               \
        hipError_t e = hipGetLastError();                                                                         \
        if (e != hipSuccess || !state_out || fused_state) return e;                                              \
        const long n = (long)B * H * (2 * DKv + DVv);                                                             \
        hipLaunchKernelGGL((conv_state_kernel<DKv, DVv>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,    \
                           (const uint16_t *)xq, (const uint16_t *)xk, (const uint16_t *)xv, state_in, state_out, \
                           B, T, H);                                                                              \
        return hipGetLastError();                                                                                 \
    }
    GDN_PRO(64, 64)
    GDN_PRO(64, 128)
    GDN_PRO(128, 64)
    GDN_PRO(128, 128)
#undef GDN_PRO
    return hipErrorInvalidValue;
}

hipError_t launch_gated_rmsnorm(const float *o, const void *z, const float *w, void *y, long rows, int Dv, float eps,
                                hipStream_t st) {
    const unsigned grid = (unsigned)((rows * (Dv / 8) + 255) / 256);
    if (Dv == 64)
        hipLaunchKernelGGL((gated_rmsnorm_kernel<64>), dim3(grid), dim3(256), 0, st, o, (const uint16_t *)z, w,
                           (uint16_t *)y, rows, eps);
    else if (Dv == 128)
        hipLaunchKernelGGL((gated_rmsnorm_kernel<128>), dim3(grid), dim3(256), 0, st, o, (const uint16_t *)z, w,
                           (uint16_t *)y, rows, eps);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
