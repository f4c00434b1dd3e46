// gdn_step.hip -- single-token Gated DeltaNet decode step, state in place.
//
// Per head:  S <- exp(g) S;  u = beta (v - S^T k);  S <- S + k u^T;
//            o = scale S^T q
// (GatedDeltaNet walkthrough, yfxerp.com, "Delta Rule" section: the
// per-token reference loop).  The d_v columns of S are independent given
// k, beta and g, so each thread owns one column: it reads its Dk state
// values once into registers (rows of S are contiguous across the threads
// of a wave, so every load instruction reads whole 256-byte row segments),
// forms the prediction S^T k, applies the update and the read-out, and
// writes the column back.  The step moves the state through HBM exactly
// once each way, which is the whole cost: the kernel is HBM-bound.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <class Pol, int DK, int DV>
__global__ __launch_bounds__(64) void step_kernel(const typename Pol::in_t *__restrict__ q,
                                                  const typename Pol::in_t *__restrict__ k,
                                                  const typename Pol::in_t *__restrict__ v,
                                                  const float *__restrict__ g,
                                                  const float *__restrict__ beta, float *__restrict__ S,
                                                  float *__restrict__ o, float scale) {
    constexpr int NCB = DV / 64;  // 64-column blocks per head
    __shared__ float sq[DK], sk[DK];
    const long unit = blockIdx.x / NCB;  // (b, h)
    const int col = (blockIdx.x % NCB) * 64 + threadIdx.x;
    for (int i = threadIdx.x; i < DK; i += 64) {
        sq[i] = load_elem(q + unit * DK + i);
        sk[i] = load_elem(k + unit * DK + i);
    }
    __syncthreads();
    const float decay = expf(g[unit]);
    const float bt = beta[unit];
    float *Sc = S + unit * (long)DK * DV + col;
    float s[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) s[i] = Sc[(long)i * DV];
    float pred = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
        s[i] *= decay;
        pred = fmaf(s[i], sk[i], pred);
    }
    const float uu = bt * (load_elem(v + unit * DV + col) - pred);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
        s[i] = fmaf(sk[i], uu, s[i]);
        acc = fmaf(s[i], sq[i], acc);
        Sc[(long)i * DV] = s[i];
    }
    o[unit * DV + col] = scale * acc;
}

// One Gated DeltaNet-2 decode token (Gated DeltaNet-2 article, "Regla-2 del
// Delta cerrado", one step of the recurrence): rows of S decay by their own
// channel rate, S <- Diag(alpha) S; u = w . v - S^T (b . k); S <- S + k u^T;
// o = scale S^T q.  Same layout as step_kernel: one thread per value column,
// the column's Dk state values in registers.
template <class Pol, int DK, int DV>
__global__ __launch_bounds__(64) void step2_kernel(const typename Pol::in_t *__restrict__ q,
                                                   const typename Pol::in_t *__restrict__ k,
                                                   const typename Pol::in_t *__restrict__ v,
                                                   const float *__restrict__ la,
                                                   const typename Pol::in_t *__restrict__ bg,
                                                   const typename Pol::in_t *__restrict__ wg, float *__restrict__ S,
                                                   float *__restrict__ o, float scale) {
    constexpr int NCB = DV / 64;  // 64-column blocks per head
    __shared__ float sq[DK], sk[DK], se[DK], sa[DK];
    const long unit = blockIdx.x / NCB;  // (b, h)
    const int col = (blockIdx.x % NCB) * 64 + threadIdx.x;
    for (int i = threadIdx.x; i < DK; i += 64) {
        const float kk = load_elem(k + unit * DK + i);
        sq[i] = load_elem(q + unit * DK + i);
        sk[i] = kk;
        se[i] = load_elem(bg + unit * DK + i) * kk;
        sa[i] = expf(la[unit * DK + i]);
    }
    __syncthreads();
    float *Sc = S + unit * (long)DK * DV + col;
    float s[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) s[i] = Sc[(long)i * DV];
    float pred = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
        s[i] *= sa[i];
        pred = fmaf(s[i], se[i], pred);
    }
    const float uu = load_elem(wg + unit * DV + col) * load_elem(v + unit * DV + col) - pred;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
        s[i] = fmaf(sk[i], uu, s[i]);
        acc = fmaf(s[i], sq[i], acc);
        Sc[(long)i * DV] = s[i];
    }
    o[unit * DV + col] = scale * acc;
}

template <class Pol, int DK, int DV>
static hipError_t launch_step_t(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                float *S, float *o, int B, int H, float scale, hipStream_t st) {
    using in_t = typename Pol::in_t;
    const long grid = (long)B * H * (DV / 64);
    hipLaunchKernelGGL((step_kernel<Pol, DK, DV>), dim3((unsigned)grid), dim3(64), 0, st, (const in_t *)q,
                       (const in_t *)k, (const in_t *)v, g, beta, S, o, scale);
    return hipGetLastError();
}

hipError_t launch_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                       float *S, float *o, int B, int H, int Dk, int Dv, bool bf16, float scale,
                       hipStream_t st) {
#define GDN_STEP(P, DKv, DVv) \
    if (Dk == DKv && Dv == DVv) return launch_step_t<P, DKv, DVv>(q, k, v, g, beta, S, o, B, H, scale, st)
    if (bf16) {
        GDN_STEP(PolBF16, 64, 64);
        GDN_STEP(PolBF16, 64, 128);
        GDN_STEP(PolBF16, 128, 64);
        GDN_STEP(PolBF16, 128, 128);
    } else {
        GDN_STEP(PolF32, 64, 64);
        GDN_STEP(PolF32, 64, 128);
        GDN_STEP(PolF32, 128, 64);
        GDN_STEP(PolF32, 128, 128);
    }
#undef GDN_STEP
    return hipErrorInvalidValue;
}

template <class Pol, int DK, int DV>
static hipError_t launch_step2_t(const void *q, const void *k, const void *v, const float *la, const void *bg,
                                 const void *wg, float *S, float *o, int B, int H, float scale, hipStream_t st) {
    using in_t = typename Pol::in_t;
    const long grid = (long)B * H * (DV / 64);
    hipLaunchKernelGGL((step2_kernel<Pol, DK, DV>), dim3((unsigned)grid), dim3(64), 0, st, (const in_t *)q,
                       (const in_t *)k, (const in_t *)v, la, (const in_t *)bg, (const in_t *)wg, S, o, scale);
    return hipGetLastError();
}

hipError_t launch_step2(const void *q, const void *k, const void *v, const float *la, const void *bg,
                        const void *wg, float *S, float *o, int B, int H, int Dk, int Dv, bool bf16, float scale,
                        hipStream_t st) {
#define GDN_STEP2(P, DKv, DVv) \
    if (Dk == DKv && Dv == DVv) return launch_step2_t<P, DKv, DVv>(q, k, v, la, bg, wg, S, o, B, H, scale, st)
    if (bf16) {
        GDN_STEP2(PolBF16, 64, 64);
        GDN_STEP2(PolBF16, 64, 128);
        GDN_STEP2(PolBF16, 128, 64);
        GDN_STEP2(PolBF16, 128, 128);
    } else {
        GDN_STEP2(PolF32, 64, 64);
        GDN_STEP2(PolF32, 64, 128);
        GDN_STEP2(PolF32, 128, 64);
        GDN_STEP2(PolF32, 128, 128);
    }
#undef GDN_STEP2
    return hipErrorInvalidValue;
}

}  // namespace gdn
