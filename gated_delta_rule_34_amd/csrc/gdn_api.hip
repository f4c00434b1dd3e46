// gdn_api.hip -- the C ABI declared in include/gdn.h: argument validation,
// workspace layout and kernel sequencing on the caller's stream.  No device
// memory is allocated here; every buffer belongs to the caller.
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

constexpr int kBT = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(gdn_dtype dt) { return dt == GDN_F32 || dt == GDN_BF16; }
size_t esize(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

struct Range {
    const void *p;
    size_t n;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Workspace of the chunked forward: G2 [B,H,NT,64] fp32, then (T - I)
// [B,H,NT,64,64] fp32, each section 256-byte aligned.
struct ChunkWs {
    size_t g2_off, t_off, total;
};

ChunkWs chunk_ws(int B, int T, int H) {
    const size_t NT = (size_t)(T + kBT - 1) / kBT;
    const size_t chunks = (size_t)B * H * NT;
    ChunkWs w;
    w.g2_off = 0;
    w.t_off = align_up(chunks * kBT * sizeof(float));
    w.total = w.t_off + align_up(chunks * kBT * kBT * sizeof(float));
    return w;
}

bool sizes_ok(int B, int T, int H) {
    if (B < 1 || T < 1 || H < 1) return false;
    const long long NT = (T + kBT - 1) / kBT;
    return (long long)B * H * NT < (1LL << 31);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Chunk-parallel plan for the bf16 forward of a dense batch (gdn_fused.hip,
// SegArgs).  The single kernel runs (Dv / 32) workgroups per head, one per
// compute unit, each walking every chunk in order; when that fills less than
// half of the 256 compute units, each sequence is cut into NS segments of L
// chunks.  The walk launch runs 2 NS - 3 workgroup sets per head (one for
// segment 0's end state, two per middle segment), so NS is the largest count
// for which they fit the compute units in one round; the single kernel then
// runs the NS segments of every head together.  NS = 0: no plan.
struct SegPlan {
    int NS, L;
};

constexpr int kPlanCUs = 256;  // compute units of the MI355X

SegPlan seg_plan(int B, int T, int H, int Dk, int Dv) {
    SegPlan p{0, 0};
    if (Dk != Dv) return p;
    const long sets = (long)B * H * (Dv / 32);   // workgroups of the single kernel
    if (sets * 2 > kPlanCUs) return p;
    const int NT = (T + kBT - 1) / kBT;
    int ns = (int)((kPlanCUs / sets + 3) / 2);
    if (ns > 16) ns = 16;
    for (; ns >= 3; --ns) {
        const int L = (NT + ns - 1) / ns;
        if (L >= 8 && (ns - 1) * L < NT) {
            p = SegPlan{ns, L};
            return p;
        }
    }
    return p;
}

// Workspace of the plan: Hin, Hout, M [B NS, H, D, D] fp32, then the B NS + 1
// segment offsets (int32); each section 256-byte aligned.
struct SegWs {
    size_t hin, hout, m, cu, total;
};

SegWs seg_ws(int B, int H, int D, const SegPlan &p) {
    const size_t st = align_up((size_t)B * p.NS * H * D * D * sizeof(float));
    SegWs w;
    w.hin = 0;
    w.hout = st;
    w.m = 2 * st;
    w.cu = 3 * st;
    w.total = w.cu + align_up(((size_t)B * p.NS + 1) * sizeof(int));
    return w;
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported head size or dtype";
        case GDN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case GDN_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

// bf16 inputs take the single-kernel path, which needs no workspace; fp32
// inputs take the two-stage path (intra-chunk stage, then the state walk).
size_t gdn_chunk_fwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype) {
    if (!sizes_ok(B, T, H) || !head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return 0;
    if (dtype == GDN_BF16) {
        const SegPlan p = seg_plan(B, T, H, Dk, Dv);
        return p.NS ? seg_ws(B, H, Dk, p).total : kAlign;
    }
    return chunk_ws(B, T, H).total;
}

gdn_status gdn_chunk_intra(const void *k, const float *g, const float *beta, float *G2, float *Tinv, int B,
                           int T, int H, int Dk, gdn_dtype dtype, void *stream) {
    if (!k || !g || !beta || !G2 || !Tinv) return GDN_ERR_INVALID_ARG;
    if (!sizes_ok(B, T, H)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    return from_hip(gdn::launch_intra(k, g, beta, G2, Tinv, B, T, H, Dk, dtype == GDN_BF16,
                                      (hipStream_t)stream));
}

gdn_status gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const float *h0, float *o, float *ht, int B, int T, int H, int Dk, int Dv,
                         gdn_dtype dtype, float scale, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !g || !beta || !o) return GDN_ERR_INVALID_ARG;
    if (!sizes_ok(B, T, H)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)B * H * Dk * Dv * sizeof(float);
    const Range rq{q, ntok * Dk * es}, rk{k, ntok * Dk * es}, rv{v, ntok * Dv * es};
    const Range rg{g, ntok * 4}, rb{beta, ntok * 4}, rh0{h0, h0 ? nstate : 0};
    const Range ro{o, ntok * Dv * 4}, rht{ht, ht ? nstate : 0};
    const bool fused = dtype == GDN_BF16;
    // the fused kernel moves q, k, v rows and output rows in 16-byte pieces
    if (fused && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)))
        return GDN_ERR_INVALID_ARG;
    const ChunkWs lay = chunk_ws(B, T, H);
    // bf16: the chunk-parallel scan when planned and the workspace holds it
    const SegPlan plan = fused ? seg_plan(B, T, H, Dk, Dv) : SegPlan{0, 0};
    const SegWs slay = plan.NS ? seg_ws(B, H, Dk, plan) : SegWs{0, 0, 0, 0, 0};
    const size_t seg_bytes = slay.total;
    const bool seg = plan.NS && ws && aligned(ws, kAlign) && ws_bytes >= seg_bytes;
    const Range rws{fused ? (seg ? ws : nullptr) : ws, fused ? seg_bytes : lay.total};
    // Outputs may not overlap inputs, each other or the workspace; ht may be exactly h0.
    for (Range in : {rq, rk, rv, rg, rb, rh0, rws})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    if (ht) {
        if (overlap(rht, rh0) && ht != h0) return GDN_ERR_INVALID_ARG;
        for (Range in : {rq, rk, rv, rg, rb, ro, rws})
            if (overlap(rht, in)) return GDN_ERR_INVALID_ARG;
    }
    hipStream_t st = (hipStream_t)stream;
    if (seg) {
        for (Range in : {rq, rk, rv, rg, rb, rh0})
            if (overlap(rws, in)) return GDN_ERR_INVALID_ARG;
        char *base = (char *)ws;
        return from_hip(gdn::launch_fused_seg_bf16(q, k, v, g, beta, h0, o, ht, B, T, H, Dk, scale, plan.NS, plan.L,
                                                   (float *)(base + slay.hin), (float *)(base + slay.hout),
                                                   (float *)(base + slay.m), (int *)(base + slay.cu), st));
    }
    if (fused)
        return from_hip(gdn::launch_fused_bf16(q, k, v, g, beta, h0, o, ht, nullptr, B, T, H, Dk, Dv, scale, st));
    if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < lay.total) return GDN_ERR_WORKSPACE;
    for (Range in : {rq, rk, rv, rg, rb, rh0})
        if (overlap(rws, in)) return GDN_ERR_INVALID_ARG;

    float *G2 = (float *)((char *)ws + lay.g2_off);
    float *Tinv = (float *)((char *)ws + lay.t_off);
    gdn_status s = from_hip(gdn::launch_intra(k, g, beta, G2, Tinv, B, T, H, Dk, dtype == GDN_BF16, st));
    if (s != GDN_OK) return s;
    return from_hip(gdn::launch_walk(q, k, v, beta, G2, Tinv, h0, o, ht, nullptr, B, T, H, Dk, Dv, dtype == GDN_BF16,
                                     scale, st));
}

gdn_status gdn_chunk_walk(const void *q, const void *k, const void *v, const float *beta, const float *G2,
                          const float *Tinv, const float *h0, float *o, float *ht, int B, int T, int H, int Dk,
                          int Dv, gdn_dtype dtype, float scale, void *stream) {
    if (!q || !k || !v || !beta || !G2 || !Tinv || !o) return GDN_ERR_INVALID_ARG;
    if (!sizes_ok(B, T, H)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)B * H * Dk * Dv * sizeof(float);
    const size_t nchunk = (size_t)B * H * ((T + kBT - 1) / kBT);
    const Range rq{q, ntok * Dk * es}, rk{k, ntok * Dk * es}, rv{v, ntok * Dv * es}, rb{beta, ntok * 4};
    const Range rg2{G2, nchunk * kBT * 4}, rt{Tinv, nchunk * kBT * kBT * 4}, rh0{h0, h0 ? nstate : 0};
    const Range ro{o, ntok * Dv * 4}, rht{ht, ht ? nstate : 0};
    for (Range in : {rq, rk, rv, rb, rg2, rt, rh0})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    if (ht) {
        if (overlap(rht, rh0) && ht != h0) return GDN_ERR_INVALID_ARG;
        for (Range in : {rq, rk, rv, rb, rg2, rt, ro})
            if (overlap(rht, in)) return GDN_ERR_INVALID_ARG;
    }
    return from_hip(gdn::launch_walk(q, k, v, beta, G2, Tinv, h0, o, ht, nullptr, B, T, H, Dk, Dv, dtype == GDN_BF16,
                                     scale, (hipStream_t)stream));
}

// Workspace of the GDN-2 forward, per chunk of each head: Ehat, Qhat, Khat
// [64, Dk] in the MFMA operand type (fp16 for bf16 inputs, else fp32),
// Gamma_C [Dk], T - I and strict P [64, 64], diag P [64], all fp32; each
// array 256-byte aligned.
struct Gdn2Ws {
    size_t e_off, q_off, k_off, gam_off, t_off, p_off, d_off, total;
};

static Gdn2Ws gdn2_ws(int B, int T, int H, int Dk, int Dv, gdn_dtype dt) {
    const size_t NT = (size_t)(T + kBT - 1) / kBT;
    const size_t chunks = (size_t)B * H * NT;
    const size_t mts = dt == GDN_BF16 ? 2 : 4;
    Gdn2Ws w;
    size_t off = 0;
    if (dt == GDN_BF16) {  // per-chunk blocks of prepared operands and a state carry (gdn2_fused.hip)
        w = Gdn2Ws{};
        w.total = align_up(gdn::gdn2_fused_ws_bytes(B, T, H, Dk, Dv));
        return w;
    }
    w.e_off = off; off += align_up(chunks * kBT * Dk * mts);
    w.q_off = off; off += align_up(chunks * kBT * Dk * mts);
    w.k_off = off; off += align_up(chunks * kBT * Dk * mts);
    w.gam_off = off; off += align_up(chunks * Dk * 4);
    w.t_off = off; off += align_up(chunks * kBT * kBT * 4);
    w.p_off = off; off += align_up(chunks * kBT * kBT * 4);
    w.d_off = off; off += align_up(chunks * kBT * 4);
    w.total = off;
    return w;
}

size_t gdn2_chunk_fwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype) {
    if (!sizes_ok(B, T, H) || !head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return 0;
    return gdn2_ws(B, T, H, Dk, Dv, dtype).total;
}

gdn_status gdn2_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha, const void *b,
                          const void *w, const float *h0, float *o, float *ht, int B, int T, int H, int Dk,
                          int Dv, gdn_dtype dtype, float scale, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !log_alpha || !b || !w || !o) return GDN_ERR_INVALID_ARG;
    if (!sizes_ok(B, T, H)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    // the bf16 kernels move q, k, v, b, w rows and output rows in 16-byte pieces
    if (dtype == GDN_BF16 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(b, 16) ||
                              !aligned(w, 16) || !aligned(o, 16)))
        return GDN_ERR_INVALID_ARG;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)B * H * Dk * Dv * sizeof(float);
    const Gdn2Ws lay = gdn2_ws(B, T, H, Dk, Dv, dtype);
    const Range rq{q, ntok * Dk * es}, rk{k, ntok * Dk * es}, rv{v, ntok * Dv * es};
    const Range rla{log_alpha, ntok * Dk * 4}, rb{b, ntok * Dk * es}, rw{w, ntok * Dv * es};
    const Range rh0{h0, h0 ? nstate : 0}, ro{o, ntok * Dv * 4}, rht{ht, ht ? nstate : 0}, rws{ws, lay.total};
    for (Range in : {rq, rk, rv, rla, rb, rw, rh0, rws})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    if (ht) {
        if (overlap(rht, rh0) && ht != h0) return GDN_ERR_INVALID_ARG;
        for (Range in : {rq, rk, rv, rla, rb, rw, ro, rws})
            if (overlap(rht, in)) return GDN_ERR_INVALID_ARG;
    }
    if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < lay.total) return GDN_ERR_WORKSPACE;
    for (Range in : {rq, rk, rv, rla, rb, rw, rh0})
        if (overlap(rws, in)) return GDN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GDN_BF16)
        return from_hip(gdn::launch_gdn2_fused_bf16(q, k, log_alpha, b, v, w, h0, o, ht, ws, B, T, H, Dk, Dv, scale, st));
    char *base = (char *)ws;
    void *E = base + lay.e_off, *Qh = base + lay.q_off, *Kh = base + lay.k_off;
    float *Gam = (float *)(base + lay.gam_off), *Tinv = (float *)(base + lay.t_off);
    float *P = (float *)(base + lay.p_off), *D = (float *)(base + lay.d_off);
    const bool bf = dtype == GDN_BF16;
    gdn_status s = from_hip(gdn::launch_gdn2_intra(q, k, log_alpha, b, E, Qh, Kh, Gam, Tinv, P, D, B, T, H, Dk, bf, st));
    if (s != GDN_OK) return s;
    return from_hip(gdn::launch_gdn2_walk(E, Qh, Kh, Gam, Tinv, P, D, v, w, h0, o, ht, B, T, H, Dk, Dv, bf, scale, st));
}

// Packed sequences for GDN-2: sizes the chunk numbering can hold (every
// prep index h NC + g and every walk workgroup id fits in 32 bits).
static bool var2_sizes_ok(int N, int total_T, int H, int Dv) {
    if (N < 1 || total_T < 1 || H < 1) return false;
    const long long NC = ((long long)total_T + kBT - 1) / kBT + N;
    return (long long)H * NC < (1LL << 31) && (long long)N * H * (Dv / 32 > 0 ? Dv / 32 : 1) < (1LL << 31);
}

size_t gdn2_chunk_fwd_varlen_workspace(int N, int total_T, int H, int Dk, int Dv, gdn_dtype dtype) {
    if (!var2_sizes_ok(N, total_T, H, Dv) || !head_ok(Dk) || !head_ok(Dv) || dtype != GDN_BF16) return 0;
    return gdn::gdn2_var_ws(N, total_T, H, Dk).total;
}

gdn_status gdn2_chunk_fwd_varlen(const void *q, const void *k, const void *v, const float *log_alpha, const void *b,
                                 const void *w, const int *cu_seqlens, const float *h0, float *o, float *ht, int N,
                                 int total_T, int H, int Dk, int Dv, gdn_dtype dtype, float scale, void *ws,
                                 size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !log_alpha || !b || !w || !cu_seqlens || !o) return GDN_ERR_INVALID_ARG;
    if (!var2_sizes_ok(N, total_T, H, Dv)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    if (dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(b, 16) || !aligned(w, 16) ||
        !aligned(o, 16))
        return GDN_ERR_INVALID_ARG;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)total_T * H;
    const size_t nstate = (size_t)N * H * Dk * Dv * sizeof(float);
    const gdn::Gdn2VarWs lay = gdn::gdn2_var_ws(N, total_T, H, Dk);
    const Range rq{q, ntok * Dk * es}, rk{k, ntok * Dk * es}, rv{v, ntok * Dv * es};
    const Range rla{log_alpha, ntok * Dk * 4}, rb{b, ntok * Dk * es}, rw{w, ntok * Dv * es};
    const Range rcu{cu_seqlens, (size_t)(N + 1) * sizeof(int)}, rh0{h0, h0 ? nstate : 0};
    const Range ro{o, ntok * Dv * 4}, rht{ht, ht ? nstate : 0}, rws{ws, lay.total};
    for (Range in : {rq, rk, rv, rla, rb, rw, rcu, rh0, rws})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    if (ht) {
        if (overlap(rht, rh0) && ht != h0) return GDN_ERR_INVALID_ARG;
        for (Range in : {rq, rk, rv, rla, rb, rw, rcu, ro, rws})
            if (overlap(rht, in)) return GDN_ERR_INVALID_ARG;
    }
    if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < lay.total) return GDN_ERR_WORKSPACE;
    for (Range in : {rq, rk, rv, rla, rb, rw, rcu, rh0})
        if (overlap(rws, in)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_gdn2_fused_varlen_bf16(q, k, log_alpha, b, v, w, cu_seqlens, h0, o, ht, ws, N,
                                                       total_T, H, Dk, Dv, scale, (hipStream_t)stream));
}

gdn_status gdn_recurrent_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                              float *S, float *o, int B, int H, int Dk, int Dv, gdn_dtype dtype, float scale,
                              void *stream) {
    if (!q || !k || !v || !g || !beta || !S || !o) return GDN_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || (long long)B * H * (Dv / 64 > 0 ? Dv / 64 : 1) >= (1LL << 31))
        return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    const size_t nh = (size_t)B * H;
    const Range rS{S, nh * Dk * Dv * 4}, ro{o, nh * Dv * 4};
    const Range rq{q, nh * Dk * es}, rk{k, nh * Dk * es}, rv{v, nh * Dv * es}, rg{g, nh * 4}, rb{beta, nh * 4};
    for (Range in : {rq, rk, rv, rg, rb, ro})
        if (overlap(rS, in)) return GDN_ERR_INVALID_ARG;
    for (Range in : {rq, rk, rv, rg, rb})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_step(q, k, v, g, beta, S, o, B, H, Dk, Dv, dtype == GDN_BF16, scale,
                                     (hipStream_t)stream));
}

gdn_status gdn2_recurrent_step(const void *q, const void *k, const void *v, const float *log_alpha, const void *b,
                               const void *w, float *S, float *o, int B, int H, int Dk, int Dv, gdn_dtype dtype,
                               float scale, void *stream) {
    if (!q || !k || !v || !log_alpha || !b || !w || !S || !o) return GDN_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || (long long)B * H * (Dv / 64 > 0 ? Dv / 64 : 1) >= (1LL << 31))
        return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    const size_t nh = (size_t)B * H;
    const Range rS{S, nh * Dk * Dv * 4}, ro{o, nh * Dv * 4};
    const Range rq{q, nh * Dk * es}, rk{k, nh * Dk * es}, rv{v, nh * Dv * es};
    const Range rla{log_alpha, nh * Dk * 4}, rb{b, nh * Dk * es}, rw{w, nh * Dv * es};
    for (Range in : {rq, rk, rv, rla, rb, rw, ro})
        if (overlap(rS, in)) return GDN_ERR_INVALID_ARG;
    for (Range in : {rq, rk, rv, rla, rb, rw})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_step2(q, k, v, log_alpha, b, w, S, o, B, H, Dk, Dv, dtype == GDN_BF16, scale,
                                      (hipStream_t)stream));
}

gdn_status gdn_chunk_fwd_varlen(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                const int *cu_seqlens, const float *h0, float *o, float *ht, int N, int total_T,
                                int H, int Dk, int Dv, gdn_dtype dtype, float scale, void *stream) {
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return GDN_ERR_INVALID_ARG;
    if (N < 1 || total_T < 1 || H < 1 || (long long)N * H * (Dv / 32 > 0 ? Dv / 32 : 1) >= (1LL << 31))
        return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    if (dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GDN_ERR_INVALID_ARG;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)total_T * H;
    const size_t nstate = (size_t)N * H * Dk * Dv * sizeof(float);
    const Range rq{q, ntok * Dk * es}, rk{k, ntok * Dk * es}, rv{v, ntok * Dv * es}, rg{g, ntok * 4},
        rb{beta, ntok * 4}, rcu{cu_seqlens, (size_t)(N + 1) * sizeof(int)}, rh0{h0, h0 ? nstate : 0},
        ro{o, ntok * Dv * 4}, rht{ht, ht ? nstate : 0};
    for (Range in : {rq, rk, rv, rg, rb, rcu, rh0})
        if (overlap(ro, in)) return GDN_ERR_INVALID_ARG;
    if (ht) {
        if (overlap(rht, rh0) && ht != h0) return GDN_ERR_INVALID_ARG;
        for (Range in : {rq, rk, rv, rg, rb, rcu, ro})
            if (overlap(rht, in)) return GDN_ERR_INVALID_ARG;
    }
    return from_hip(gdn::launch_fused_bf16(q, k, v, g, beta, h0, o, ht, cu_seqlens, N, total_T, H, Dk, Dv, scale,
                                           (hipStream_t)stream));
}

// Workspace of the backward: the forward's intra stage (G2, T - I), then the
// entry state and the leaving-state gradient of every chunk, fp32
// [B, H, NT, Dk, Dv] each.
struct BwdWs {
    size_t ck_off, dck_off, g2d_off, total;
};

static BwdWs bwd_ws(int B, int T, int H, int Dk, int Dv) {
    const size_t NT = (size_t)(T + kBT - 1) / kBT;
    const size_t st = align_up((size_t)B * H * NT * Dk * Dv * sizeof(float));
    BwdWs w;
    w.ck_off = chunk_ws(B, T, H).total;
    w.dck_off = w.ck_off + st;
    w.g2d_off = w.dck_off + st;  // fp64 gate sums [B, H, NT, 64]
    w.total = w.g2d_off + align_up((size_t)B * H * NT * kBT * sizeof(double));
    return w;
}

size_t gdn_chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype) {
    if (!sizes_ok(B, T, H) || !head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return 0;
    return bwd_ws(B, T, H, Dk, Dv).total;
}

gdn_status gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const float *h0, const float *dO, const float *dht, float *dq, float *dk, float *dv,
                         float *dg, float *dbeta, float *dh0, int B, int T, int H, int Dk, int Dv, gdn_dtype dtype,
                         float scale, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta) return GDN_ERR_INVALID_ARG;
    if (!sizes_ok(B, T, H)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    // the bf16 recompute walk reads q, k, v rows in 16-byte pieces
    if (dtype == GDN_BF16 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))) return GDN_ERR_INVALID_ARG;
    const BwdWs lay = bwd_ws(B, T, H, Dk, Dv);
    if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < lay.total) return GDN_ERR_WORKSPACE;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)B * H * Dk * Dv * sizeof(float);
    const Range ins[] = {{q, ntok * Dk * es}, {k, ntok * Dk * es}, {v, ntok * Dv * es}, {g, ntok * 4},
                         {beta, ntok * 4}, {h0, h0 ? nstate : 0}, {dO, ntok * Dv * 4}, {dht, dht ? nstate : 0}};
    const Range outs[] = {{dq, ntok * Dk * 4}, {dk, ntok * Dk * 4}, {dv, ntok * Dv * 4}, {dg, ntok * 4},
                          {dbeta, ntok * 4}, {dh0, dh0 ? nstate : 0}, {ws, lay.total}};
    const int nouts = sizeof(outs) / sizeof(outs[0]);
    for (int a = 0; a < nouts; ++a) {
        for (Range in : ins)
            if (overlap(outs[a], in)) return GDN_ERR_INVALID_ARG;
        for (int c = a + 1; c < nouts; ++c)
            if (overlap(outs[a], outs[c])) return GDN_ERR_INVALID_ARG;
    }
    hipStream_t st = (hipStream_t)stream;
    const ChunkWs cw = chunk_ws(B, T, H);
    char *base = (char *)ws;
    float *G2 = (float *)(base + cw.g2_off), *Tinv = (float *)(base + cw.t_off);
    float *Sck = (float *)(base + lay.ck_off), *dSck = (float *)(base + lay.dck_off);
    const bool bf = dtype == GDN_BF16;
    double *G2d = (double *)(base + lay.g2d_off);
    gdn_status s = from_hip(gdn::launch_intra(k, g, beta, G2, Tinv, B, T, H, Dk, bf, st, true, G2d));
    if (s != GDN_OK) return s;
    // entry state of every chunk: for bf16 inputs the fused forward's walk
    // (bf16 hi + lo state products, T - I and the residuals as fp16 hi + lo),
    // else the staged fp32 walk
    if (bf)
        s = from_hip(gdn::launch_fused_states_bf16(q, k, v, g, beta, Tinv, h0, Sck, B, T, H, Dk, Dv, st));
    else
        s = from_hip(
            gdn::launch_walk(q, k, v, beta, G2, Tinv, h0, nullptr, nullptr, Sck, B, T, H, Dk, Dv, bf, scale, st, true));
    if (s != GDN_OK) return s;
    return from_hip(gdn::launch_bwd(q, k, v, beta, dO, dht, G2d, Tinv, Sck, dSck, dq, dk, dv, dg, dbeta, dh0, B, T, H,
                                    Dk, Dv, bf, scale, st));
}

// Workspace of the GDN-2 backward, fp32 sections each 256-byte aligned:
// Ehat, Qhat, Khat [B,H,NT,64,Dk]; Gamma_C [B,H,NT,Dk]; T - I, P
// [B,H,NT,64,64]; diag(P) [B,H,NT,64]; chunk entry states and leaving-state
// gradients [B,H,NT,Dk,Dv].
struct Bwd2Ws {
    size_t e_off, q_off, k_off, gam_off, t_off, p_off, d_off, ck_off, dck_off, total;
};

static Bwd2Ws bwd2_ws(int B, int T, int H, int Dk, int Dv) {
    const size_t chunks = (size_t)B * H * ((T + kBT - 1) / kBT);
    Bwd2Ws w;
    size_t off = 0;
    w.e_off = off; off += align_up(chunks * kBT * Dk * 4);
    w.q_off = off; off += align_up(chunks * kBT * Dk * 4);
    w.k_off = off; off += align_up(chunks * kBT * Dk * 4);
    w.gam_off = off; off += align_up(chunks * Dk * 4);
    w.t_off = off; off += align_up(chunks * kBT * kBT * 4);
    w.p_off = off; off += align_up(chunks * kBT * kBT * 4);
    w.d_off = off; off += align_up(chunks * kBT * 4);
    w.ck_off = off; off += align_up(chunks * (size_t)Dk * Dv * 4);
    w.dck_off = off; off += align_up(chunks * (size_t)Dk * Dv * 4);
    w.total = off;
    return w;
}

size_t gdn2_chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype) {
    if (!sizes_ok(B, T, H) || !head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return 0;
    return bwd2_ws(B, T, H, Dk, Dv).total;
}

gdn_status gdn2_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha, const void *b,
                          const void *w, const float *h0, const float *dO, const float *dht, float *dq, float *dk,
                          float *dv, float *dlog_alpha, float *db, float *dw, float *dh0, int B, int T, int H, int Dk,
                          int Dv, gdn_dtype dtype, float scale, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv || !dlog_alpha || !db || !dw)
        return GDN_ERR_INVALID_ARG;
    if (!sizes_ok(B, T, H)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    // the bf16 path moves q, k, b, log_alpha, v and w rows in 16-byte pieces
    if (dtype == GDN_BF16 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(b, 16) ||
                              !aligned(w, 16) || !aligned(log_alpha, 16)))
        return GDN_ERR_INVALID_ARG;
    const Bwd2Ws lay = bwd2_ws(B, T, H, Dk, Dv);
    if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < lay.total) return GDN_ERR_WORKSPACE;
    const size_t es = esize(dtype);
    const size_t ntok = (size_t)B * T * H;
    const size_t nstate = (size_t)B * H * Dk * Dv * sizeof(float);
    const Range ins[] = {{q, ntok * Dk * es}, {k, ntok * Dk * es}, {v, ntok * Dv * es}, {log_alpha, ntok * Dk * 4},
                         {b, ntok * Dk * es}, {w, ntok * Dv * es}, {h0, h0 ? nstate : 0}, {dO, ntok * Dv * 4},
                         {dht, dht ? nstate : 0}};
    const Range outs[] = {{dq, ntok * Dk * 4}, {dk, ntok * Dk * 4}, {dv, ntok * Dv * 4}, {dlog_alpha, ntok * Dk * 4},
                          {db, ntok * Dk * 4}, {dw, ntok * Dv * 4}, {dh0, dh0 ? nstate : 0}, {ws, lay.total}};
    const int nouts = sizeof(outs) / sizeof(outs[0]);
    for (int a = 0; a < nouts; ++a) {
        for (Range in : ins)
            if (overlap(outs[a], in)) return GDN_ERR_INVALID_ARG;
        for (int c = a + 1; c < nouts; ++c)
            if (overlap(outs[a], outs[c])) return GDN_ERR_INVALID_ARG;
    }
    hipStream_t st = (hipStream_t)stream;
    char *base = (char *)ws;
    float *Eh = (float *)(base + lay.e_off), *Qh = (float *)(base + lay.q_off), *Kh = (float *)(base + lay.k_off);
    float *Gam = (float *)(base + lay.gam_off), *Tm = (float *)(base + lay.t_off), *P = (float *)(base + lay.p_off);
    float *D = (float *)(base + lay.d_off), *Sck = (float *)(base + lay.ck_off), *dSck = (float *)(base + lay.dck_off);
    const bool bf = dtype == GDN_BF16;
    gdn_status s = from_hip(gdn::launch_gdn2_recompute(q, k, log_alpha, b, v, w, h0, Eh, Qh, Kh, Gam, Tm, P, D, Sck,
                                                       B, T, H, Dk, Dv, bf, st));
    if (s != GDN_OK) return s;
    return from_hip(gdn::launch_gdn2_bwd(q, k, v, log_alpha, b, w, dO, dht, Eh, Qh, Kh, Gam, Tm, P, D, Sck, dSck, dq,
                                         dk, dv, dlog_alpha, db, dw, dh0, B, T, H, Dk, Dv, bf, scale, st));
}

gdn_status gdn_prologue(const void *xq, const void *xk, const void *xv, const float *a, const float *b,
                        const float *wq, const float *wk, const float *wv, const float *A_log, const float *dt_bias,
                        const float *conv_in, void *q, void *k, void *v, float *g, float *beta, float *conv_out,
                        int B, int T, int H, int Dk, int Dv, void *stream) {
    if (!xq || !xk || !xv || !a || !b || !wq || !wk || !wv || !A_log || !dt_bias || !q || !k || !v || !g || !beta)
        return GDN_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || H < 1 || (long long)B * T * H >= (1LL << 33)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dk) || !head_ok(Dv)) return GDN_ERR_UNSUPPORTED;
    for (const void *p : {xq, xk, xv, (const void *)q, (const void *)k, (const void *)v, (const void *)wq,
                          (const void *)wk, (const void *)wv, (const void *)conv_in})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    if (!aligned(conv_out, 4)) return GDN_ERR_INVALID_ARG;
    const size_t ntok = (size_t)B * T * H, C = (size_t)H * (2 * Dk + Dv);
    const size_t nstate = (size_t)B * 3 * C * sizeof(float);
    const Range rxq{xq, ntok * Dk * 2}, rxk{xk, ntok * Dk * 2}, rxv{xv, ntok * Dv * 2}, ra{a, ntok * 4},
        rb{b, ntok * 4}, rwq{wq, (size_t)H * Dk * 16}, rwk{wk, (size_t)H * Dk * 16}, rwv{wv, (size_t)H * Dv * 16},
        rA{A_log, (size_t)H * 4}, rdt{dt_bias, (size_t)H * 4}, rci{conv_in, conv_in ? nstate : 0},
        rq{q, ntok * Dk * 2}, rk{k, ntok * Dk * 2}, rv{v, ntok * Dv * 2}, rg{g, ntok * 4}, rbe{beta, ntok * 4},
        rco{conv_out, conv_out ? nstate : 0};
    const Range ins[] = {rxq, rxk, rxv, ra, rb, rwq, rwk, rwv, rA, rdt, rci};
    const Range outs[] = {rq, rk, rv, rg, rbe};
    for (int i = 0; i < 5; ++i) {
        for (Range in : ins)
            if (overlap(outs[i], in)) return GDN_ERR_INVALID_ARG;
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_INVALID_ARG;
        if (overlap(outs[i], rco)) return GDN_ERR_INVALID_ARG;
    }
    if (conv_out) {
        if (overlap(rco, rci) && conv_out != conv_in) return GDN_ERR_INVALID_ARG;
        for (int i = 0; i < 10; ++i)
            if (overlap(rco, ins[i])) return GDN_ERR_INVALID_ARG;
    }
    return from_hip(gdn::launch_prologue(xq, xk, xv, a, b, wq, wk, wv, A_log, dt_bias, conv_in, q, k, v, g, beta,
                                         conv_out, B, T, H, Dk, Dv, (hipStream_t)stream));
}

gdn_status gdn_gated_rmsnorm(const float *o, const void *z, const float *weight, void *y, long long rows, int Dv,
                             float eps, void *stream) {
    if (!o || !z || !weight || !y || rows < 1 || rows >= (1LL << 33) || !(eps > 0.f)) return GDN_ERR_INVALID_ARG;
    if (!head_ok(Dv)) return GDN_ERR_UNSUPPORTED;
    if (!aligned(o, 16) || !aligned(z, 16) || !aligned(weight, 16) || !aligned(y, 16)) return GDN_ERR_INVALID_ARG;
    const Range ry{y, (size_t)rows * Dv * 2};
    for (Range in : {Range{o, (size_t)rows * Dv * 4}, Range{z, (size_t)rows * Dv * 2}, Range{weight, (size_t)Dv * 4}})
        if (overlap(ry, in)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_gated_rmsnorm(o, z, weight, y, (long)rows, Dv, eps, (hipStream_t)stream));
}

}  // extern "C"
