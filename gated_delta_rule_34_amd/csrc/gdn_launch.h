// gdn_launch.h -- host-side launch functions of the gfx950 kernels (internal;
// the public boundary is include/gdn.h).  Each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// exact: fp32 operands also for bf16 inputs (used by the backward's recompute).
// G2d (nullable): the gate sums also in fp64 [B, H, NT, 64] (for the backward).
hipError_t launch_intra(const void *k, const float *g, const float *beta, float *G2, float *Tinv, int B,
                        int T, int H, int Dk, bool bf16, hipStream_t st, bool exact = false,
                        double *G2d = nullptr);

// ck (nullable): entry state of every chunk, [B, H, NT, Dk, Dv] fp32; o may
// then be null to skip the output.
hipError_t launch_walk(const void *q, const void *k, const void *v, const float *beta, const float *G2,
                       const float *Tinv, const float *h0, float *o, float *ht, float *ck, int B, int T, int H,
                       int Dk, int Dv, bool bf16, float scale, hipStream_t st, bool exact = false);

// Single-kernel chunked forward for bf16 inputs (no workspace).  With
// cu_seqlens (device, B + 1 int32 offsets) the tensors hold B packed
// sequences of T tokens in total; otherwise a dense [B, T, H, D] batch.
// The forward walk of bf16 inputs storing only the state that enters every
// chunk: states [B, H, ceil(T / 64), Dk, Dv] fp32 (a backward's recompute),
// with T - I of every chunk from Tws (fp32 [B, H, ceil(T / 64), 64, 64]).
hipError_t launch_fused_states_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                    const float *Tws, const float *h0, float *states, int B, int T, int H, int Dk,
                                    int Dv, hipStream_t st);
hipError_t launch_fused_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                             const float *h0, float *o, float *ht, const int *cu_seqlens, int B, int T, int H, int Dk,
                             int Dv, float scale, hipStream_t st);

// The same forward over a dense batch as a chunk-parallel state scan (Dk =
// Dv = D): each sequence in NS segments of L chunks; output-free walks give
// every segment but the last its end state from its entry (segment 0) or from
// zero, and its transfer matrix (middle segments); a scan gives every
// segment's true entry state; then the single kernel runs all segments as
// packed sequences.  Hin, Hout, M: [B NS, H, D, D] fp32, cu: B NS + 1 int32
// (the caller's workspace).
hipError_t launch_fused_seg_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                 const float *h0, float *o, float *ht, int B, int T, int H, int D, float scale,
                                 int NS, int L, float *Hin, float *Hout, float *M, int *cu, hipStream_t st);

// Gated DeltaNet-2, two stages: per-chunk prepared operands (decayed e, q
// and k; Gamma_C; T - I; strict P; diag P), then the state walk.
hipError_t launch_gdn2_intra(const void *q, const void *k, const float *la, const void *bg, void *Ehat, void *Qhat,
                             void *Khat, float *GamC, float *Tinv, float *P, float *D, int B, int T, int H, int Dk,
                             bool bf16, hipStream_t st);

hipError_t launch_gdn2_walk(const void *Ehat, const void *Qhat, const void *Khat, const float *GamC,
                            const float *Tinv, const float *P, const float *D, const void *v, const void *wg,
                            const float *h0, float *o, float *ht, int B, int T, int H, int Dk, int Dv, bool bf16,
                            float scale, hipStream_t st);

// Gated DeltaNet-2 for bf16 inputs: a parallel prep kernel writes one block
// of prepared operands per chunk into ws (gdn2_fused_block_bytes(Dk) each),
// then the walk kernel carries the state through the chunks; when the walk
// leaves compute units idle, the sequence runs in time parts and the prep of
// one part shares a launch with the walk of the previous one.  ws holds
// gdn2_fused_ws_bytes() bytes.
size_t gdn2_fused_block_bytes(int Dk);
size_t gdn2_fused_ws_bytes(int B, int T, int H, int Dk, int Dv);
hipError_t launch_gdn2_fused_bf16(const void *q, const void *k, const float *la, const void *bg, const void *v,
                                  const void *wg, const float *h0, float *o, float *ht, void *ws, int B, int T,
                                  int H, int Dk, int Dv, float scale, hipStream_t st);

// The same kernels over packed variable-length sequences (cu_seqlens on the
// device, N + 1 offsets into total_T tokens): two small kernels number the
// chunks of every sequence into NC = ceil(total_T / 64) + N chunk numbers,
// the prep fills block (head, number) of each, and one walk workgroup per
// (sequence, head, 32 value columns) carries the state.  ws layout in
// Gdn2VarWs (total bytes, offsets of the sequence and chunk tables).
struct Gdn2VarWs {
    long long NC;
    size_t seq_off, tab_off, total;
};
Gdn2VarWs gdn2_var_ws(int N, int total_T, int H, int Dk);
hipError_t launch_gdn2_fused_varlen_bf16(const void *q, const void *k, const float *la, const void *bg,
                                         const void *v, const void *wg, const int *cu, const float *h0, float *o,
                                         float *ht, void *ws, int N, int total_T, int H, int Dk, int Dv, float scale,
                                         hipStream_t st);

hipError_t launch_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                       float *S, float *o, int B, int H, int Dk, int Dv, bool bf16, float scale,
                       hipStream_t st);

hipError_t launch_step2(const void *q, const void *k, const void *v, const float *la, const void *bg,
                        const void *wg, float *S, float *o, int B, int H, int Dk, int Dv, bool bf16, float scale,
                        hipStream_t st);

// The reverse state walk of the GDN backward for bf16 inputs in one fused
// kernel (gdn_bwd_fused.hip): dS' of every chunk into dSck, dh0 (nullable).
hipError_t launch_bwd_walk_fused(const void *q, const void *k, const float *beta, const float *dO, const float *dht,
                                 const double *G2, const float *Tinv, float *dSck, float *dh0, int B, int T, int H,
                                 int Dk, int Dv, float scale, hipStream_t st);

// Backward of the chunked GDN forward (gdn_bwd.hip): the reverse state walk
// (dS' of every chunk into dSck, dh0) and the per-chunk gradients, given the
// intra stage (G2, T - I) and the entry state of every chunk (Sck).
hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *beta, const float *dO,
                      const float *dht, const double *G2, const float *Tinv, const float *Sck, float *dSck, float *dq,
                      float *dk, float *dv, float *dg, float *dbeta, float *dh0, int B, int T, int H, int Dk, int Dv,
                      bool bf16, float scale, hipStream_t st);

// Backward of the chunked GDN-2 forward: the fp32 forward recompute
// (gdn2_chunk.hip; intra operands into Eh .. D, chunk entry states into ck),
// then the reverse walk and the per-chunk gradients (gdn2_bwd.hip), which
// overwrite Eh, Qh, Kh, GamC, Tinv and P with their gradients.
// Entry state of every chunk of the GDN-2 forward from the intra stage's
// fp32 operands (bf16 v and w), on split 16-bit MFMA operands.
hipError_t launch_gdn2_states_bf16(const float *Eh, const float *Kh, const float *Tws, const float *GamC,
                                   const void *v, const void *w, const float *h0, float *ck, int B, int T, int H,
                                   int Dk, int Dv, hipStream_t st);
hipError_t launch_gdn2_recompute(const void *q, const void *k, const float *la, const void *bg, const void *v,
                                 const void *wg, const float *h0, float *Eh, float *Qh, float *Kh, float *GamC,
                                 float *Tinv, float *P, float *D, float *ck, int B, int T, int H, int Dk, int Dv,
                                 bool bf16, hipStream_t st);
hipError_t launch_gdn2_bwd(const void *q, const void *k, const void *v, const float *la, const void *bg,
                           const void *wg, const float *dO, const float *dht, float *Eh, float *Qh, float *Kh,
                           float *GamC, float *Tws, float *Pws, const float *Dws, const float *Sck, float *dSck,
                           float *dq, float *dk, float *dv, float *dla, float *db, float *dw, float *dh0, int B, int T,
                           int H, int Dk, int Dv, bool bf16, float scale, hipStream_t st);

// Prologue and epilogue around the rule (gdn_prologue.hip).
hipError_t launch_prologue(const void *xq, const void *xk, const void *xv, const float *a, const float *b,
                           const float *wq, const float *wk, const float *wv, const float *A_log,
                           const float *dt_bias, const float *state_in, void *q, void *k, void *v, float *g,
                           float *beta, float *state_out, int B, int T, int H, int Dk, int Dv, hipStream_t st);
hipError_t launch_gated_rmsnorm(const float *o, const void *z, const float *w, void *y, long rows, int Dv, float eps,
                                hipStream_t st);

}  // namespace gdn
