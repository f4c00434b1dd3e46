/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library.
 *
 * The operation (per independent (batch b, head h) pair, tokens t = 0..T-1):
 *
 *   Gated DeltaNet ("GatedDeltaNet walkthrough", yfxerp.com, section
 *   "Delta Rule: predict first, then correct" -- the recurrence and the
 *   per-token reference loop):
 *       S_t = (I - beta_t k_t k_t^T) exp(g_t) S_{t-1} + beta_t k_t v_t^T
 *       o_t = scale * S_t^T q_t          (read-out after the update)
 *   S_t is d_k x d_v (key rows, value columns).  The forward is evaluated in
 *   64-token chunks through the WY form (same article, section on the
 *   chunked Triton kernels: block size 64, one state matrix carried between
 *   blocks, the gate cumsum scaled by log2(e) for exp2).
 *
 *   Gated DeltaNet-2 ("NVIDIA AI lanza Gated DeltaNet-2", 7minutos.es,
 *   section "Regla-2 del Delta cerrado"):
 *       S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T
 *   with per-key-channel decay alpha_t = exp(log_alpha_t), erase gate b_t
 *   (key channels) and write gate w_t (value channels); same read-out.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *     row-major and densely packed in the layouts stated per argument.
 *     The caller owns every buffer (inputs, outputs, workspace); the library
 *     never allocates device memory and keeps no per-call state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  Inputs must stay valid
 *     until the stream has executed the work.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call returns a status and touches no memory.  A failed
 *     launch returns GDN_ERR_HIP.  Nothing is thrown across the ABI.
 *   - `dtype` is the element type of q, k, v (and GDN-2's b, w):
 *     GDN_F32 (fp32) or GDN_BF16 (bf16).  Gates (g, beta, log_alpha), the
 *     state (h0, ht, S) and the output o are always fp32.
 *   - Supported head sizes: Dk, Dv in {64, 128}.  B, T, H >= 1.  Any T
 *     (the last chunk may be partial).  Offsets are 64-bit.
 *   - g and log_alpha are log-decays and must be finite and <= 0; positive
 *     values are accepted but not guaranteed (exp2 of a positive difference
 *     may overflow).  beta, b, w are expected in [0, 1].
 *   - Results are bitwise reproducible for identical inputs, sizes and device.
 *   - Operand range of the bf16 paths.  They round some intermediate values
 *     to fp16 (11 significant bits, largest finite value 65,504) for the
 *     matrix-core products: in gdn_chunk_fwd and gdn_chunk_fwd_varlen the
 *     chunk residuals R = beta (v - gamma K S), the new values, T - I and P;
 *     in gdn2_chunk_fwd and gdn2_chunk_fwd_varlen also the decayed keys and queries and the state as
 *     hi + lo parts.  With ||k_t|| <= 1, beta in [0, 1] and g <= 0 one has
 *     |T - I| <= 1, |P| <= scale, and for every value column c
 *       |R|, |new values| <= max_t |v_{t,c}| + sqrt(||h0[:, c]||^2 + sum_t beta_t v_{t,c}^2)
 *     (each token grows the squared norm of a state column by at most
 *     beta v^2); keep this below 32,768.  For Gated DeltaNet-2 keep the state
 *     entries and |w . v| below 32,768.  Beyond that the output may hold inf
 *     or NaN and no error is reported.  Magnitudes below 2^-14 fall into
 *     fp16's subnormal range and lose precision, so v and h0 should not be
 *     uniformly tiny (rms below about 2^-10).  The fp32 paths have fp32 range.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, bad alias */
    GDN_ERR_UNSUPPORTED = 2,  /* head size or dtype not built */
    GDN_ERR_WORKSPACE = 3,    /* workspace null, misaligned or too small */
    GDN_ERR_HIP = 4           /* a HIP launch failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *gdn_status_string(gdn_status s);

/* Bytes of device workspace gdn_chunk_fwd needs for these sizes (0 only if
 * the sizes are invalid).  The workspace must be 256-byte aligned.  bf16
 * inputs run as one kernel and use no workspace (ws may then be NULL);
 * fp32 inputs run the two stages below and keep their per-chunk results
 * (G2, Tinv) in the workspace. */
size_t gdn_chunk_fwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype);

/*
 * gdn_chunk_fwd -- chunked Gated DeltaNet forward.
 *   q, k   [B, T, H, Dk]  dtype          queries / keys (the pages L2-normalise them
 *                                         upstream; not required here)
 *   v      [B, T, H, Dv]  dtype          values
 *   g      [B, T, H]      fp32           log-decay per token-head (exp(g) in (0, 1])
 *   beta   [B, T, H]      fp32           write strength
 *   h0     [B, H, Dk, Dv] fp32, nullable initial state (NULL = zeros)
 *   o      [B, T, H, Dv]  fp32           output, fully overwritten
 *   ht     [B, H, Dk, Dv] fp32, nullable final state; may alias h0 exactly
 *   scale  read-out scale (1/sqrt(Dk) in the pages' layer)
 *   ws, ws_bytes  device workspace of at least gdn_chunk_fwd_workspace(...) bytes
 * No other aliasing between arguments is allowed.  With bf16 inputs q, k, v
 * and o must be 16-byte aligned (GDN_ERR_INVALID_ARG otherwise).
 */
gdn_status gdn_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0,
                         float *o, float *ht,
                         int B, int T, int H, int Dk, int Dv, gdn_dtype dtype, float scale,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_chunk_intra -- the per-chunk, state-independent stage of gdn_chunk_fwd,
 * exposed for stage-wise checks.  For chunk c = 0..NT-1 (NT = ceil(T/64)) of
 * head (b, h), with tokens past T treated as k = 0, g = 0, beta = 0:
 *   G2    [B, H, NT, 64]      fp32  log2(e) * chunk-local cumsum of g
 *   Tinv  [B, H, NT, 64, 64]  fp32  (I + A)^-1 - I, A_ij = beta_i (k_i . k_j)
 *                                   2^(G2_i - G2_j) for i > j, else 0
 *                                   (strictly lower triangular; upper part 0)
 */
gdn_status gdn_chunk_intra(const void *k, const float *g, const float *beta,
                           float *G2, float *Tinv,
                           int B, int T, int H, int Dk, gdn_dtype dtype, void *stream);

/*
 * gdn_chunk_walk -- the sequential stage of gdn_chunk_fwd: given the
 * per-chunk G2 and Tinv that gdn_chunk_intra produced for the same k, g,
 * beta, walk the chunks in order carrying the state and write o and ht.
 * gdn_chunk_intra followed by gdn_chunk_walk on one stream enqueues exactly
 * the work of gdn_chunk_fwd.  Argument meanings as in gdn_chunk_fwd;
 * G2 [B, H, NT, 64] and Tinv [B, H, NT, 64, 64] are read only.
 */
gdn_status gdn_chunk_walk(const void *q, const void *k, const void *v, const float *beta,
                          const float *G2, const float *Tinv, const float *h0,
                          float *o, float *ht,
                          int B, int T, int H, int Dk, int Dv, gdn_dtype dtype, float scale,
                          void *stream);

/* Bytes of workspace gdn2_chunk_fwd needs (256-byte aligned buffer). */
size_t gdn2_chunk_fwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype);

/*
 * gdn2_chunk_fwd -- chunked Gated DeltaNet-2 forward.
 *   q, k       [B, T, H, Dk] dtype;  v [B, T, H, Dv] dtype
 *   log_alpha  [B, T, H, Dk] fp32    per-key-channel log-decay (alpha = exp(log_alpha))
 *   b          [B, T, H, Dk] dtype   erase gate (key channels)
 *   w          [B, T, H, Dv] dtype   write gate (value channels)
 *   h0, o, ht, scale, ws, ws_bytes, stream: as gdn_chunk_fwd.
 * With bf16 inputs q, k, v, b, w and o must be 16-byte aligned
 * (GDN_ERR_INVALID_ARG otherwise).
 */
gdn_status gdn2_chunk_fwd(const void *q, const void *k, const void *v,
                          const float *log_alpha, const void *b, const void *w,
                          const float *h0, float *o, float *ht,
                          int B, int T, int H, int Dk, int Dv, gdn_dtype dtype, float scale,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * gdn2_chunk_fwd_noalloc -- gdn2_chunk_fwd for callers that cannot allocate
 * device memory at all (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * gdn2_chunk_fwd, without ws / ws_bytes: the workspace is a fixed device
 * array inside the library, GDN2_NOALLOC_SCRATCH_BYTES (144 MiB) per GPU,
 * held from the library's first use on that GPU until the process ends.  It
 * holds gdn2_chunk_fwd_workspace(B, T, H, Dk, Dv, dtype) bytes: with bf16
 * inputs and Dk = Dv = 128, 66,304 bytes per chunk-head
 * (B * H * ceil(T / 64) of them) and 65,536 bytes per (batch, head), e.g.
 * 137.9 MB for B = 4, H = 8, T = 4096.  Larger sizes return
 * GDN_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing; its first call on a
 * device looks up that device's copy of the array.  Every call on one GPU
 * shares that copy, so calls that overlap on one GPU (several streams or
 * host threads) race: the caller serialises them.
 */
#define GDN2_NOALLOC_SCRATCH_BYTES (144u * 1024u * 1024u)

size_t gdn2_chunk_fwd_noalloc_max_bytes(void);

gdn_status gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                  const float *log_alpha, const void *b, const void *w,
                                  const float *h0, float *o, float *ht,
                                  int B, int T, int H, int Dk, int Dv, gdn_dtype dtype,
                                  float scale, void *stream);

/*
 * gdn_recurrent_step -- one decode token of Gated DeltaNet, state updated in
 * place (the per-token loop of the walkthrough's "Delta Rule" section):
 *   S <- exp(g) S;  u = beta (v - S^T k);  S <- S + k u^T;  o = scale S^T q
 *   q, k [B, H, Dk] dtype;  v [B, H, Dv] dtype;  g, beta [B, H] fp32
 *   S    [B, H, Dk, Dv] fp32, read and written in place
 *   o    [B, H, Dv] fp32
 */
gdn_status gdn_recurrent_step(const void *q, const void *k, const void *v,
                              const float *g, const float *beta, float *S, float *o,
                              int B, int H, int Dk, int Dv, gdn_dtype dtype, float scale,
                              void *stream);

/*
 * gdn2_recurrent_step -- one decode token of Gated DeltaNet-2, state updated
 * in place (one step of the recurrence in the Gated DeltaNet-2 article,
 * section "Regla-2 del Delta cerrado"):
 *   S <- Diag(exp(log_alpha)) S;  u = w . v - S^T (b . k);  S <- S + k u^T;
 *   o = scale S^T q
 *   q, k [B, H, Dk] dtype;  v [B, H, Dv] dtype
 *   log_alpha [B, H, Dk] fp32 (<= 0);  b [B, H, Dk] dtype;  w [B, H, Dv] dtype
 *   S    [B, H, Dk, Dv] fp32, read and written in place
 *   o    [B, H, Dv] fp32
 * Errors: GDN_ERR_INVALID_ARG for null pointers, non-positive sizes or
 * overlapping S / o with any other buffer; GDN_ERR_UNSUPPORTED for head sizes
 * other than 64 and 128 or an unknown dtype; GDN_ERR_HIP if the launch fails.
 * Asynchronous on `stream`; the caller owns every buffer.
 */
gdn_status gdn2_recurrent_step(const void *q, const void *k, const void *v,
                               const float *log_alpha, const void *b, const void *w,
                               float *S, float *o, int B, int H, int Dk, int Dv,
                               gdn_dtype dtype, float scale, void *stream);

/*
 * gdn_chunk_fwd_varlen -- gdn_chunk_fwd on N packed sequences of different
 * lengths (the production input form; each sequence is chunked and carried
 * on its own, exactly as a batch entry of gdn_chunk_fwd).
 *   q, k [total_T, H, Dk] and v [total_T, H, Dv] bf16; g, beta [total_T, H] fp32
 *   cu_seqlens  device int32 [N + 1]: sequence n is tokens cu_seqlens[n] ..
 *               cu_seqlens[n + 1] - 1; non-decreasing from 0 to total_T (the
 *               kernel clamps the offsets into [0, total_T], so malformed
 *               offsets give wrong sequences but never an out-of-range access;
 *               an empty sequence passes its initial state through)
 *   h0, ht [N, H, Dk, Dv] fp32 (nullable; ht may alias h0);  o [total_T, H, Dv] fp32
 * bf16 only (GDN_ERR_UNSUPPORTED for fp32); no workspace.  Errors as
 * gdn_chunk_fwd, plus GDN_ERR_INVALID_ARG for a null cu_seqlens.
 */
gdn_status gdn_chunk_fwd_varlen(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const int *cu_seqlens, const float *h0,
                                float *o, float *ht, int N, int total_T, int H, int Dk, int Dv,
                                gdn_dtype dtype, float scale, void *stream);

/* Bytes of workspace gdn2_chunk_fwd_varlen needs (256-byte aligned buffer);
 * 0 for unsupported arguments (fp32, head sizes, sizes out of range). */
size_t gdn2_chunk_fwd_varlen_workspace(int N, int total_T, int H, int Dk, int Dv, gdn_dtype dtype);

/*
 * gdn2_chunk_fwd_varlen -- gdn2_chunk_fwd on N packed sequences of different
 * lengths (Gated DeltaNet-2 article, "Regla-2 del Delta cerrado", for the
 * recurrence; each sequence is chunked from its own first token and carried
 * on its own, exactly as a batch entry of gdn2_chunk_fwd).
 *   q, k, b [total_T, H, Dk] and v, w [total_T, H, Dv] bf16, 16-byte aligned
 *   log_alpha  [total_T, H, Dk] fp32
 *   cu_seqlens device int32 [N + 1], as in gdn_chunk_fwd_varlen (offsets
 *              clamped into [0, total_T]; an empty sequence passes its
 *              initial state through)
 *   h0, ht [N, H, Dk, Dv] fp32 (nullable; ht may alias h0);  o [total_T, H, Dv] fp32
 *   ws  device, 256-byte aligned, >= gdn2_chunk_fwd_varlen_workspace(...)
 *       bytes, owned by the caller: the per-chunk blocks of all sequences
 *       (numbered into ceil(total_T / 64) + N chunk numbers per head) and two
 *       small tables the call derives from cu_seqlens on the device.
 * bf16 only (GDN_ERR_UNSUPPORTED for fp32).  Errors as gdn2_chunk_fwd, plus
 * GDN_ERR_INVALID_ARG for a null cu_seqlens.  Asynchronous on `stream`.
 */
gdn_status gdn2_chunk_fwd_varlen(const void *q, const void *k, const void *v,
                                 const float *log_alpha, const void *b, const void *w,
                                 const int *cu_seqlens, const float *h0, float *o, float *ht,
                                 int N, int total_T, int H, int Dk, int Dv, gdn_dtype dtype,
                                 float scale, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of gdn_chunk_fwd (training): gradients of
 * L = sum(dO . o) + sum(dht . ht) with respect to every input, by reverse-mode
 * differentiation of the chunk equations of the forward (WY form over 64-token
 * chunks, the chunked-kernel section of the walkthrough): a forward walk
 * recomputes the state entering every chunk, a reverse walk over the chunks
 * carries the state gradient, then every chunk is recomputed and
 * differentiated in parallel.  fp32 values and accumulation throughout.  With
 * fp32 inputs the products run on fp32 MFMA.  With bf16 inputs they run on
 * bf16 or fp16 MFMA: exact where an operand is a bf16 input, and otherwise on
 * hi + lo (about 16 bits) or hi + mid + lo (about 24 bits) parts of the fp32
 * operands, chosen per product so that every gradient stays near the error of
 * the same equations with fp32 products; q, k and v must then be 16-byte
 * aligned.
 *   inputs  as gdn_chunk_fwd (h0 nullable), dO [B, T, H, Dv] fp32,
 *           dht [B, H, Dk, Dv] fp32 or NULL (no gradient on the final state)
 *   outputs dq, dk [B, T, H, Dk], dv [B, T, H, Dv], dg, dbeta [B, T, H],
 *           dh0 [B, H, Dk, Dv] or NULL, all fp32
 *   ws      gdn_chunk_bwd_workspace() bytes, 256-byte aligned, caller-owned
 * Errors: GDN_ERR_INVALID_ARG for null required pointers, bad sizes,
 * misaligned bf16 q, k, v or any output overlapping an input, another output
 * or the workspace; GDN_ERR_UNSUPPORTED for head sizes other than 64 and 128
 * or an unknown dtype; GDN_ERR_WORKSPACE for a missing, misaligned or short
 * workspace; GDN_ERR_HIP if a launch fails.  Asynchronous on `stream`.
 */
size_t gdn_chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype);

gdn_status gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, const float *dO,
                         const float *dht, float *dq, float *dk, float *dv, float *dg,
                         float *dbeta, float *dh0, int B, int T, int H, int Dk, int Dv,
                         gdn_dtype dtype, float scale, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * Backward of gdn2_chunk_fwd (training): gradients of
 * L = sum(dO . o) + sum(dht . ht) with respect to every input, by reverse-mode
 * differentiation of the GDN-2 chunk equations (the WY form with the channel
 * decay inside both factors of every product, "NVIDIA AI lanza Gated
 * DeltaNet-2", sections "Regla-2 del Delta cerrado" and on chunked training):
 * a forward recompute stores every chunk's entry state, a reverse walk
 * carries the state gradient, then every chunk is differentiated in parallel
 * (the decay-weighted contractions with exact per-channel exponentials).
 * fp32 accumulation throughout; with bf16 inputs the recompute's products
 * take their fp32 operands as bf16 or fp16 hi + lo parts (about 16 and 22
 * bits), and q, k, v, b, w and log_alpha must be 16-byte aligned.
 *   inputs  as gdn2_chunk_fwd (h0 nullable), dO [B, T, H, Dv] fp32,
 *           dht [B, H, Dk, Dv] fp32 or NULL (no gradient on the final state)
 *   outputs dq, dk, dlog_alpha, db [B, T, H, Dk], dv, dw [B, T, H, Dv],
 *           dh0 [B, H, Dk, Dv] or NULL, all fp32
 *   ws      gdn2_chunk_bwd_workspace() bytes, 256-byte aligned, caller-owned
 * Errors as gdn_chunk_bwd (GDN_ERR_INVALID_ARG also for a misaligned bf16
 * input).  Asynchronous on `stream`.
 */
size_t gdn2_chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv, gdn_dtype dtype);

gdn_status gdn2_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                          const void *b, const void *w, const float *h0, const float *dO,
                          const float *dht, float *dq, float *dk, float *dv, float *dlog_alpha,
                          float *db, float *dw, float *dh0, int B, int T, int H, int Dk, int Dv,
                          gdn_dtype dtype, float scale, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_prologue -- the per-token work between the input projections and the
 * rule, in one pass ("GatedDeltaNet walkthrough", the data-flow overview and
 * the sections on the short convolution and the gates):
 *   q = l2norm(SiLU(conv(xq))), k = l2norm(SiLU(conv(xk))), v = SiLU(conv(xv))
 *   g = -exp(A_log[h]) * softplus(a + dt_bias[h]),  beta = sigmoid(b)
 * conv is a causal depthwise convolution over the last 4 tokens of each
 * channel, without bias, whose last tap multiplies the current token:
 *   conv(x)_t[c] = sum_{j=0..3} w[c][j] x_{t-3+j}[c]
 * Before t = 0 it reads the carried convolution state (zeros when NULL).
 * l2norm divides by sqrt(sum of squares over the head's channels + 1e-6).
 *   xq, xk  [B, T, H, Dk] bf16,  xv [B, T, H, Dv] bf16  projections
 *   a, b    [B, T, H] fp32      gate pre-activations
 *   wq, wk  [H*Dk, 4] fp32, wv [H*Dv, 4] fp32  taps per channel
 *   A_log, dt_bias [H] fp32
 *   conv_in  [B, 3, H*(2 Dk + Dv)] fp32, nullable: the 3 inputs before t = 0,
 *            oldest first; channels are the q channels, then k, then v
 *   q, k [B, T, H, Dk] bf16, v [B, T, H, Dv] bf16, g, beta [B, T, H] fp32: outputs,
 *            ready as inputs of gdn_chunk_fwd / gdn_recurrent_step
 *   conv_out same layout as conv_in, nullable: the 3 inputs ending at token
 *            T - 1 (the decode cache); may be conv_in itself (updated in place)
 * Every pointer except a, b, A_log, dt_bias, g, beta and conv_out must be
 * 16-byte aligned (conv_out 4-byte).
 * Errors: GDN_ERR_INVALID_ARG for null required pointers, bad sizes,
 * misalignment or overlapping outputs; GDN_ERR_UNSUPPORTED for head sizes
 * other than 64 and 128; GDN_ERR_HIP if a launch fails.  Asynchronous.
 */
gdn_status gdn_prologue(const void *xq, const void *xk, const void *xv, const float *a,
                        const float *b, const float *wq, const float *wk, const float *wv,
                        const float *A_log, const float *dt_bias, const float *conv_in, void *q,
                        void *k, void *v, float *g, float *beta, float *conv_out, int B, int T,
                        int H, int Dk, int Dv, void *stream);

/*
 * gdn_gated_rmsnorm -- the output stage after the rule (same walkthrough,
 * data-flow overview: RMS normalisation with a SiLU output gate):
 *   y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z), per row of Dv channels
 *   o [rows, Dv] fp32, z [rows, Dv] bf16, weight [Dv] fp32 (one weight per
 *   channel, shared by every head), y [rows, Dv] bf16; all 16-byte aligned;
 *   rows = B * T * H for the layout of gdn_chunk_fwd's o.  eps > 0.
 * Errors: GDN_ERR_INVALID_ARG (null, rows < 1, eps <= 0, misalignment, y
 * overlapping an input), GDN_ERR_UNSUPPORTED (Dv not 64 or 128),
 * GDN_ERR_HIP.  Asynchronous.
 */
gdn_status gdn_gated_rmsnorm(const float *o, const void *z, const float *weight, void *y,
                             long long rows, int Dv, float eps, void *stream);

/*
 * gdn_clock_probe -- measurement aid, not part of the operation: enqueues
 * nblocks single-wave workgroups that each spin for spin_us microseconds of
 * real time and write two counts to out (device, 2 * nblocks uint64): the
 * shader cycles (s_memtime) and the 100 MHz real-time ticks (s_memrealtime)
 * that passed, so that clock_MHz = 100 * cycles / ticks.  Enqueued right
 * after a run of kernels it reads the clock those kernels ran at.  Errors:
 * GDN_ERR_INVALID_ARG (null out, nblocks outside 1..65536, spin_us outside
 * 1..100000), GDN_ERR_HIP.  Asynchronous.
 */
gdn_status gdn_clock_probe(unsigned long long *out, int nblocks, int spin_us, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
