/*
 * hwa.h -- C ABI of the MI355X (gfx950) hybrid window-softmax attention.
 *
 * The operation is the forward pass of the VDN-H3 hybrid attention as the
 * VDN-H3 article ("VDN-Minimax-H3", icman.com.cn news 81972) defines it:
 *
 *   out = o_sm + y
 *
 * o_sm  windowed softmax attention: query frame t attends to every token of
 *       key frames [lo_t, hi_t], a chunk-aligned window (article section
 *       "What the far field outside the window is").
 * y     bidirectional delta-rule linear branch for every frame outside the
 *       window (article sections "Step 1" .. "Step 5" and "Text state"):
 *         q^ = L2(SiLU(q)), k^ = L2(SiLU(conv_k(k))), v^ = conv_v(v)
 *         A_f = sum_{n in f} beta_n k^_n k^_n^T,  B_f = sum beta_n v^_n k^_n^T
 *         scans P_f = R(P_{f-1}), Q_f = R(Q_{f+1}) from text_scale * S_text
 *         S_t = P_{lo_t-1} diag(prod_{lo_t..t} alpha) + Q_{hi_t+1} diag(prod_{t..hi_t} alpha)
 *         y_n = RMSNorm(S_t q^_n) * w * sigmoid(gate_n)
 *       with R one of the article's three update rules ("Step 3" table):
 *         vdn_solve   (S D + B)(I + A)^-1
 *         sana_scaled (S D)(I - c^2 A) + c B
 *         vdn_scaled  (S D + c B)(I + c^2 A)^-1,   D = diag(alpha_f).
 *
 * Conventions for every entry point:
 *  - Tensors are device pointers to row-major contiguous memory; tokens are
 *    frame-major (token n = t * tokens_per_frame + s). Shapes use B = batch,
 *    H = heads, d = head_dim, F = frames, S = tokens_per_frame, N = F * S.
 *  - The library never allocates or frees memory and keeps no pointer after
 *    a call returns; the caller owns every buffer, including the workspace.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising. Faults during execution surface
 *    at the caller's next synchronisation.
 *  - Every argument check happens before the first enqueue: on an error the
 *    call returns a status and writes nothing. No exception crosses the ABI
 *    and nothing is printed. Non-finite inputs are not checked.
 *  - Calls are stateless and thread-safe.
 */
#ifndef HWA_H
#define HWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, declared as HIP's own headers declare it (an opaque
 * pointer; the identical typedef may appear again when hip_runtime.h is
 * included too). */
struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  HWA_OK = 0,
  HWA_ERR_INVALID_ARG = 1, /* NULL pointer, size <= 0, bad enum, aliasing  */
  HWA_ERR_UNSUPPORTED = 2, /* head_dim or dtype the kernels do not handle  */
  HWA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required      */
  HWA_ERR_HIP = 4          /* a HIP launch error                           */
} hwa_status;

/* Update rule R of the scans (article "Step 3", rules table). */
typedef enum {
  HWA_RULE_VDN_SOLVE = 0,
  HWA_RULE_SANA_SCALED = 1,
  HWA_RULE_VDN_SCALED = 2
} hwa_rule;

/* Element type of q, k, v, gate, out (and of the text tokens). */
typedef enum { HWA_F32 = 0, HWA_BF16 = 1 } hwa_dtype;

/* Flags. Every hybrid_attn_fwd call leaves its intermediates (window table,
 * A, B, M, the state banks, S_t) in the workspace at the offsets
 * hwa_get_workspace_layout reports, so no flag asks for them; bit 4 is
 * unused and, like any unknown bit, rejected with HWA_ERR_INVALID_ARG. */
enum {
  HWA_FLAG_SOFTMAX_ONLY = 1,      /* out = o_sm (linear branch skipped)      */
  HWA_FLAG_LINEAR_ONLY = 2,       /* out = y (softmax branch skipped)        */
  HWA_FLAG_ACCUMULATE = 8,         /* hwa_linear_bwd only: add dq, dk, dv to */
                                   /* what those buffers hold (the softmax   */
                                   /* branch's gradient, for out = o_sm + y) */
  HWA_FLAG_ROUTED = 16             /* hybrid_attn_fwd, bf16: block-sparse    */
                                   /* softmax branch (hwa_params.route_tau;  */
                                   /* see below)                             */
};

typedef struct {
  uint32_t struct_size;  /* = sizeof(hwa_params)                              */
  int32_t batch;         /* B >= 1                                            */
  int32_t heads;         /* H >= 1                                            */
  int32_t head_dim;      /* d: 16, 32, 64 or 128 with fp32; 64 or 128 with     */
                         /* bf16 (other values: HWA_ERR_UNSUPPORTED)           */
  int32_t dtype;         /* hwa_dtype                                          */
  float c;               /* scale c of sana_scaled / vdn_scaled (ignored by    */
                         /* vdn_solve)                                         */
  float text_scale;      /* initial state of both scans = text_scale * S_text  */
                         /* (0.5 in the article's "Text state")                */
  float rms_eps;         /* RMSNorm epsilon (> 0)                              */
  const float* conv_k;   /* [H, d, 4] fp32 causal taps; tap j multiplies the   */
  const float* conv_v;   /*   token j places earlier in the same frame         */
  const float* rms_weight; /* [d] fp32, NULL = ones                            */
  const void* q_rope;    /* [B,H,N,d] softmax-branch q, NULL = use q           */
  const void* k_rope;    /* [B,H,N,d] softmax-branch k, NULL = use k           */
  void* workspace;       /* device scratch of >= hwa_workspace_bytes() bytes,  */
  size_t workspace_bytes;/*   256-byte aligned; contents undefined afterwards  */
  uint32_t flags;        /* HWA_FLAG_*                                         */
  void* const* stage_events; /* NULL, or HWA_NUM_STAGE_EVENTS caller-created  */
                         /* hipEvent_t recorded on `stream` at the kernel     */
                         /* boundaries of hybrid_attn_fwd, for per-kernel     */
                         /* timing: [0] start, then after [1] window table,   */
                         /* [2] statistics, [3] inverses, [4] scan, [5] decay */
                         /* products and (bf16) S_t of every frame, [6] V    */
                         /* transpose (a separate pass only where the         */
                         /* statistics kernel does not write it: frames of a  */
                         /* token count that is not a multiple of 4, or       */
                         /* HWA_FLAG_SOFTMAX_ONLY) and the routing of         */
                         /* HWA_FLAG_ROUTED,                                  */
                         /* [7] softmax (with the                             */
                         /* linear-branch readout fused in, on bf16 calls     */
                         /* that run both branches), [8]                      */
                         /* separate readout (a skipped stage records its     */
                         /* event with the previous one)                      */
  /* Fields below were added later; a caller whose struct_size ends before   */
  /* them gets NULL for each.                                                 */
  float* softmax_lse;    /* NULL, or [B,H,N] fp32: hybrid_attn_fwd writes      */
                         /* lse_n = log sum_m exp(q_n . k_m / sqrt(d)) over    */
                         /* query n's window (the softmax branch's normaliser, */
                         /* for hwa_softmax_bwd)                               */
  void* softmax_out;     /* NULL, or [B,H,N,d] dtype: hybrid_attn_fwd also     */
                         /* writes o_sm alone there (for hwa_softmax_bwd)      */
  float route_tau;       /* HWA_FLAG_ROUTED: keep threshold mean + tau * std   */
                         /* (-INFINITY keeps every block; NaN is rejected)     */
} hwa_params;

/*
 * Block-sparse routing of the softmax branch (HWA_FLAG_ROUTED), an
 * approximation of the windowed softmax after the H3 acceleration report
 * (section 9.7.3, "Sol-Attn": 128-token blocks, block means of Q and K,
 * trial scores q_mean . k_mean, keep the blocks above mean + tau * std,
 * exact attention on the kept blocks). Per (batch, head) and chunk, with the
 * chunk's key window [kb, ke):
 *   query tiles: 256 queries from the chunk's first one; key blocks: the
 *   global 128-token blocks [128 j, 128 j + 128) cut to the window;
 *   q_mean, k_mean: means over the tile's queries / the block's window keys
 *   (of the softmax branch's q and k); s_j = q_mean . k_mean_j / sqrt(d);
 *   block j is kept when s_j >= mean_j s + tau * std_j s (population
 *   standard deviation over the window's blocks), and so is the first block
 *   of largest s; every query of the tile then attends to the keys of its
 *   kept blocks only (fp32 scores, so a block within rounding of the
 *   threshold may go either way).
 * bf16 only; the window may span at most 4096 64-key tiles
 * (HWA_ERR_UNSUPPORTED otherwise). The kept blocks stay in the workspace at
 * the offsets hwa_get_route_layout reports.
 */
hwa_status hwa_get_route_layout(int32_t frames, int32_t tokens_per_frame, int32_t chunk,
                                const hwa_params* p, size_t* count_offset,
                                size_t* list_offset, int32_t* tiles_per_chunk,
                                int32_t* list_stride);

#define HWA_NUM_STAGE_EVENTS 9

/*
 * Byte offsets of the intermediates inside the workspace of one
 * hybrid_attn_fwd call (all fp32 unless stated):
 *   lohi     int32 [2, F]         window bounds lo then hi (inclusive frames)
 *   stat_a   [B, H, F, d, d]      A_f
 *   stat_b   [B, H, F, d, d]      B_f (d_v x d_k)
 *   map_m    [B, H, F, d, d]      fp32 calls: M_f = (I + c~^2 A_f)^-1 (c~ = 1 for
 *                                 vdn_solve, c for vdn_scaled; not written for
 *                                 sana_scaled). bf16 calls: the same bytes hold
 *                                 per frame two bf16 d x d matrices, hi =
 *                                 bf16(M_f) and lo = bf16(M_f - hi), with M_f =
 *                                 I - c^2 A_f for sana_scaled, element (r, c)
 *                                 at ((((r/32)*(d/16) + c/16)*64 + (c%16)/8*32
 *                                 + r%32)*8 + c%8 (the scan's operand order)
 *   bank_p   [B, H, n_ch+1, d, d] prefix states, slot m = P_{min(F, m*chunk)-1}
 *   bank_q   [B, H, n_ch+1, d, d] suffix states, slot m = Q_{min(F, m*chunk)}
 *   decay    [B, H, F, 2, d]      bridge decays prod_{lo..t} alpha, prod_{t..hi} alpha
 *   bank_e   int32 [2, B, H, n_ch+1, d] power-of-two exponent of every
 *                                 state row: row i of the state = row i of the
 *                                 bank * 2^e_i (prefix then suffix; e stays 0
 *                                 unless a row exceeds 2^64, i.e. a diverging
 *                                 sana_scaled scan)
 *   v_t      bf16 [B, H, d, N]    v transposed (bf16 only, else unused)
 *   st16     fp16 [B, H, F, d, d] (bf16 only) S_t = P_{lo-1} diag(a_t) +
 *                                 Q_{hi+1} diag(b_t) of every frame, times 2^-m
 *   st_eps   [B, H, F]            (bf16 only) rms_eps * 2^-2m, the same m
 * With HWA_FLAG_ROUTED the workspace also holds the routing's block means and
 * kept-block lists (hwa_get_route_layout): count int32 [B, H, n_ch, tiles]
 * and list uint16 [B, H, n_ch, tiles, stride], block indices relative to the
 * window's first 128-token block, in increasing order.
 * n_ch = ceil(F / chunk). The last 256 bytes before `total` hold the softmax
 * kernel's work-queue counters (internal; each call zeroes them itself).
 */
typedef struct {
  size_t lohi, stat_a, stat_b, map_m, bank_p, bank_q, decay, bank_e, v_t;
  size_t st16, st_eps;
  size_t total;
} hwa_workspace_layout;

/*
 * hybrid_attn_fwd -- out = windowed softmax + delta-rule linear branch.
 *
 *   q, k, v    [B, H, N, d]  dtype  raw (pre-RoPE) q/k and v, shared by both
 *                                   branches (article: one QKV projection)
 *   beta       [B, H, N]     fp32   per-token write strength, any sign (with
 *                                   beta < 0, I + c~^2 A_f must stay positive
 *                                   definite: the inverse takes its pivots in
 *                                   order, without exchanges)
 *   alpha      [B, H, F, d]  fp32   per-frame, per-key-channel forget gate
 *   gate       [B, H, N, d]  dtype  output-gate pre-activation (sigmoid)
 *   text_state [B, H, d, d]  fp32   S_text (d_v x d_k) or NULL (zero start)
 *   frames, tokens_per_frame        F >= 1, S >= 1, N = F * S <= 2^30; with
 *                                   bf16, roundup(N, 64) * d * 2 < 2^31 too
 *   chunk, radius                   chunk >= 1, radius >= 0
 *   rule                            hwa_rule
 *   out        [B, H, N, d]  dtype  written; must not alias any input
 *   stream                          hipStream_t
 *   p                               shapes, dtype, scalars, workspace, flags
 *
 * Returns HWA_OK, or an error status before anything is enqueued.
 */
hwa_status hybrid_attn_fwd(const void* q, const void* k, const void* v,
                           const float* beta, const float* alpha,
                           const void* gate, const float* text_state,
                           int32_t frames, int32_t tokens_per_frame,
                           int32_t chunk, int32_t radius, int32_t rule,
                           void* out, hipStream_t stream, const hwa_params* p);

/*
 * hybrid_attn_fwd_noalloc -- hybrid_attn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, semantics and kernels as
 * hybrid_attn_fwd, except that p->workspace and p->workspace_bytes are
 * ignored: the scratch is a device array inside the library, one per GPU, of
 * HWA_NOALLOC_SCRATCH_BYTES bytes, which each GPU the library runs on holds
 * until the process ends. The call never allocates or frees memory. Its
 * first call on a device looks up that device's copy of the array (the
 * current device, which must be the one `stream` belongs to).
 *   Returns HWA_ERR_WORKSPACE when hwa_workspace_bytes() for these sizes
 *   exceeds HWA_NOALLOC_SCRATCH_BYTES (nothing is enqueued), HWA_ERR_HIP if
 *   the array's address cannot be obtained, otherwise what hybrid_attn_fwd
 *   returns. The array keeps the last call's contents (every value a call
 *   reads from it is written by that call first). Calls on one GPU share the
 *   array: calls that overlap in time on one GPU (different streams, or
 *   threads) race and must be serialised by the caller.
 */
#define HWA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

hwa_status hybrid_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* beta, const float* alpha,
                                   const void* gate, const float* text_state,
                                   int32_t frames, int32_t tokens_per_frame,
                                   int32_t chunk, int32_t radius, int32_t rule,
                                   void* out, hipStream_t stream, const hwa_params* p);

/*
 * softmax_lse and softmax_out (when not NULL) are written by calls that run
 * the softmax branch; they must not overlap each other, out, an input or the
 * workspace. With HWA_FLAG_LINEAR_ONLY they must be NULL.
 */

/* Workspace bytes hybrid_attn_fwd needs for these sizes (0 on bad args). */
size_t hwa_workspace_bytes(int32_t frames, int32_t tokens_per_frame,
                           int32_t chunk, const hwa_params* p);

/* Offsets of the intermediates inside that workspace. */
hwa_status hwa_get_workspace_layout(int32_t frames, int32_t tokens_per_frame,
                                    int32_t chunk, const hwa_params* p,
                                    hwa_workspace_layout* layout);

/*
 * hwa_window_bounds -- the window table on the host (article, "What the far
 * field outside the window is"): frame t in chunk c = t / chunk sees key
 * frames lo[t] = max(0, (c - radius) * chunk) .. hi[t] = min(F - 1,
 * (c + radius + 1) * chunk - 1). lo and hi are host arrays of `frames`
 * int32, written by the call.
 */
hwa_status hwa_window_bounds(int32_t frames, int32_t chunk, int32_t radius,
                             int32_t* lo, int32_t* hi);

/*
 * hwa_text_state -- S_text of every (batch, head) from T text tokens.
 *
 * The article ("Text state") starts both scans from half a text state but
 * does not say how the prompt becomes that state. This entry point builds it
 * as one vdn_solve update from zero over one "frame" of text tokens, with the
 * branch's feature map on k and no conv:
 *   k^ = L2(SiLU(k_txt)),  A = sum beta k^ k^^T,  B = sum beta v k^^T,
 *   S_text = B (I + A)^-1.
 *   k_txt, v_txt [B, H, T, d] dtype;  beta_txt [B, H, T] fp32;
 *   state_out    [B, H, d, d] fp32 (written).
 * Uses p->batch, heads, head_dim, dtype, workspace (>= hwa_text_state_
 * workspace_bytes) and ignores the other fields.
 */
hwa_status hwa_text_state(const void* k_txt, const void* v_txt,
                          const float* beta_txt, int32_t text_tokens,
                          float* state_out, hipStream_t stream,
                          const hwa_params* p);

size_t hwa_text_state_workspace_bytes(int32_t text_tokens,
                                      const hwa_params* p);

/*
 * hwa_softmax_bwd -- gradient of the windowed softmax branch o_sm (article,
 * "What the far field outside the window is"; needed to train the hybrid
 * attention as its "Training" section does). For a loss L with upstream
 * gradient g = dL/do_sm, s_nm = q_n . k_m / sqrt(d), p_nm = exp(s_nm - lse_n)
 * over query n's window and delta_n = g_n . o_n:
 *   dv_m = sum_n p_nm g_n
 *   ds_nm = p_nm (g_n . v_m - delta_n)
 *   dq_n = sum_m ds_nm k_m / sqrt(d),   dk_m = sum_n ds_nm q_n / sqrt(d)
 * (sums over the query-key pairs of the window: query frame t, key frames
 * lo_t .. hi_t). For out = o_sm + y, g is dL/dout itself.
 *
 *   q, k, v    [B, H, N, d] dtype  the softmax branch's inputs (q_rope/k_rope
 *                                  if the forward used them)
 *   o_sm       [B, H, N, d] dtype  its output: softmax_out of the forward, or
 *                                  out of a HWA_FLAG_SOFTMAX_ONLY call
 *   lse        [B, H, N]    fp32   softmax_lse of the same forward call
 *   d_o        [B, H, N, d] dtype  g
 *   frames .. radius               as for hybrid_attn_fwd
 *   dq, dk, dv [B, H, N, d] dtype  written (bf16: rounded from fp32
 *                                  accumulation); must not overlap each other,
 *                                  an input or the workspace
 *   p          batch, heads, head_dim, dtype, workspace (>= hwa_softmax_bwd_
 *              workspace_bytes), stage_events (NULL, or
 *              HWA_NUM_BWD_STAGE_EVENTS events recorded at [0] start, [1]
 *              after the window table, delta and lse scaling,
 *              [2] after the dq kernel, [3] after the dk/dv kernel); the
 *              other fields are ignored
 * Returns HWA_OK, or an error status before anything is enqueued.
 */
#define HWA_NUM_BWD_STAGE_EVENTS 4

hwa_status hwa_softmax_bwd(const void* q, const void* k, const void* v,
                           const void* o_sm, const float* lse, const void* d_o,
                           int32_t frames, int32_t tokens_per_frame,
                           int32_t chunk, int32_t radius, void* dq, void* dk,
                           void* dv, hipStream_t stream, const hwa_params* p);

/* Workspace bytes hwa_softmax_bwd needs (0 on bad args): the window table
 * and delta and lse * log2(e) per query (2 * B * H * roundup(N, 64) * 4
 * bytes, plus alignment). */
size_t hwa_softmax_bwd_workspace_bytes(int32_t frames, int32_t tokens_per_frame,
                                       int32_t chunk, const hwa_params* p);

/*
 * hwa_linear_bwd -- gradient of the linear branch y (article, "Step 1:
 * NoPE features" .. "Step 5", "Text state"; needed to train the hybrid
 * attention as its "Training" section does) for a loss L with upstream
 * gradient d_o = dL/dy. With the forward's definitions (features q^, k^, v^;
 * statistics A_f, B_f; the update rule's scans P, Q from s0 = text_scale *
 * text_state; S_t gathered with the bridge decays; y = RMSNorm(S_t q^) *
 * w * sigmoid(gate)), the call writes dL/d(every input):
 *
 *   q, k, v, gate, d_o [B, H, N, d] dtype  as for hybrid_attn_fwd (the raw q:
 *                                          the branch never reads q_rope)
 *   beta [B, H, N], alpha [B, H, F, d], text_state [B, H, d, d] or NULL
 *                                          fp32, as for hybrid_attn_fwd
 *   frames .. rule                         as for hybrid_attn_fwd (all
 *                                          three rules; see sana_scaled
 *                                          below)
 *   dq, dk, dv, dgate [B, H, N, d] dtype   written (bf16: rounded from fp32)
 *   dbeta [B, H, N], dalpha [B, H, F, d]   fp32, written
 *   dtext_state [B, H, d, d] fp32 or NULL  dL/dtext_state (with a NULL
 *                                          text_state: at the zero state)
 *   dconv_k, dconv_v [H, d, 4] fp32        summed over the batch
 *   drms_weight [d] fp32 or NULL           summed over batch and heads
 *   p   batch, heads, head_dim, dtype, c, text_scale, rms_eps, conv_k, conv_v,
 *       rms_weight (NULL => ones), workspace (>= hwa_linear_bwd_workspace_
 *       bytes), stage_events (NULL, or HWA_NUM_LIN_BWD_STAGE_EVENTS events
 *       recorded at [0] start, [1] after recomputing the statistics, inverses
 *       and every frame's scan states, [2] after the readout, [3] after the
 *       gather, adjoint scans and per-frame gradients, [4] after the
 *       statistics and features, [5] after the convs and parameter sums)
 * p->flags: 0, or HWA_FLAG_ACCUMULATE to add dq, dk, dv to the contents of
 * those buffers (one fp32 sum, then the rounding to dtype) -- with
 * hwa_softmax_bwd's output there, the sum is the gradient of out = o_sm + y
 * with respect to q, k and v (when the forward used no q_rope / k_rope).
 * Outputs must not overlap each other, an input or the workspace. All
 * arithmetic is fp32, except that bf16 calls recompute the scan states with
 * the forward's split-bf16 MFMA scan (about 16 significant bits per product).
 * sana_scaled: the backward carries no power-of-two exponents; it is exact
 * (to fp32 rounding) while every recomputed state P_f, Q_f, every adjoint and
 * every gathered state's gradient stays inside fp32's normal range (about
 * 2^-126 .. 2^127). The states grow by up to ||I - c^2 A_f|| per frame (about
 * 28 for the 1,560-token frames of the clip workloads, so about 20 frames
 * there); past that the outputs are not finite.
 * Returns HWA_OK, or an error status before anything is enqueued.
 */
#define HWA_NUM_LIN_BWD_STAGE_EVENTS 6

hwa_status hwa_linear_bwd(const void* q, const void* k, const void* v, const float* beta,
                          const float* alpha, const void* gate, const float* text_state,
                          const void* d_o, int32_t frames, int32_t tokens_per_frame,
                          int32_t chunk, int32_t radius, int32_t rule, void* dq, void* dk,
                          void* dv, float* dbeta, float* dalpha, void* dgate,
                          float* dtext_state, float* dconv_k, float* dconv_v,
                          float* drms_weight, hipStream_t stream, const hwa_params* p);

/* Workspace bytes hwa_linear_bwd needs (0 on bad args): per (b, h) seven
 * fp32 d x d matrices per frame (statistics, inverses, both scans' states,
 * their adjoints), the bank gradients, and two fp32 [N, d] arrays (the
 * feature gradients before the convs), plus alignment. */
size_t hwa_linear_bwd_workspace_bytes(int32_t frames, int32_t tokens_per_frame,
                                      int32_t chunk, const hwa_params* p);

/*
 * hwa_frame_alpha -- the per-frame, per-key-channel forget gate alpha that
 * hybrid_attn_fwd takes (article, "Step 3": D = diag(alpha), a gate in (0, 1)
 * produced by the model's FrameKDAAlpha layer). The article gives no formula
 * or weights for that layer; this entry point computes the stated form
 *   m_f = mean_{n in frame f} k_n,  z_f = m_f W_h + b_h,
 *   alpha_f = exp(-exp(a_h) * softplus(z_f)),  softplus(z) = log(1 + e^z)
 * per (batch, head h, frame f), in fp32:
 *   k      [B, H, N, d]  dtype  the raw k of the linear branch (16-byte aligned)
 *   w      [H, d, d]     fp32   W_h[i][j]: input channel i, output channel j
 *   bias   [H, d]        fp32
 *   a_log  [H, d]        fp32   log decay rate a_h
 *   frames, tokens_per_frame    F >= 1, S >= 1
 *   alpha  [B, H, F, d]  fp32   written; must not overlap an input
 * Uses p->batch, heads, head_dim, dtype and ignores the other fields (no
 * workspace). Returns HWA_OK, or an error status before anything is enqueued.
 */
hwa_status hwa_frame_alpha(const void* k, const float* w, const float* bias,
                           const float* a_log, int32_t frames, int32_t tokens_per_frame,
                           float* alpha, hipStream_t stream, const hwa_params* p);

/*
 * hwa_block_fwd -- the attention block around the hybrid attention (article,
 * "Why video models are stuck on attention": one QKV projection feeds both
 * branches and their outputs are summed; "Step 1": the softmax branch uses
 * RoPE'd q and k, the linear branch unrotated ones). The article defines
 * neither the projections' layout nor the RoPE; this entry point computes,
 * per batch element, with D = H * d:
 *   [q | k | v] = x W_qkv^T            (q, k, v rounded to bf16)
 *   q_rope, k_rope = RoPE3D(q), RoPE3D(k)
 *   out_h = hybrid_attn_fwd(q, k, v, ..., q_rope, k_rope) of every head h
 *   y = [out_0 | ... | out_{H-1}] W_o^T
 * RoPE3D: token n of frame t = n / S sits at row r = (n % S) / grid_w and
 * column (n % S) % grid_w of the latent grid; its d / 2 channel pairs
 * (2i, 2i + 1) are split into p_t = d/2 - 2 floor(d/6) time pairs, then
 * p_h = floor(d/6) row pairs, then p_w = floor(d/6) column pairs, and pair u
 * of an axis with P pairs is turned by the angle pos * rope_theta^(-u / P)
 * (pos = t, r or the column): (a, b) -> (a cos - b sin, a sin + b cos).
 *   x      [B, N, D]   bf16   block input (tokens frame-major, N = F * S)
 *   w_qkv  [3 D, D]    bf16   rows = output features: q (head h at rows
 *                             h d .. h d + d - 1), then k, then v
 *   w_o    [D, D]      bf16   rows = output features
 *   beta, alpha, gate, text_state, chunk, radius, rule: as hybrid_attn_fwd
 *                             (per head, [B, H, ...])
 *   grid_w                    latent grid columns, >= 1, dividing S
 *   rope_theta                RoPE base (> 0; 10000 is the usual one)
 *   y      [B, N, D]   bf16   written; must not overlap an input or the
 *                             workspace
 * bf16 only (HWA_ERR_UNSUPPORTED for fp32), d = 64 or 128, and B * N * D * 2 <
 * 2^31. p: batch, heads, head_dim, dtype, c, text_scale, rms_eps, conv_k,
 * conv_v, rms_weight as for hybrid_attn_fwd; workspace >=
 * hwa_block_workspace_bytes (q, k, v, their rotations and the attention
 * output, then the attention's own workspace); stage_events (NULL or
 * HWA_NUM_BLOCK_STAGE_EVENTS events: [0] start, [1] after the QKV
 * projection, [2] after the hybrid attention, [3] after the output
 * projection); flags, q_rope, k_rope, softmax_lse and softmax_out must be 0 /
 * NULL. Returns HWA_OK, or an error status before anything is enqueued.
 */
#define HWA_NUM_BLOCK_STAGE_EVENTS 4

hwa_status hwa_block_fwd(const void* x, const void* w_qkv, const void* w_o, const float* beta,
                         const float* alpha, const void* gate, const float* text_state,
                         int32_t frames, int32_t tokens_per_frame, int32_t grid_w,
                         float rope_theta, int32_t chunk, int32_t radius, int32_t rule, void* y,
                         hipStream_t stream, const hwa_params* p);

size_t hwa_block_workspace_bytes(int32_t frames, int32_t tokens_per_frame, int32_t chunk,
                                 const hwa_params* p);

/* Static English text of a status. */
const char* hwa_status_string(hwa_status s);

#ifdef __cplusplus
}
#endif

#endif /* HWA_H */
