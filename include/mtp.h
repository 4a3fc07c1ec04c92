/*
 * mtp.h -- C ABI of the MI355X (gfx950) library for the teacher-forced
 * sequential multi-token-prediction (MTP) depth chain, its shared-head masked
 * cross-entropy (forward and backward, with top-1 accuracy by depth), draft
 * verification, and one recurrent draft step of a retained module.
 *
 * Sources (web pages; cited by title and section):
 *   [M7.6] "M7.6 - DeepSeek MTP: Sequential Modules, Teacher Forcing, and
 *          Speculative Runtime"
 *   [SPEC] the speculative-decoding explainer page (ailearn,
 *          "speculative-decoding"): gamma-token accept/correct/bonus rule
 *   [M7.4] "M7.4 - Multi-Token Prediction Foundations"
 *
 * General conventions
 *   - Every tensor pointer is a DEVICE pointer unless marked [host].  Tensors
 *     are dense row-major.  "rows" means the B*T positions of the dense
 *     [B, T] layout, row index b*T + i.
 *   - Matrices follow the y = x W^T convention: a weight W of shape [out, in]
 *     is stored row-major with `in` contiguous.
 *   - Every device pointer (NULL aside) must be 16-byte aligned: the kernels
 *     access tensors in 16-byte vectors.  A misaligned pointer is rejected
 *     with MTP_ERR_ARG.
 *   - The caller allocates and frees every buffer, including the workspace
 *     (size from the matching *_workspace_size call).  The library keeps no
 *     device memory of its own, apart from the static scratch of
 *     mtp_verify_noalloc (MTP_NOALLOC_SCRATCH_BYTES per device it runs on).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  No call synchronises the host.  Calls on different streams
 *     with disjoint buffers may run concurrently.
 *   - Errors: argument checks (null pointers, shapes, dtypes, depth,
 *     workspace size) run on the host before any launch; on failure the call
 *     returns a negative mtp_status and launches nothing, so outputs are left
 *     untouched.  Data-dependent errors are reported on the device (see each
 *     call) so that no host sync is needed.  MTP_ERR_HIP means a launch
 *     failed; outputs are then undefined.
 *   - dtype MTP_BF16: activations, embeddings and weight matrices are
 *     bfloat16 (bit pattern in uint16); MTP_F32: float32.  RMSNorm gains are
 *     always float32.  Matrix products run on MFMA with float32
 *     accumulation; RMS statistics, softmax and loss sums are float32 or
 *     wider.
 */
#ifndef MTP_H_
#define MTP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTP_OK = 0,
  MTP_ERR_NULL = -1,         /* a required pointer is NULL                       */
  MTP_ERR_SHAPE = -2,        /* a size is <= 0, inconsistent or not supported    */
  MTP_ERR_DEPTH = -3,        /* D < 1 ([M7.6] 0x04C: depth must be positive)     */
  MTP_ERR_DTYPE = -4,        /* unknown dtype                                    */
  MTP_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than required          */
  MTP_ERR_ARG = -6,          /* other invalid argument (reduce mode, denom, ...)  */
  MTP_ERR_HIP = -7,          /* a HIP launch failed                              */
  MTP_ERR_UNSUPPORTED = -8,  /* valid request outside what the kernels handle    */
  MTP_ERR_TOO_LARGE = -9     /* *_noalloc: needs more than the static scratch    */
} mtp_status;

typedef enum { MTP_F32 = 0, MTP_BF16 = 1 } mtp_dtype;

/* Per-depth loss reduction ([M7.6] 0x05).  FIXED divides depth k's summed
 * token loss by a declared constant (the paper's fixed 1/T; default B*T);
 * VALID_MEAN divides by |V_k| (the loss-valid rows of depth k).  An empty
 * depth contributes a zero term that stays in the D-way mean. */
typedef enum { MTP_REDUCE_FIXED = 0, MTP_REDUCE_VALID_MEAN = 1 } mtp_reduce;

/* Per-request verify status codes (mtp_verify_args.status). */
enum {
  MTP_VERIFY_OK = 0,
  MTP_VERIFY_BAD_UNIFORM = 1,      /* a uniform outside [0, 1) or NaN            */
  MTP_VERIFY_BAD_TOKEN = 2,        /* a draft token outside [0, V)               */
  MTP_VERIFY_ZERO_DRAFT_PROB = 3,  /* a tested draft token has q = 0             */
  MTP_VERIFY_ZERO_RESIDUAL = 4,    /* rejection with zero residual mass          */
  MTP_VERIFY_NONFINITE = 5,        /* a used logit row has NaN/+inf or is all -inf */
  MTP_VERIFY_BAD_POSITION = 6      /* mtp_propose_step: a position outside [0, L_max) */
};

/* ------------------------------------------------------------------------
 * MTP module weights of one depth k ([M7.6] 0x03, 0x03C, 0x04B).
 *   g_h, g_e  [d] f32   gains of RMSNorm_{h,k} (hnorm) and RMSNorm_{e,k} (enorm)
 *   M         [d, 2d]   eh_proj; columns [0,d) multiply the normalised hidden
 *                       state and [d,2d) the normalised embedding ("he" order,
 *                       [M7.6] 0x07B).  No bias.
 *   g_attn    [d] f32   gain of the block's attention pre-norm (Norm_a)
 *   Wqkv      [3*H*hd, d]  rows [0,H*hd) = W_q, then W_k, then W_v
 *   Wo        [d, H*hd]
 *   g_ffn     [d] f32   gain of the block's FFN pre-norm (Norm_f)
 *   Wgate, Wup [ffn, d]; Wdown [d, ffn]   SwiGLU: (silu(y Wg^T) * y Wu^T) Wd^T
 * The block is pre-norm ([M7.6] 0x03C): a = u + Attn(Norm_a(u)),
 * h = a + FFN(Norm_f(a)); attention is multi-head (H heads of width hd, no
 * biases, scale 1/sqrt(hd)), segment-causal, with rotate-half RoPE at the
 * position inside the segment run.
 * ---------------------------------------------------------------------- */
typedef struct {
  const float *g_h, *g_e, *g_attn, *g_ffn;
  const void *M;
  const void *Wqkv;
  const void *Wo;
  const void *Wgate, *Wup;
  const void *Wdown;
} mtp_depth_weights;

/* ------------------------------------------------------------------------
 * mtp_chain_forward: rows, masks and labels of every depth, then the
 * teacher-forced depth chain h^(1..D) ([M7.6] 0x02, 0x03, 0x04, 0x04C, 0x06A).
 *
 * Depth k at row (b, i) reads h^(k-1)[b,i] and the ground-truth token
 * x[b, i+k] and produces h^(k)[b,i]; its label is x[b, i+k+1].
 * A run is a maximal stretch of one non-negative segment id inside a batch
 * row (segment < 0 = padding).  For i in run [r0, r1]:
 *   state_mask[k,b,i] = (i + k     <= r1)   the chain i..i+k is inside the run
 *   loss_mask [k,b,i] = (i + k + 1 <= r1)   the label exists in the run
 *   labels    [k,b,i] = loss ? x[b,i+k+1] : -1;  counts[k] = sum of loss_mask
 * (padding rows: both masks 0).  h^(k) is defined on state rows; other rows
 * hold unspecified finite values.  Attention of row i sees rows j of its own
 * run with j <= i (a padding row sees only itself).
 *
 * Inputs : tokens, segment_ids int32 [B,T]; h0 [B*T, d]; embed [V, d] (the
 *          main model's shared embedding); w [host] D entries.
 * Outputs: h_out [host] D device pointers, each [B*T, d] in dtype;
 *          state_mask, loss_mask uint8 [D,B,T]; labels int32 [D,B,T];
 *          counts int32 [D]; device_error int32 [1]: set to 1 if an active
 *          position (segment >= 0) holds a token outside [0, V) (such tokens
 *          are clamped when gathered), else written 0.
 * Requirements: B,T,d,n_heads,ffn,V >= 1, D >= 1;
 *   bf16: d, ffn, n_heads*head_dim multiples of 8; head_dim in {32, 64, 128};
 *   f32 : d, ffn, n_heads*head_dim multiples of 4; head_dim in {16, 32, 64}
 *   (other widths return MTP_ERR_UNSUPPORTED); B*T <= 2^30; one batch row's
 *   [q | k | v] activation, T * 3 * n_heads * head_dim elements, must span
 *   less than 2 GiB (else MTP_ERR_UNSUPPORTED).
 * Saved activations (optional, bf16 only): with saved != NULL the call also
 * keeps, per depth, the activations mtp_chain_backward would otherwise
 * recompute (the concat, the residual streams, the normed inputs, q|k|v
 * after RoPE, the attention output and its per-query log-sum-exps, and the
 * gate and up projections before SwiGLU, in f32) in
 * saved, which must hold mtp_chain_saved_bytes(a) bytes (else
 * MTP_ERR_WORKSPACE; MTP_F32 with saved returns MTP_ERR_UNSUPPORTED).  The
 * layout is internal to the library; the buffer is caller-owned and is
 * handed to mtp_chain_backward for the same shapes and inputs.  h_out and
 * every other output are the same with or without it.
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, T, d, n_heads, head_dim, ffn, V, D;
  mtp_dtype dtype;
  float eps;                /* RMSNorm epsilon ([M7.6] 0x03C)                    */
  float rope_theta;         /* RoPE base; 0 disables RoPE                        */
  const int32_t *tokens, *segment_ids;
  const void *h0, *embed;
  const mtp_depth_weights *w;        /* [host] D entries                       */
  void *const *h_out;                /* [host] D device pointers               */
  uint8_t *state_mask, *loss_mask;
  int32_t *labels;
  int32_t *counts;
  int32_t *device_error;
  void *workspace;
  size_t workspace_bytes;
  void *saved;                       /* optional: per-depth activations kept  */
  size_t saved_bytes;                /* for mtp_chain_backward                */
} mtp_chain_args;

/* ------------------------------------------------------------------------
 * mtp_chain_backward: the gradient of L_MTP through the whole depth chain
 * ([M7.6] 0x05A: the MTP loss reaches each module's enorm, hnorm, eh_proj
 * and Transformer block, the shared token embedding, and the main model
 * through h^(0), a deeper loss passing through every module before it;
 * 0x05B: a depth-j module's parameters receive its own loss and every deeper
 * one, sum_{k=j..D} (lambda/D) dL^(k)/dtheta_j, and the shared embedding sums
 * every depth's share).
 *
 * The call runs the modules in reverse, depth D down to 1.  Module k first
 * recomputes its forward from h^(k-1) (h0 for k = 1, else h[k-2]) exactly as
 * mtp_chain_forward does, then takes the gradient arriving at h^(k) -- dh[k-1]
 * (the gradient from outside the chain, normally mtp_head_ce_fwd_bwd's dh
 * for depth k) plus, for k < D, what module k+1 sent back through its hnorm
 * input -- back through the block (SwiGLU MLP and its norm, segment-causal
 * attention with RoPE and its norm, the residual adds), eh_proj and the two
 * input norms.  The gradient at h^(0) is dh0; the embedding rows that module
 * k read (x[b, i+k] on its state rows) receive their share in dE.
 *
 * Precision (bf16 only): the recomputed activations are stored in bf16 where
 * the forward stores them; every gradient handed to a matrix product is
 * rounded to bf16 once (the gradient entering a module, the SwiGLU product's
 * and gate/up gradients, da, dO, dq/dk/dv, du); residual sums, norm
 * statistics and all outputs are float32.
 *
 * Inputs : the arguments of mtp_chain_forward (tokens, segment_ids, h0,
 *          embed, w, shapes, eps, rope_theta); h [host] D device pointers,
 *          h^(1..D) [B*T, d] as mtp_chain_forward wrote them (h[D-1] is not
 *          read); dh [host] D device pointers, f32 [B*T, d] each.
 * Outputs: dh0 f32 [B*T, d] (written; 0 on rows no loss reaches, such as
 *          padding and run-final rows);
 *          dE f32 [V, d]: ADDED to (the main model's embedding gradient and
 *          the MTP path's share one buffer, [M7.6] 0x05B; zero it first for
 *          the MTP share alone);
 *          dw [host] D entries of per-depth gradients (f32, the shapes of
 *          mtp_depth_weights): written, or added to with accumulate = 1;
 *          device_error int32 [1] (may be NULL): 1 if an active position
 *          holds a token outside [0, V), else 0.
 * Saved activations (optional): saved != NULL must be the buffer that
 * mtp_chain_forward filled for the same shapes, tokens, segment ids, h0,
 * embedding and weights (saved_bytes >= mtp_chain_saved_bytes of those
 * shapes, else MTP_ERR_WORKSPACE); the recompute is then skipped (the
 * gate/up product too: the reverse of SwiGLU reads the kept projections)
 * and the results are bitwise the same as with saved = NULL.
 * Requirements: as mtp_chain_forward, and: dtype MTP_BF16 (MTP_F32 returns
 * MTP_ERR_UNSUPPORTED), head_dim 64 or 128, d <= 8192.
 * ---------------------------------------------------------------------- */
typedef struct {
  float *g_h, *g_e, *g_attn, *g_ffn;  /* [d]                                  */
  float *M;                            /* [d, 2d]                              */
  float *Wqkv;                         /* [3*H*hd, d]                          */
  float *Wo;                           /* [d, H*hd]                            */
  float *Wgate, *Wup;                  /* [ffn, d]                             */
  float *Wdown;                        /* [d, ffn]                             */
} mtp_depth_grads;

typedef struct {
  int B, T, d, n_heads, head_dim, ffn, V, D;
  mtp_dtype dtype;
  float eps, rope_theta;
  const int32_t *tokens, *segment_ids;
  const void *h0, *embed;
  const mtp_depth_weights *w;        /* [host] D entries                       */
  const void *const *h;              /* [host] D pointers (h^(1..D))           */
  const float *const *dh;            /* [host] D pointers (f32)                */
  float *dh0;
  float *dE;
  const mtp_depth_grads *dw;         /* [host] D entries                       */
  int accumulate;                    /* 1: add into dw                         */
  int32_t *device_error;             /* optional                               */
  void *workspace;
  size_t workspace_bytes;
  const void *saved;                 /* optional: mtp_chain_forward's saved   */
  size_t saved_bytes;                /* activations                           */
} mtp_chain_bwd_args;

/* ------------------------------------------------------------------------
 * mtp_horizon_heads: K independent horizon heads on one trunk state, each a
 * Transformer block of its own followed by the shared head, run in the
 * sequential per-head schedule ([M7.4] 0x02: head k predicts x[t+k] from
 * the trunk state at t; 0x05B: an independent transformer head per horizon
 * with a shared vocabulary projection; 0x06A: each head's forward and
 * backward finish before the next head's, and the trunk receives the sum of
 * the heads' gradients once).
 *
 * Head k (1..K): u^(k) = Block_k(h) -- the block of mtp_chain_forward's
 * module (pre-norm segment-causal multi-head attention with RoPE at the
 * position inside the run, then SwiGLU, residual adds), with h as its input
 * -- then the shared head (Norm_out with g_out, W_out) and the masked CE
 * against x[b, t+k], labelled where t + k stays inside t's run.  The
 * objective is (lambda / K) sum_k L^(k), L^(k) = (sum of head k's token
 * losses) / (B*T).  Per head, in order: the block forward, the head CE
 * forward and backward (its logits bounded by logit slabs as in
 * mtp_head_ce_fwd_bwd), the block backward; only one head's activations
 * and logits are live at a time.
 *
 * Inputs : tokens, segment_ids int32 [B,T]; h [B*T, d] (dtype); w [host] K
 *          block weights; W_out [V, d]; g_out [d] f32.
 * Outputs: loss f32 [K] (L^(k)), counts int32 [K] (labelled rows),
 *          loss_total f32 [1] ((lambda / K) sum_k L^(k));
 *          dh f32 [B*T, d]: the summed gradient at the trunk state (written);
 *          dW_out f32 [V, d], dg_out f32 [d] and dw [host] K block gradients
 *          (f32, shapes of mtp_block_weights): written, or added to with
 *          accumulate = 1;
 *          device_error int32 [1] (may be NULL): 1 if an active position
 *          holds a token outside [0, V).
 * Requirements: as mtp_chain_backward (bf16; head_dim 64 or 128; d <= 8192)
 * and V % 8 == 0, V < 2^21; K >= 1.
 * ---------------------------------------------------------------------- */
typedef struct {
  const float *g_attn, *g_ffn;         /* [d] f32                              */
  const void *Wqkv;                    /* [3*H*hd, d]                          */
  const void *Wo;                      /* [d, H*hd]                            */
  const void *Wgate, *Wup;             /* [ffn, d]                             */
  const void *Wdown;                   /* [d, ffn]                             */
} mtp_block_weights;

typedef struct {
  float *g_attn, *g_ffn, *Wqkv, *Wo, *Wgate, *Wup, *Wdown;   /* f32, shapes as above */
} mtp_block_grads;

typedef struct {
  int B, T, d, n_heads, head_dim, ffn, V, K;
  mtp_dtype dtype;
  float eps, rope_theta, lambda;
  const int32_t *tokens, *segment_ids;
  const void *h;
  const mtp_block_weights *w;        /* [host] K entries                       */
  const void *W_out;
  const float *g_out;
  float *loss;                       /* [K]                                    */
  int32_t *counts;                   /* [K]                                    */
  float *loss_total;                 /* [1]                                    */
  float *dh;                         /* [B*T, d]                               */
  float *dW_out, *dg_out;
  const mtp_block_grads *dw;         /* [host] K entries                       */
  int accumulate;
  int32_t *device_error;             /* optional                               */
  void *workspace;
  size_t workspace_bytes;
} mtp_horizon_args;

/* ------------------------------------------------------------------------
 * mtp_head_ce_fwd_bwd: shared output head Norm_out + W_U, masked CE against
 * the labels of every depth, and the gradients of
 *   L_MTP = (lambda / D) * sum_k L^(k),  L^(k) = loss_sum[k] / denom_k
 * ([M7.6] 0x03, 0x04B, 0x05, 0x05A, 0x05B).  Rows are processed in slabs
 * of R rows with R * V * w <= logit_slab_bytes, w the width of a kept logit
 * (4 bytes for f32, 2 for bf16; R rounded down to a multiple of 256 when it
 * is at least 256, and at least 1).  Under the default bound R is also at
 * most half of the B*T rows (rounded up to a multiple of 256 from 256 rows
 * on), so the logits of the whole batch are never held at once; an explicit
 * bound is taken as given.  Per slab the forward GEMM reduces each
 * vocabulary tile to an online (max, sum-exp) partial per row and keeps the
 * slab's logits (f32: as fp32; bf16: as fp16 offsets from the row's maximum
 * over its 256-wide vocabulary tile, which are <= 0); the partials give the
 * row's log-sum-exp and softmax - onehot is formed from the kept logits,
 * stored in dtype.  That gradient is
 * kept for a group of G rows, G * V * sizeof(dtype) <= logit_slab_bytes (a
 * whole number of slabs, at least one), and the dx_hat and
 * dW_out GEMMs run once per group.  The logit and gradient buffers are
 * bounded by the slab and the group, not by B*T (the per-row buffers, such
 * as x_hat [B*T, d], do grow with B*T).
 *
 * Inputs : h [host] D pointers [B*T, d] (dtype); labels int32 [D,B,T]
 *          (-1 = no loss, as written by mtp_chain_forward); W_out [V, d]
 *          (dtype); g_out [d] f32 (the shared final-norm gain).
 * Outputs: loss_sum f32 [D] (sum of token losses of depth k), counts int32
 *          [D] (labelled rows), loss f32 [D] (L^(k)), loss_mtp f32 [1];
 *          lse f32 [D, B*T] (optional, may be NULL: log-sum-exp of every
 *          row's logits; unlabelled rows included);
 *          dh [host] D pointers, each f32 [B*T, d] = dL_MTP/dh^(k) through the
 *          head (0 on unlabelled rows); written, or added to the existing
 *          values with dh_accumulate = 1 (D pointers to one buffer then sum
 *          the depths' gradients: the trunk gradient of independent
 *          horizons that all read one hidden state, [M7.4] 0x02, 0x06A);
 *          dW_out f32 [V, d] and dg_out f32 [d]: the depths' contributions
 *          summed; accumulate = 1 adds them to the existing values (e.g. the
 *          main loss's), 0 overwrites;
 *          pred int32 [D, B*T], correct int32 [D], accuracy f32 [D]
 *          (each optional, may be NULL): top-1 accuracy by depth ([M7.6]
 *          0x0E; [M7.4] 0x0C).  pred is the argmax of each labelled row's
 *          logits (the lowest id among equal maxima; -1 on unlabelled rows),
 *          correct[k] counts the labelled rows with pred = label and
 *          accuracy[k] = correct[k] / counts[k] (0 for an empty depth).  The
 *          decision is taken on the fp32 logits (bf16 runs: on the kept fp16
 *          offsets, so values within 2^-25 of the row maximum tie with it).
 * reduce: MTP_REDUCE_FIXED with denom > 0 (0 selects B*T), or
 *          MTP_REDUCE_VALID_MEAN (denom ignored).
 * logit_slab_bytes: bound on the kept logits of a slab and on the gradient
 *          group (0 selects 1 GiB with at most half of the rows per slab:
 *          2048-row slabs and one 4096-row group at B*T = 4096,
 *          V = 129280 in bf16).
 * Requirements: bf16: d % 8 == 0, V % 8 == 0; f32: d % 4 == 0, V % 4 == 0;
 * V < 2^21.  Labels outside [-1, V) are treated as -1 and set device_error
 * (may be NULL).
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, T, d, V, D;
  mtp_dtype dtype;
  float eps, lambda;
  mtp_reduce reduce;
  double denom;
  const void *const *h;              /* [host] D pointers                      */
  const int32_t *labels;
  const void *W_out;
  const float *g_out;
  float *loss_sum;
  int32_t *counts;
  float *loss, *loss_mtp;
  float *lse;                        /* optional                               */
  void *const *dh;                   /* [host] D pointers (f32)                */
  float *dW_out, *dg_out;
  int accumulate;
  int32_t *device_error;             /* optional                               */
  size_t logit_slab_bytes;           /* 0 = 1 GiB                              */
  int dh_accumulate;                 /* 1: add into dh[k]                      */
  int32_t *pred;                     /* optional                               */
  int32_t *correct;                  /* optional                               */
  float *accuracy;                   /* optional                               */
  void *workspace;
  size_t workspace_bytes;
} mtp_ce_args;

/* ------------------------------------------------------------------------
 * mtp_verify: one exact speculative round per request ([M7.6] 0x09 for one
 * proposal; [SPEC] for gamma proposals).
 *   p_j = softmax(target_logits[r,j,:] / temperature), j = 0..gamma
 *   q_j = softmax(draft_logits [r,j,:] / temperature), j = 0..gamma-1
 * Left to right, draft j is accepted iff u_accept[r,j] < p_j(y_j) / q_j(y_j)
 * (strict; u in [0,1) makes min(1, .) redundant).  A = index of the first
 * rejection, or gamma if none.  If A < gamma the emitted token is drawn from
 * the normalised residual (p_A - q_A)+ ; otherwise from p_gamma (the bonus).
 * A draw uses u_sample[r, A] by inverse CDF over ascending token ids: the
 * smallest t with sum_{s<=t} w_s > u * sum_s w_s.  The round emits
 * N_emit = A + 1 tokens: the accepted drafts and next_token.  EOS and output
 * budget truncation are the caller's.
 *
 * Inputs : target_logits [R, gamma+1, V], draft_logits [R, gamma, V] in
 *          logits_dtype; draft_tokens int32 [R, gamma] (each sampled from its
 *          q); u_accept f32 [R, gamma]; u_sample f32 [R, gamma+1].
 * Outputs: accepted_len int32 [R] (A), next_token int32 [R], status int32 [R]
 *          (MTP_VERIFY_*; on a nonzero status A = 0 and next_token = -1);
 *          margin f32 [R] optional (may be NULL): the smallest distance of a
 *          decision from its threshold (|u - p/q| over the tests made, and the
 *          sample's distance to the nearer CDF step relative to the mass).
 * Checks in order: uniforms, token ids, then per used row: non-finite row,
 * q_j(y_j) = 0, zero residual mass.  Every logit row is read once (its
 * log-sum-exp); rows after the first rejection do not affect any output
 * (a non-finite value there is not reported).
 * Requirements: R >= 1, gamma >= 1, V >= 1, temperature > 0 and finite;
 * R <= 65535 (else MTP_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------- */
typedef struct {
  int R, gamma, V;
  float temperature;
  mtp_dtype logits_dtype;
  const void *target_logits;
  const void *draft_logits;
  const int32_t *draft_tokens;
  const float *u_accept;
  const float *u_sample;
  int32_t *accepted_len;
  int32_t *next_token;
  int32_t *status;
  float *margin;                     /* optional                               */
  void *workspace;
  size_t workspace_bytes;
} mtp_verify_args;

/* ------------------------------------------------------------------------
 * mtp_propose_step: one recurrent draft step of a retained MTP module for R
 * requests ([M7.6] 0x09: the proposal after the incoming token f is seeded by
 * the saved parent hidden state and E(f), and y is drawn from the module's
 * normalised distribution q that verification then uses; 0x09A: a module
 * served autoregressively keeps its own K/V cache; 0x09D: one module rolled
 * out for several draft steps feeds back its own output state and the
 * drafted token).  Per request r, with p = positions[r]:
 *   the module of mtp_chain_forward on the one row (h_prev[r], E[tokens[r]])
 *   at RoPE position p, its attention reading the cached keys and values of
 *   slots 0..p-1 and the row's own, which it writes to slot p;
 *   h_out[r]  = the module output (stored in dtype);
 *   logits[r] = W_out RMSNorm_{g_out}(h_out[r]), stored in dtype;
 *   draft_token[r] = the draw from q = softmax(logits[r] / temperature)
 *   over the stored logits (the values mtp_verify reads) by inverse CDF with
 *   u_sample[r]: the smallest t with cdf(t) > u * mass, float64 sums.
 * A gamma-token rollout calls again with h_prev = h_out, tokens =
 * draft_token and positions + 1, and hands the stored logits to mtp_verify as
 * draft_logits.  Slots of drafts that verification rejects are the caller's
 * to discard (a later step at the same position overwrites them).
 *
 * Inputs : h_prev [R, d] and the module's weights (one mtp_depth_weights),
 *          embed [V, d], W_out [V, d] (dtype), g_out [d] f32;
 *          tokens int32 [R]; positions int32 [R]; u_sample f32 [R].
 * In/out : kv_cache [R, 2, L_max, n_heads * head_dim] (dtype): K (after RoPE)
 *          and V of every slot; slots < p are read, slot p is written.
 * Outputs: h_out [R, d], logits [R, V] (dtype), draft_token int32 [R],
 *          status int32 [R] (MTP_VERIFY_BAD_POSITION, _BAD_TOKEN for tokens
 *          outside [0, V), _BAD_UNIFORM, _NONFINITE for a non-finite logit
 *          row; on a nonzero status draft_token = -1 and that request's other
 *          outputs are unspecified; a request rejected before the step
 *          (bad position or token) leaves its kv_cache untouched), margin
 *          f32 [R] optional:
 *          the draw's distance to the nearer CDF step relative to the mass.
 * Requirements: as mtp_chain_forward for d, n_heads, head_dim, ffn, V and
 * dtype; 1 <= R <= 65535; 1 <= L_max <= 2^20; temperature > 0 and finite.
 * ---------------------------------------------------------------------- */
typedef struct {
  int R, L_max, d, n_heads, head_dim, ffn, V;
  mtp_dtype dtype;
  float eps, rope_theta, temperature;
  const mtp_depth_weights *w;        /* [host] one entry                       */
  const void *embed, *W_out;
  const float *g_out;
  const void *h_prev;
  const int32_t *tokens, *positions;
  const float *u_sample;
  void *kv_cache;
  void *h_out, *logits;
  int32_t *draft_token, *status;
  float *margin;                     /* optional                               */
  void *workspace;
  size_t workspace_bytes;
} mtp_propose_args;

/* ------------------------------------------------------------------------
 * mtp_round_commit: the bookkeeping of one carried-frontier round per request
 * ([M7.6] 0x09: the selector's new tokens, target rows to keep, pending
 * frontier and stop flag, with its EOS and budget truncation; 0x09C: only
 * verified rows are committed; generalised to gamma drafts by [SPEC]).
 * Per request, from mtp_verify's outputs: the accepted drafts
 * y_0 .. y_(A-1) are emitted in order, then next_token (the correction, or
 * the bonus when A = gamma); emission stops once `remaining` tokens are out
 * or right after an emitted EOS, so an accepted EOS or a last-budget draft
 * gets no bonus.  rows_to_keep = A + 1 (the incoming frontier's target row
 * and the accepted drafts' rows); pending_frontier = next_token when it was
 * emitted (it has no target row yet), else -1; stopped = the budget is used
 * up or the last emitted token is EOS.  A request with a nonzero status,
 * remaining < 1 or A outside [0, gamma] emits nothing: n_new = 0,
 * rows_to_keep = 0, pending_frontier = -1, stopped = 1.
 * Inputs : draft_tokens int32 [R, gamma]; accepted_len, next_token, status
 *          int32 [R] (as written by mtp_verify); remaining int32 [R]; eos
 *          (a token id, or -1 for none).
 * Outputs: new_tokens int32 [R, gamma + 1] (the emitted tokens, then -1),
 *          n_new, rows_to_keep, pending_frontier, stopped int32 [R].
 * No workspace.  Requirements: R >= 1, gamma >= 1,
 * R * (gamma + 1) < 2^31.
 * ---------------------------------------------------------------------- */
typedef struct {
  int R, gamma, eos;
  const int32_t *draft_tokens, *accepted_len, *next_token, *status, *remaining;
  int32_t *new_tokens, *n_new, *rows_to_keep, *pending_frontier, *stopped;
} mtp_round_args;

int mtp_chain_forward(const mtp_chain_args *a, void *stream);
int mtp_chain_backward(const mtp_chain_bwd_args *a, void *stream);
int mtp_horizon_heads(const mtp_horizon_args *a, void *stream);
int mtp_head_ce_fwd_bwd(const mtp_ce_args *a, void *stream);
int mtp_verify(const mtp_verify_args *a, void *stream);

/* ------------------------------------------------------------------------
 * mtp_verify_noalloc: mtp_verify for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, checks, kernels and outputs as
 * mtp_verify, except that `workspace` and `workspace_bytes` are ignored: the
 * call uses a static scratch buffer of MTP_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends.  It calls
 * no allocating routine.  The caller still passes (and owns) the inputs and
 * outputs.  Requests needing more scratch than that (the bytes
 * mtp_verify_workspace_size reports; e.g. R <= 500 at V = 129280 and
 * gamma = 4, bf16 logits) return MTP_ERR_TOO_LARGE and launch nothing.
 * The stream must belong to the current device (else MTP_ERR_ARG).  All
 * calls on one device share its scratch, which keeps the last call's
 * contents: calls that overlap on one device (on different streams, or from
 * different threads without ordering) race and must not be issued.
 * ---------------------------------------------------------------------- */
#define MTP_NOALLOC_SCRATCH_BYTES (64u << 20)
int mtp_verify_noalloc(const mtp_verify_args *a, void *stream);

int mtp_propose_step(const mtp_propose_args *a, void *stream);
int mtp_round_commit(const mtp_round_args *a, void *stream);

/* Workspace bytes the call needs for these arguments (pointers are not
 * inspected); 0 if the arguments are invalid. */
size_t mtp_chain_workspace_size(const mtp_chain_args *a);
size_t mtp_chain_backward_workspace_size(const mtp_chain_bwd_args *a);
/* Bytes of the optional saved-activation buffer of mtp_chain_forward /
 * mtp_chain_backward for these shapes (about 2 d x 2 + d x 4 + d x 2 +
 * 3 A x 2 + A x 2 + 8 H + d x 4 + d x 2 + 2 ffn x 4 bytes per row and
 * depth, A = n_heads * head_dim); 0 if the arguments are invalid or not
 * bf16. */
size_t mtp_chain_saved_bytes(const mtp_chain_args *a);
size_t mtp_horizon_heads_workspace_size(const mtp_horizon_args *a);
size_t mtp_ce_workspace_size(const mtp_ce_args *a);
size_t mtp_verify_workspace_size(const mtp_verify_args *a);
size_t mtp_propose_workspace_size(const mtp_propose_args *a);

/* ------------------------------------------------------------------------
 * Optional instrumentation.  mtp_profile_stage arms the library to record
 * caller-created hipEvent_t pairs around every launch of one stage: launch
 * number j (counted from the arming call) records start_events[j % n] before
 * and stop_events[j % n] after the stage's kernel(s), on the call's stream.
 * The caller reads the elapsed times once the stream is synchronised.
 * stage < 0 disarms.  The setting is process-wide (not thread-safe); events
 * stay owned by the caller and must outlive the armed period.
 * mtp_profile_count returns the number of launches recorded since arming.
 * ---------------------------------------------------------------------- */
typedef enum {
  MTP_STAGE_ROWS = 0, MTP_STAGE_DUAL_NORM = 1, MTP_STAGE_EH_PROJ = 2, MTP_STAGE_NORM_A = 3,
  MTP_STAGE_QKV = 4, MTP_STAGE_ATTN = 5, MTP_STAGE_O_PROJ = 6, MTP_STAGE_NORM_F = 7,
  MTP_STAGE_GATE_UP = 8, MTP_STAGE_DOWN = 9, MTP_STAGE_OUT_NORM = 10, MTP_STAGE_CE_FWD = 11,
  MTP_STAGE_CE_REDUCE = 12, MTP_STAGE_CE_GRAD = 13, MTP_STAGE_CE_DX = 14,
  MTP_STAGE_CE_NORM_BWD = 15, MTP_STAGE_CE_DW = 16, MTP_STAGE_VERIFY = 17,
  MTP_STAGE_BWD_RECOMPUTE = 18,     /* mtp_chain_backward: the module's forward again          */
  MTP_STAGE_BWD_MLP = 19,           /* SwiGLU reverse, its products and Norm_f's reverse       */
  MTP_STAGE_BWD_ATTN_PROJ = 20,     /* dO and dW_o products                                    */
  MTP_STAGE_BWD_ATTN = 21,          /* the attention reverse                                   */
  MTP_STAGE_BWD_QKV = 22,           /* dx_a, dW_qkv products and Norm_a's reverse              */
  MTP_STAGE_BWD_EH = 23,            /* eh_proj products, hnorm / enorm reverse, dE             */
  MTP_STAGE_COUNT = 24
} mtp_stage;
int mtp_profile_stage(int stage, void *const *start_events, void *const *stop_events, int n);
/* As mtp_profile_stage for every stage at once: launch j of any stage
 * records start_events[j % n] / stop_events[j % n] and writes the stage's
 * id to stage_ids[j % n] ([host] array owned by the caller).
 * mtp_profile_stage(-1, ...) disarms. */
int mtp_profile_all(void *const *start_events, void *const *stop_events, int *stage_ids, int n);
int mtp_profile_count(void);

/* Static string naming a status code. */
const char *mtp_strerror(int status);

/* ABI version of this header, incremented on every incompatible change (a
 * struct field added, moved or retyped, a call's meaning changed).  A
 * binding that mirrors the argument structs must refuse a library whose
 * mtp_abi_version() differs from the MTP_ABI_VERSION it was written for. */
#define MTP_ABI_VERSION 9
int mtp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MTP_H_ */
